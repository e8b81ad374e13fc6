"""Pins of the oracle against facts that do not come from the oracle itself.

The pages (speakrs 0.6.0, `lstmproj.rs` and `lstm.rs`) fix the data flow and the tensor
contract but print no worked example, so the oracle is pinned by:

* the closed form of the first step of a one-unit case (zero state: f and R drop out),
* an independent library implementation of the same cell: torch.nn.LSTM in float64,
* the invariant |h| < 1,
* the R = 0 scan closed form c_t = sum_s (prod_{r=s+1..t} f_r) i_s g_s,
* per-step independence when R = 0 and the forget gate is switched off,
* time-reversal symmetry: reversing the input and swapping the directions' weights
  reverses the output and swaps its halves,
* numpy's matmul for the projection alone.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_stack(x: np.ndarray, layers) -> np.ndarray:
    """torch.nn.LSTM(bidirectional, batch_first) in float64 with the same weights."""
    hidden = layers[0]["r"].shape[2]
    features = layers[0]["w"].shape[2]
    net = torch.nn.LSTM(features, hidden, num_layers=len(layers), bidirectional=True,
                        batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        for k, layer in enumerate(layers):
            for d, suffix in enumerate(["", "_reverse"]):
                getattr(net, f"weight_ih_l{k}{suffix}").copy_(torch.from_numpy(layer["w"][d].astype(np.float64)))
                getattr(net, f"weight_hh_l{k}{suffix}").copy_(torch.from_numpy(layer["r"][d].astype(np.float64)))
                getattr(net, f"bias_ih_l{k}{suffix}").copy_(torch.from_numpy(layer["b"][d, 0].astype(np.float64)))
                getattr(net, f"bias_hh_l{k}{suffix}").copy_(torch.from_numpy(layer["b"][d, 1].astype(np.float64)))
        y, _ = net(torch.from_numpy(x.astype(np.float64)))
    return y.numpy()


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def one_unit_layers():
    with open(os.path.join(GOLDEN, "one_unit_case.json")) as f:
        case = json.load(f)
    w = np.array(case["W"], np.float32).reshape(4, 1)
    r = np.array(case["R"], np.float32).reshape(4, 1)
    b = np.stack([np.array(case["Wb"], np.float32), np.array(case["Rb"], np.float32)])
    layer = {"w": np.stack([w, w]), "r": np.stack([r, r]), "b": np.stack([b, b])}
    x = np.array(case["x"], np.float32).reshape(3, 1)
    return [layer], x


def test_one_unit_first_step_closed_form(oracle_lib):
    """Step 0 from zero state: h = σ(a_o)·tanh(σ(a_i)·tanh(a_g)), a = W x + Wb + Rb.

    With the fixture's numbers a = (0.16, 0.28, 0.40, 0.52) forward (x = 1) and
    (0.11, 0.18, 0.25, 0.32) for the reverse direction's first step (x = 0.5, t = 2).
    A swapped gate order, a dropped bias or a wrong reverse index changes these values.
    """
    layers, x = one_unit_layers()
    y = oracle_lib.stack_window(x, layers)
    f32 = lambda v: float(np.float32(v))
    a_fwd = [f32(0.1) * 1.0 + f32(0.01) + f32(0.05), None, f32(0.3) * 1.0 + f32(0.03) + f32(0.07),
             f32(0.4) * 1.0 + f32(0.04) + f32(0.08)]
    c0 = (1 / (1 + math.exp(-a_fwd[0]))) * math.tanh(a_fwd[2])
    h0 = (1 / (1 + math.exp(-a_fwd[3]))) * math.tanh(c0)
    assert abs(a_fwd[0] - 0.16) < 1e-7 and abs(a_fwd[2] - 0.40) < 1e-7
    assert y[0, 0] == pytest.approx(h0, abs=1e-15)
    assert h0 == pytest.approx(0.1268783, abs=1e-7)  # hand evaluation of the closed form
    xr = f32(0.5)
    a_rev = [f32(0.1) * xr + f32(0.01) + f32(0.05), f32(0.3) * xr + f32(0.03) + f32(0.07),
             f32(0.4) * xr + f32(0.04) + f32(0.08)]
    c2 = (1 / (1 + math.exp(-a_rev[0]))) * math.tanh(a_rev[1])
    h2 = (1 / (1 + math.exp(-a_rev[2]))) * math.tanh(c2)
    assert y[2, 1] == pytest.approx(h2, abs=1e-15)


def test_one_unit_all_steps_match_torch(oracle_lib):
    layers, x = one_unit_layers()
    y = oracle_lib.stack_window(x, layers)
    ref = torch_stack(x[None], layers)[0]
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-15)
    # the three forward steps differ from the reverse ones: the directions are not mixed up
    assert np.abs(y[:, 0] - y[:, 1]).max() > 1e-3


@pytest.mark.parametrize("hidden,features,nl,steps,batch", [
    (1, 1, 1, 5, 1), (3, 5, 2, 7, 2), (8, 6, 3, 9, 2), (128, 60, 4, 16, 2)])
def test_matches_torch_float64_small(oracle_lib, hidden, features, nl, steps, batch):
    layers = workloads.random_layers(7 + hidden, hidden, features, nl, scale=0.5)
    x = np.random.default_rng(3).standard_normal((batch, steps, features)).astype(np.float32)
    y = oracle_lib.stack(x, layers)
    ref = torch_stack(x, layers)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


def test_matches_torch_float64_full_window(oracle_lib):
    """One full 589-frame window of the production shape (H=128, 60 -> 256, 4 layers)."""
    x, layers = workloads.make_workload("b1")
    y = oracle_lib.stack(x, layers)
    ref = torch_stack(x, layers)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


@pytest.mark.slow
def test_matches_torch_float64_stress_window(oracle_lib):
    """One window of the long, saturating workload (σ = 2 input, R × 2), first 1024 steps."""
    wl = workloads.WORKLOADS["b64_t4096"]
    x, layers = workloads.make_workload(wl)
    xs = np.ascontiguousarray(x[5:6, :1024])
    y = oracle_lib.stack(xs, layers)
    ref = torch_stack(xs, layers)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("name", ["b1", "b256", "b64_t4096"])
def test_hidden_state_strictly_bounded(oracle_lib, name):
    """|h| = |o · tanh(c)| < 1 in exact arithmetic; the double oracle keeps it strict."""
    wl = workloads.WORKLOADS[name]
    x, layers = workloads.make_workload(wl)
    steps = min(wl.steps, 1024)
    windows = [0, 1] if wl.batch > 1 else [0]
    y = oracle_lib.stack(np.ascontiguousarray(x[:, :steps]), layers, windows=windows, threads=2)
    assert np.all(np.abs(y) < 1.0)
    assert np.all(np.isfinite(y))
    if wl.zero_every:
        # an all-zero window still produces a nonzero output (the biases drive it)
        assert np.abs(y[0]).max() > 1e-3


def _projection_np(x, layer):
    w = layer["w"].astype(np.float64)
    b = layer["b"].astype(np.float64)
    return np.einsum("mk,drk->mdr", x.astype(np.float64), w) + (b[:, 0] + b[:, 1])[None]


def test_projection_matches_numpy_matmul(oracle_lib):
    layers = workloads.random_layers(11, 128, 60, 1)
    x = np.random.default_rng(5).standard_normal((37, 60)).astype(np.float32)
    got = oracle_lib.projection(x, layers[0]["w"], layers[0]["b"])
    np.testing.assert_allclose(got, _projection_np(x, layers[0]), rtol=0, atol=1e-13)


def test_gate_dump_is_the_projection(oracle_lib):
    layers = workloads.random_layers(12, 16, 10, 2)
    x = np.random.default_rng(6).standard_normal((9, 10)).astype(np.float32)
    y, dump = oracle_lib.stack_window(x, layers, dump_gates=True)
    np.testing.assert_allclose(dump[0], _projection_np(x, layers[0]), rtol=0, atol=1e-13)
    # the recurrence alone, fed the first layer's gates, reproduces the first layer
    y1 = oracle_lib.stack_window(x, layers[:1])
    np.testing.assert_allclose(oracle_lib.recurrence(dump[0], layers[0]["r"]), y1, rtol=0, atol=0)


def _scan_closed_form(x, layer, hidden):
    """R = 0: gates depend on x_t only, and c_t = sum_{s<=t} (prod_{r=s+1..t} f_r) i_s g_s."""
    a = _projection_np(x, layer)  # [T, 2, 4H]
    steps = x.shape[0]
    y = np.zeros((steps, 2 * hidden))
    for d in range(2):
        i = sigmoid(a[:, d, 0:hidden])
        f = sigmoid(a[:, d, hidden:2 * hidden])
        g = np.tanh(a[:, d, 2 * hidden:3 * hidden])
        o = sigmoid(a[:, d, 3 * hidden:4 * hidden])
        order = list(range(steps)) if d == 0 else list(range(steps - 1, -1, -1))
        for pos, t in enumerate(order):
            c = np.zeros(hidden)
            for spos in range(pos + 1):
                s = order[spos]
                prod = np.ones(hidden)
                for rpos in range(spos + 1, pos + 1):
                    prod = prod * f[order[rpos]]
                c = c + prod * i[s] * g[s]
            y[t, d * hidden:(d + 1) * hidden] = o[t] * np.tanh(c)
    return y


def test_zero_recurrent_weights_scan_closed_form(oracle_lib):
    hidden = 6
    layers = workloads.random_layers(13, hidden, 5, 2, scale=0.8)
    for layer in layers:
        layer["r"][:] = 0.0
    x = np.random.default_rng(7).standard_normal((8, 5)).astype(np.float32)
    expected0 = _scan_closed_form(x, layers[0], hidden)
    got0 = oracle_lib.stack_window(x, layers[:1])
    np.testing.assert_allclose(got0, expected0, rtol=0, atol=1e-14)
    # second layer: its input is the first layer's output, which the closed form gives too
    # (rounded to float32 here, because the projection takes float32 input)
    expected1 = _scan_closed_form(expected0.astype(np.float32), layers[1], hidden)
    y1, dump = oracle_lib.stack_window(x, layers, dump_gates=True)
    got1 = oracle_lib.recurrence(_projection_np(expected0.astype(np.float32), layers[1]),
                                 layers[1]["r"])
    np.testing.assert_allclose(got1, expected1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(y1, expected1, rtol=0, atol=1e-6)


def _forget_off(layers, hidden):
    for layer in layers:
        layer["r"][:] = 0.0
        layer["w"][:, hidden:2 * hidden, :] = 0.0
        layer["b"][:, :, hidden:2 * hidden] = -60.0  # f = σ(-120) ≈ 8e-53


def test_forget_off_steps_are_independent(oracle_lib):
    """R = 0 and f ≈ 0: every layer is a per-step map, so permuting time permutes outputs."""
    hidden = 16
    layers = workloads.random_layers(14, hidden, 12, 4)
    _forget_off(layers, hidden)
    x = np.random.default_rng(8).standard_normal((20, 12)).astype(np.float32)
    perm = np.random.default_rng(9).permutation(20)
    y = oracle_lib.stack_window(x, layers)
    yp = oracle_lib.stack_window(np.ascontiguousarray(x[perm]), layers)
    np.testing.assert_allclose(yp, y[perm], rtol=0, atol=1e-15)
    # and the per-step closed form h = σ(a_o)·tanh(σ(a_i)·tanh(a_g)) holds for layer 0
    a = _projection_np(x, layers[0])
    h = sigmoid(a[:, :, 3 * hidden:]) * np.tanh(sigmoid(a[:, :, :hidden]) *
                                                 np.tanh(a[:, :, 2 * hidden:3 * hidden]))
    y0 = oracle_lib.stack_window(x, layers[:1])
    np.testing.assert_allclose(y0, h.reshape(20, 2 * hidden), rtol=0, atol=1e-15)


def _swap_directions(layers, hidden):
    out = []
    for k, layer in enumerate(layers):
        w = layer["w"][::-1].copy()
        if k > 0:  # the input arrives as [rev | fwd]: swap the column halves too
            w = np.concatenate([w[:, :, hidden:], w[:, :, :hidden]], axis=2)
        out.append({"w": np.ascontiguousarray(w), "r": np.ascontiguousarray(layer["r"][::-1]),
                    "b": np.ascontiguousarray(layer["b"][::-1])})
    return out


@pytest.mark.parametrize("hidden,features,nl,steps", [(5, 3, 1, 11), (12, 7, 3, 13), (128, 60, 4, 40)])
def test_time_reversal_symmetry(oracle_lib, hidden, features, nl, steps):
    layers = workloads.random_layers(15 + nl, hidden, features, nl)
    x = np.random.default_rng(10).standard_normal((steps, features)).astype(np.float32)
    y = oracle_lib.stack_window(x, layers)
    y_rev = oracle_lib.stack_window(np.ascontiguousarray(x[::-1]), _swap_directions(layers, hidden))
    expected = np.concatenate([y[::-1, hidden:], y[::-1, :hidden]], axis=1)
    tol = 0 if nl == 1 else 1e-12  # one layer: the same operations in the same order
    np.testing.assert_allclose(y_rev, expected, rtol=0, atol=tol)


def test_float_mode_tracks_double_mode(oracle_lib):
    """The fp32 build of the same body stays near the double one (it shows the fp32 noise floor)."""
    x, layers = workloads.make_workload("b1")
    xs = np.ascontiguousarray(x[:, :128])
    y64 = oracle_lib.stack(xs, layers, precision="f64")
    y32 = oracle_lib.stack(xs, layers, precision="f32")
    err = np.abs(y32 - y64).max()
    assert 0 < err < 1e-5


def test_batch_windows_are_independent(oracle_lib):
    x, layers = workloads.make_workload("b8")
    xs = np.ascontiguousarray(x[:, :24])
    ya = oracle_lib.stack(xs, layers, threads=4)
    yb = oracle_lib.stack(xs, layers, windows=[5, 2])
    np.testing.assert_array_equal(ya[[5, 2]], yb)


# ---- segmentation heads (the `segdense.rs` page: linear0, linear1, classifier) -------------

def _head_case():
    with open(os.path.join(GOLDEN, "heads_one_unit_case.json")) as f:
        case = json.load(f)
    head = {k: np.array(case[k], np.float32) for k in ("w0", "b0", "w1", "b1", "w2", "b2")}
    head["slope"] = case["slope"]
    return head, np.array(case["y"], np.float32).reshape(1, 1)


def test_heads_one_unit_closed_form(oracle_lib):
    """y = -2 falls on LeakyReLU's negative branch (h0 = 0.01 * -2 = -0.02), then
    h1 = 3 * -0.02 + 0.5 = 0.44 and z = (0.44, -0.44), whose log-softmax is
    z - log(e^0.44 + e^-0.44) = z - log(2 cosh 0.44)."""
    head, y = _head_case()
    out = oracle_lib.heads(y, head)
    lse = math.log(2.0 * math.cosh(0.44))
    np.testing.assert_allclose(out[0], [0.44 - lse, -0.44 - lse], rtol=0, atol=1e-7)


def torch_heads(y: np.ndarray, head: dict) -> np.ndarray:
    """torch.nn.functional linear / leaky_relu / log_softmax in float64 with the same weights."""
    import torch.nn.functional as F
    t = torch.from_numpy(y.astype(np.float64))
    for i in range(3):
        w = torch.from_numpy(head[f"w{i}"].astype(np.float64))  # [k, n]
        b = torch.from_numpy(head[f"b{i}"].astype(np.float64))
        t = F.linear(t, w.T.contiguous(), b)
        if i < 2:
            t = F.leaky_relu(t, negative_slope=head["slope"])
    return F.log_softmax(t, dim=-1).numpy()


@pytest.mark.parametrize("rows,sizes", [(5, (3, 4, 5, 2)), (64, (16, 8, 12, 7)), (600, workloads.HEAD_SIZES)])
def test_heads_match_torch_float64(oracle_lib, rows, sizes):
    head = workloads.make_heads(77 + rows, sizes=sizes)
    y = np.random.default_rng(rows).uniform(-1, 1, size=(rows, sizes[0])).astype(np.float32)
    np.testing.assert_allclose(oracle_lib.heads(y, head), torch_heads(y, head), rtol=0, atol=1e-12)


def test_heads_log_softmax_normalised_and_shift_invariant(oracle_lib):
    head = workloads.make_heads(5)
    # classifier bias on a 2^-12 grid, so adding 3 to it is exact in float32
    head["b2"] = (np.round(head["b2"] * 4096.0) / 4096.0).astype(np.float32)
    y = np.random.default_rng(6).uniform(-1, 1, size=(300, 256)).astype(np.float32)
    out = oracle_lib.heads(y, head)
    assert np.all(out <= 0.0)
    np.testing.assert_allclose(np.exp(out).sum(axis=1), 1.0, rtol=0, atol=1e-12)
    shifted = dict(head, b2=(head["b2"] + np.float32(3.0)).astype(np.float32))
    assert np.array_equal(shifted["b2"].astype(np.float64) - 3.0, head["b2"].astype(np.float64))
    np.testing.assert_allclose(oracle_lib.heads(y, shifted), out, rtol=0, atol=1e-12)
