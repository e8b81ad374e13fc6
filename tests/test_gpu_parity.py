"""GPU parity: the HIP library against the oracle, element by element, on seeded inputs.

Tolerance on the final [B, T, 256] output (allclose form): |gpu - oracle| <= 2e-5 + 1e-4·|oracle|.
The projection alone is held to the rigorous fp32 dot-product bound
|err| <= (K + 2)·u·(sum_k |w_k x_k| + |bias|), u = 2^-24, which holds for any summation order.
"""

import os
import sys

import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL = 2e-5
RTOL = 1e-4


def note(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def bl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bidirectional_lstm_sequence_amd as bl
    bl.library()  # fails loudly if the HIP library was not built
    return bl


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def assert_close(got, ref, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside tolerance; worst at "
                             f"{idx}: gpu {got[idx]!r} oracle {ref[idx]!r} (max abs err {err.max():.3e})")
    return float(err.max())


def to_packed(oracle_gates):
    """[rows, 2, 512] in source order (g*128 + j) -> [rows, 1024] packed (d*512 + 4j + g)."""
    rows = oracle_gates.shape[0]
    g = oracle_gates.reshape(rows, 2, 4, 128)          # d, gate, unit
    return np.ascontiguousarray(g.transpose(0, 1, 3, 2).reshape(rows, 1024))


def projection_bound(x, layer, split=False):
    """|gpu - exact| bound of a gate pre-activation. FP32: (K + 2)·u·(sum|w x| + |bias|), any
    summation order. Split precision (bf16 x 3): the dropped lo·lo term and the parts'
    residuals add 3·2^-16·(1 + 2^-7)·sum|w x|, the FP32 sum runs over 3K products."""
    w = layer["w"].astype(np.float64)
    b = layer["b"].astype(np.float64)
    k = x.shape[1]
    mag = np.einsum("mk,drk->mdr", np.abs(x.astype(np.float64)), np.abs(w)) + np.abs(b[:, 0] + b[:, 1])[None]
    if not split:
        return to_packed((k + 2) * 2.0 ** -24 * mag * 1.01 + 1e-30)
    coeff = 3 * 2.0 ** -16 * (1 + 2.0 ** -7) + (3 * k + 2) * 2.0 ** -24 * 1.01
    return to_packed(coeff * mag * 1.01 + 1e-30)


@pytest.mark.parametrize("layer_index,rows,projection", [(0, 200, 0), (0, 589, 0), (1, 333, 0), (1, 4712, 0),
                                                         (1, 18848, 0), (0, 589, 1), (1, 4712, 1),
                                                         (0, 589, 2), (1, 333, 2), (1, 18848, 2)])
def test_projection_matches_oracle(bl, orc, layer_index, rows, projection):
    """The projection alone (projection = 1: the vendor-GEMM comparator) against the oracle,
    within the summation-order-free fp32 bound."""
    layers = workloads.make_layers(31)
    width = 60 if layer_index == 0 else 256
    x = np.random.default_rng(rows).standard_normal((rows, width)).astype(np.float32)
    if layer_index > 0:
        x = np.tanh(x).astype(np.float32)  # later layers see hidden states in (-1, 1)
    note(f"projection layer={layer_index} rows={rows} projection={projection}")
    plan = bl.Plan(layers, rows, 1, projection=projection)
    gates = plan.project(layer_index, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    ref = to_packed(orc.projection(x, layers[layer_index]["w"], layers[layer_index]["b"]))
    err = np.abs(gates.cpu().numpy().astype(np.float64) - ref)
    bound = projection_bound(x, layers[layer_index], split=projection == 2)
    assert np.all(err <= bound), f"max err {err.max():.3e}, worst ratio {(err / bound).max():.2f}"
    note(f"projection layer={layer_index} rows={rows} projection={projection} max err {err.max():.3e} "
         f"worst ratio to bound {(err / bound).max():.3f}")
    plan.close()


SPLITS = [(1, 1), (1, 2), (1, 4), (2, 1), (2, 2), (2, 4), (4, 1), (4, 2), (4, 4)]


@pytest.mark.parametrize("groups,tile", SPLITS)
def test_recurrence_matches_oracle(bl, orc, groups, tile):
    """The recurrence alone, fed fp32 gate pre-activations, for every workgroup split."""
    batch, steps = 5, 48  # 5 windows: a ragged last tile for tile sizes 2 and 4
    layers = workloads.make_layers(32)
    rng = np.random.default_rng(7)
    gates_src = (rng.standard_normal((batch * steps, 2, 512)) * 1.5).astype(np.float32)
    note(f"recurrence groups={groups} tile={tile} batch={batch} steps={steps}")
    plan = bl.Plan(layers, batch, steps, groups=groups, tile=tile)
    info = plan.info()
    assert info["recur_groups"] == groups and info["recur_tile"] == tile
    g_dev = torch.from_numpy(to_packed(gates_src)).cuda()
    y = plan.recur(1, g_dev)
    plan.check()
    got = y.cpu().numpy()
    per_window = gates_src.reshape(batch, steps, 2, 512)
    for b in range(batch):
        ref = orc.recurrence(per_window[b].astype(np.float64), layers[1]["r"])
        assert_close(got[b], ref, f"window {b}")
    plan.close()


def test_recurrence_splits_are_bitwise_identical(bl):
    """Every workgroup split sums in the same canonical order, so outputs agree bit for bit."""
    batch, steps = 6, 40
    layers = workloads.make_layers(33)
    rng = np.random.default_rng(8)
    g = torch.from_numpy(to_packed((rng.standard_normal((batch * steps, 2, 512))).astype(np.float32))).cuda()
    outs = {}
    for groups, tile in SPLITS:
        note(f"bitwise split groups={groups} tile={tile}")
        plan = bl.Plan(layers, batch, steps, groups=groups, tile=tile)
        outs[(groups, tile)] = plan.recur(2, g).cpu().numpy()
        plan.check()
        plan.close()
    base = outs[(1, 1)]
    for key, val in outs.items():
        assert np.array_equal(val.view(np.uint32), base.view(np.uint32)), f"split {key} differs"


def run_stack(bl, x, layers, **kw):
    plan = bl.Plan(layers, x.shape[0], x.shape[1], **kw)
    xd = torch.from_numpy(x).cuda()
    y = plan.forward(xd)
    plan.check()
    out = y.cpu().numpy()
    info = plan.info()
    plan.close()
    return out, info


@pytest.mark.parametrize("name", ["b1", "b8", "b32"])
def test_stack_matches_oracle_whole_batch(bl, orc, name):
    x, layers = workloads.make_workload(name)
    note(f"stack {name} shape={x.shape}")
    got, info = run_stack(bl, x, layers)
    ref = orc.stack(x, layers, threads=min(16, os.cpu_count() or 1))
    err = assert_close(got, ref, name)
    assert np.all(np.abs(got) <= 1.0)
    note(f"stack {name} max abs err {err:.3e} plan {info}")


@pytest.mark.parametrize("name,windows", [("b256", [0, 1, 10, 127, 200, 255]), ("b64_t4096", [0, 37])])
def test_stack_matches_oracle_sampled_windows(bl, orc, name, windows):
    """Full-size workloads in the default launch configuration; the oracle checks sampled windows."""
    x, layers = workloads.make_workload(name)
    note(f"stack {name} shape={x.shape} sampled windows={windows}")
    got, info = run_stack(bl, x, layers)
    ref = orc.stack(x, layers, windows=windows, threads=min(16, os.cpu_count() or 1))
    err = assert_close(got[windows], ref, name)
    assert np.all(np.abs(got) <= 1.0) and np.all(np.isfinite(got))
    note(f"stack {name} max abs err {err:.3e} plan {info}")
    if name == "b256":
        # every all-zero window (b % 10 == 0) gives bitwise the same output
        zeros = got[::10]
        assert np.all(zeros.view(np.uint32) == zeros[0].view(np.uint32)[None])


def test_stack_bit_stable_and_batch_invariant(bl):
    x, layers = workloads.make_workload("b32")
    note("bit stability b32 x3, batch invariance b1/b8/b32")
    plan = bl.Plan(layers, 32, x.shape[1])
    xd = torch.from_numpy(x).cuda()
    runs = [plan.forward(xd).cpu().numpy() for _ in range(3)]
    plan.check()
    plan.close()
    for r in runs[1:]:
        assert np.array_equal(r.view(np.uint32), runs[0].view(np.uint32))
    y1, _ = run_stack(bl, np.ascontiguousarray(x[5:6]), layers)
    y8, _ = run_stack(bl, np.ascontiguousarray(x[:8]), layers)
    assert np.array_equal(y1[0].view(np.uint32), runs[0][5].view(np.uint32))
    assert np.array_equal(y8.view(np.uint32), runs[0][:8].view(np.uint32))


@pytest.mark.parametrize("name,windows", [("b8", None), ("b32", None), ("b256", [0, 3, 10, 255]),
                                          ("b64_t4096", [5])])
def test_stack_with_split_projection_matches_oracle(bl, orc, name, windows):
    """Split-precision projections (bf16 x 3) keep the whole stack within the output tolerance."""
    x, layers = workloads.make_workload(name)
    note(f"stack {name} projection=2 windows={windows}")
    got, info = run_stack(bl, x, layers, projection=2)
    assert info["projection"] == 2
    ref = orc.stack(x, layers, windows=windows, threads=min(16, os.cpu_count() or 1))
    err = assert_close(got if windows is None else got[windows], ref, f"{name} split projection")
    note(f"stack {name} projection=2 max abs err {err:.3e}")


def test_split_projection_batch_invariant(bl):
    """A window's split-precision output is bitwise the same at B = 1 and inside B = 32."""
    x, layers = workloads.make_workload("b32")
    xs = np.ascontiguousarray(x[:, :120])
    y32, _ = run_stack(bl, xs, layers, projection=2)
    y1, _ = run_stack(bl, np.ascontiguousarray(xs[9:10]), layers, projection=2)
    assert np.array_equal(y1[0].view(np.uint32), y32[9].view(np.uint32))


def test_stack_with_library_projection_matches_oracle(bl, orc):
    """The whole stack with the vendor-GEMM projection (comparator) against the oracle."""
    x, layers = workloads.make_workload("b8")
    note("stack b8 projection=1")
    got, info = run_stack(bl, x, layers, projection=1)
    assert info["projection"] == 1 and info["slices"] == 1
    ref = orc.stack(x, layers, threads=min(16, os.cpu_count() or 1))
    err = assert_close(got, ref, "b8 library projection")
    note(f"stack b8 projection=1 max abs err {err:.3e}")


@pytest.mark.parametrize("name,steps,slices", [("b8", 200, 2), ("b8", 200, 3), ("b32", 150, 4), ("b32", 150, 8)])
def test_batch_slices_agree_bitwise(bl, name, steps, slices):
    """Windows are independent, so running the batch as concurrent slices changes nothing."""
    x, layers = workloads.make_workload(name)
    xs = np.ascontiguousarray(x[:, :steps])
    note(f"batch slices {name} steps={steps} slices={slices}")
    got, info = run_stack(bl, xs, layers, slices=slices)
    base, binfo = run_stack(bl, xs, layers, slices=1)
    assert binfo["slices"] == 1 and info["slices"] == min(slices, xs.shape[0])
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))


@pytest.mark.parametrize("concurrent", [0, 1, 2])
def test_direction_modes_agree(bl, concurrent):
    x, layers = workloads.make_workload("b8")
    xs = np.ascontiguousarray(x[:, :200])
    note(f"direction mode concurrent={concurrent}")
    got, info = run_stack(bl, xs, layers, concurrent=concurrent)
    base, _ = run_stack(bl, xs, layers, concurrent=0)
    assert info["concurrent"] == concurrent
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))


def _swap_layer0(layer):
    return {"w": np.ascontiguousarray(layer["w"][::-1]), "r": np.ascontiguousarray(layer["r"][::-1]),
            "b": np.ascontiguousarray(layer["b"][::-1])}


def test_time_reversal_layer0_bitwise(bl):
    """Layer 0 with the directions' weights swapped, on the time-reversed input, gives the
    reversed output with its halves swapped — bit for bit, since both directions run the same
    code and the projection's per-row sum does not depend on the row's position."""
    x, layers = workloads.make_workload("b8")
    x = np.ascontiguousarray(x[:, :100])
    b, t = x.shape[:2]
    note("time reversal layer 0")
    plan = bl.Plan(layers, b, t)
    swapped = [_swap_layer0(layers[0])] + layers[1:]
    plan_s = bl.Plan(swapped, b, t)
    y = plan.recur(0, plan.project(0, torch.from_numpy(x.reshape(b * t, 60)).cuda())).cpu().numpy()
    xr = np.ascontiguousarray(x[:, ::-1])
    yr = plan_s.recur(0, plan_s.project(0, torch.from_numpy(xr.reshape(b * t, 60)).cuda())).cpu().numpy()
    expected = np.concatenate([y[:, ::-1, 128:], y[:, ::-1, :128]], axis=2)
    assert np.array_equal(yr.view(np.uint32), np.ascontiguousarray(expected).view(np.uint32))
    plan.close()
    plan_s.close()


@pytest.mark.parametrize("concurrent", [0, 2])
def test_watchdog_reports_timeout_and_grid_drains(bl, concurrent):
    """Exchange waits forced to time out from the host (watchdog_us = -1: each wait expects a
    flag no producer writes and gives up on its first poll): the kernels still finish, and
    the plan reports BILSTM_TIMEOUT instead of hanging."""
    x, layers = workloads.make_workload("b8")
    xs = np.ascontiguousarray(x[:, :64])
    note(f"watchdog first-miss groups=4 concurrent={concurrent}")
    plan = bl.Plan(layers, 8, 64, groups=4, tile=1, concurrent=concurrent, watchdog_us=-1)
    plan.forward(torch.from_numpy(xs).cuda())
    with pytest.raises(bl.BilstmError) as e:
        plan.check()
    assert e.value.name == "BILSTM_TIMEOUT"
    plan.check()  # the flag was cleared
    plan.close()


def test_forward_rejects_bad_buffers(bl):
    layers = workloads.make_layers(34)
    plan = bl.Plan(layers, 2, 10)
    x = torch.zeros((2, 10, 60), device="cuda")
    with pytest.raises(ValueError):
        plan.forward(torch.zeros((2, 9, 60), device="cuda"))
    lib = bl.library()
    y = torch.zeros((2, 10, 256), device="cuda")
    import ctypes
    st = lib.bilstm_forward(plan._h, ctypes.c_void_p(x.data_ptr()), x.numel() - 1,
                            ctypes.c_void_p(y.data_ptr()), y.numel(), None)
    assert st == 2 and "forward input" in bl.last_error()
    st = lib.bilstm_forward(plan._h, ctypes.c_void_p(x.data_ptr() + 4), x.numel(),
                            ctypes.c_void_p(y.data_ptr()), y.numel(), None)
    assert st == 1 and "aligned" in bl.last_error()
    plan.close()


def test_exchange_probe(bl):
    note("exchange probe")
    same = bl.probe_exchange(0, True, 2000)
    cross = bl.probe_exchange(0, False, 2000)
    note(f"exchange one-way: same-xcd {same} cross-xcd {cross}")
    assert 0 < same["one_way_ns"] < 100000 and 0 < cross["one_way_ns"] < 100000


@pytest.mark.parametrize("steps", [1, 2, 3, 5, 7])
@pytest.mark.parametrize("groups,tile", [(1, 1), (1, 2), (1, 4), (2, 2), (4, 1)])
def test_recurrence_short_sequences(bl, orc, steps, groups, tile):
    """Sequences shorter than the 4-step prefetch ring and its straight-line groups, with a
    ragged last tile (3 windows), for single- and multi-workgroup splits."""
    batch = 3
    layers = workloads.make_layers(35)
    rng = np.random.default_rng(100 + steps)
    gates_src = (rng.standard_normal((batch * steps, 2, 512)) * 1.5).astype(np.float32)
    note(f"short recurrence steps={steps} groups={groups} tile={tile}")
    plan = bl.Plan(layers, batch, steps, groups=groups, tile=tile)
    y = plan.recur(3, torch.from_numpy(to_packed(gates_src)).cuda())
    plan.check()
    got = y.cpu().numpy()
    plan.close()
    per_window = gates_src.reshape(batch, steps, 2, 512)
    for b in range(batch):
        assert_close(got[b], orc.recurrence(per_window[b].astype(np.float64), layers[3]["r"]), f"window {b}")


@pytest.mark.parametrize("batch,steps,slices,projection", [(1, 1, 0, 0), (3, 2, 0, 0), (3, 5, 2, 0), (5, 3, 3, 2),
                                                            (2, 130, 0, 1)])
def test_stack_degenerate_shapes(bl, orc, batch, steps, slices, projection):
    """One frame, a handful of frames (projection rows far below one 128-row tile), sliced
    batches of odd sizes, and every projection mode."""
    layers = workloads.make_layers(36)
    x = workloads.make_input(36, batch, steps)
    note(f"degenerate stack batch={batch} steps={steps} slices={slices} projection={projection}")
    got, info = run_stack(bl, x, layers, slices=slices, projection=projection)
    ref = orc.stack(x, layers)
    assert_close(got, ref, f"b{batch} t{steps}")


def test_torch_lstm_parameters_run_on_the_library(bl):
    # an nn.LSTM's own parameters, converted by the binding, against the module in float64
    torch.manual_seed(21)
    net = torch.nn.LSTM(60, 128, num_layers=4, bidirectional=True, batch_first=True)
    layers = bl.layers_from_state_dict(net.state_dict())
    x = torch.randn(3, 61, 60)
    note("torch nn.LSTM parameters: batch 3, steps 61")
    with torch.no_grad():
        ref, _ = net.double()(x.double())
    plan = bl.Plan(layers, 3, 61, device=0)
    try:
        y = plan.forward(x.to("cuda:0"))
        plan.check()
        assert_close(y.cpu().numpy(), ref.numpy(), "nn.LSTM parameters")
    finally:
        plan.close()
