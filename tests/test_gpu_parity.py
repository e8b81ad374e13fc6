"""GPU parity: the HIP library against the oracle, element by element, on seeded inputs.

Tolerance on the final [B, T, 256] output (allclose form): |gpu - oracle| <= 2e-5 + 1e-4·|oracle|.
The projection alone is held to the rigorous fp32 dot-product bound
|err| <= (K + 2)·u·(sum_k |w_k x_k| + |bias|), u = 2^-24, which holds for any summation order.
"""

import os
import sys
import time

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
    bad = ~(err <= bound)  # NaN (an element never written) fails too
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, np.nan_to_num(err - bound, nan=np.inf), -np.inf)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside tolerance; worst at "
                             f"{idx}: gpu {got[idx]!r} oracle {ref[idx]!r} (max abs err {err.max():.3e})")
    return float(err.max())


def to_packed(oracle_gates):
    """[rows, 2, 512] in source order (g*128 + j) -> [rows, 1024] packed (d*512 + 4j + g)."""
    rows = oracle_gates.shape[0]
    g = oracle_gates.reshape(rows, 2, 4, 128)          # d, gate, unit
    return np.ascontiguousarray(g.transpose(0, 1, 3, 2).reshape(rows, 1024))


def projection_bound(x, layer, parts=0):
    """|gpu - exact| bound of a gate pre-activation. FP32 (parts = 0): (K + 2)·u·(sum|w x| +
    |bias|), any summation order. Split precision in two bf16 parts (three products): the
    dropped part products and the parts' residuals add 3·2^-16·(1 + 2^-7)·sum|w x|, the FP32 sum
    runs over 3K products. Three parts (six products): 4·2^-24·(1 + 2^-7)·sum|w x| for what is
    dropped, over 6K products."""
    w = layer["w"].astype(np.float64)
    b = layer["b"].astype(np.float64)
    k = x.shape[1]
    mag = np.einsum("mk,drk->mdr", np.abs(x.astype(np.float64)), np.abs(w)) + np.abs(b[:, 0] + b[:, 1])[None]
    if parts == 0:
        return to_packed((k + 2) * 2.0 ** -24 * mag * 1.01 + 1e-30)
    if parts == 2:
        coeff = 3 * 2.0 ** -16 * (1 + 2.0 ** -7) + (3 * k + 2) * 2.0 ** -24 * 1.01
    else:
        coeff = 4 * 2.0 ** -24 * (1 + 2.0 ** -7) + (6 * k + 2) * 2.0 ** -24 * 1.01
    return to_packed(coeff * mag * 1.01 + 1e-30)


@pytest.mark.parametrize("layer_index,rows,projection", [(0, 200, 4), (0, 589, 4), (1, 333, 4), (1, 4712, 4),
                                                         (1, 18848, 4), (0, 589, 0), (1, 18848, 0),
                                                         (0, 589, 1), (1, 4712, 1),
                                                         (0, 589, 2), (1, 333, 2), (1, 18848, 2),
                                                         (0, 589, 3), (0, 18848, 3), (1, 333, 3), (1, 18848, 3)])
def test_projection_matches_oracle(bl, orc, layer_index, rows, projection):
    """The projection alone against the oracle, within the summation-order-free bound of the
    arithmetic the plan runs: FP32 products (4, and the vendor-GEMM comparator 1), two or three
    bf16 parts (2, 3); 0 checks the bound of what the plan's rule chose."""
    layers = workloads.make_layers(31)
    width = 60 if layer_index == 0 else 256
    x = np.random.default_rng(rows).standard_normal((rows, width)).astype(np.float32)
    if layer_index > 0:
        x = np.tanh(x).astype(np.float32)  # later layers see hidden states in (-1, 1)
    note(f"projection layer={layer_index} rows={rows} projection={projection}")
    plan = bl.Plan(layers, rows, 1, projection=projection)
    assert projection == 0 or plan.info()["projection"] == projection
    gates = plan.project(layer_index, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    ref = to_packed(orc.projection(x, layers[layer_index]["w"], layers[layer_index]["b"]))
    err = np.abs(gates.cpu().numpy().astype(np.float64) - ref)
    chosen = plan.info()["projection"]
    bound = projection_bound(x, layers[layer_index], parts=chosen if chosen in (2, 3) else 0)
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


def run_repeated(bl, x, layers, repeats=3, **kw):
    """`repeats` forwards on one plan, each into an output filled with NaN first, so an element
    a forward leaves unwritten cannot pass as stable or as close to the oracle."""
    plan = bl.Plan(layers, x.shape[0], x.shape[1], **kw)
    xd = torch.from_numpy(x).cuda()
    outs = []
    for _ in range(repeats):
        y = torch.full((x.shape[0], x.shape[1], 256), float("nan"), dtype=torch.float32, device="cuda")
        plan.forward(xd, y)
        outs.append(y.cpu().numpy())
    plan.check()
    info = plan.info()
    plan.close()
    return outs, info


THREADS = min(16, os.cpu_count() or 1)
_REFERENCE = {}


def oracle_reference(orc, name):
    """The oracle's whole [B, T, 256] output of a workload (fp64), computed once per session."""
    if name not in _REFERENCE:
        x, layers = workloads.make_workload(name)
        t0 = time.perf_counter()
        _REFERENCE[name] = orc.stack(x, layers, threads=THREADS)
        note(f"oracle {name}: {x.shape[0]} windows in {time.perf_counter() - t0:.1f} s on {THREADS} threads")
    return _REFERENCE[name]


ALL_WORKLOADS = ["b1", "b8", "b32", "b256", "b64_t4096"]


def assert_bitwise_equal(runs, what):
    for k, r in enumerate(runs[1:], 1):
        same = r.view(np.uint32) == runs[0].view(np.uint32)
        assert same.all(), f"{what}: forward {k} differs from forward 0 in {(~same).sum()} elements"


@pytest.mark.parametrize("name", ALL_WORKLOADS)
def test_stack_whole_output_matches_oracle_and_is_bit_stable(bl, orc, name):
    """Every window of every workload, in the plan the library chooses by default (the launch
    configuration the benchmark times): three forwards on one plan agree bit for bit, and
    every element of the [B, T, 256] output is within tolerance of the fp64 oracle."""
    x, layers = workloads.make_workload(name)
    note(f"stack {name} shape={x.shape}: 3 forwards, whole output against the oracle")
    runs, info = run_repeated(bl, x, layers)
    assert_bitwise_equal(runs, name)
    got = runs[0]
    assert np.all(np.isfinite(got)) and np.all(np.abs(got) <= 1.0)
    err = assert_close(got, oracle_reference(orc, name), name)
    note(f"stack {name} max abs err {err:.3e} plan {info}")
    if name == "b256":
        # every all-zero window (b % 10 == 0) gives bitwise the same output
        zeros = got[::10]
        assert np.all(zeros.view(np.uint32) == zeros[0].view(np.uint32)[None])


def test_stack_batch_invariant(bl):
    """A window's output is bitwise the same alone, inside 8 windows and inside 32."""
    x, layers = workloads.make_workload("b32")
    note("batch invariance b1/b8/b32")
    y32, _ = run_stack(bl, x, layers)
    y1, _ = run_stack(bl, np.ascontiguousarray(x[5:6]), layers)
    y8, _ = run_stack(bl, np.ascontiguousarray(x[:8]), layers)
    assert np.array_equal(y1[0].view(np.uint32), y32[5].view(np.uint32))
    assert np.array_equal(y8.view(np.uint32), y32[:8].view(np.uint32))


@pytest.mark.parametrize("projection", [2, 3])
@pytest.mark.parametrize("name", ALL_WORKLOADS)
def test_stack_with_split_projection_matches_oracle(bl, orc, name, projection):
    """Split-precision projections (two bf16 parts, three products; three parts, six products),
    streamed where the plan streams: every element of the whole stack's output within the
    output tolerance, bit-stable over three forwards."""
    x, layers = workloads.make_workload(name)
    note(f"stack {name} projection={projection}: 3 forwards, whole output against the oracle")
    runs, info = run_repeated(bl, x, layers, projection=projection)
    assert info["projection"] == projection
    assert_bitwise_equal(runs, f"{name} split projection")
    err = assert_close(runs[0], oracle_reference(orc, name), f"{name} split projection")
    note(f"stack {name} projection={projection} streamed={info['pipeline']} max abs err {err:.3e}")


EXCHANGE_SPLITS = [(2, 1), (2, 2), (2, 4), (4, 1), (4, 2), (4, 4)]


@pytest.mark.parametrize("groups,tile", EXCHANGE_SPLITS)
def test_exchange_stack_matches_oracle_over_repeated_forwards(bl, orc, groups, tile):
    """The whole four-layer stack with KG workgroups per tile exchanging h through flagged
    words. Each layer's flags start above the previous layer's and each pass's above the last
    pass's, so three forwards on one plan run flag_base = epoch + layer·T over twelve layer
    passes: all three agree bit for bit, match the oracle, and equal the single-workgroup
    default (every split sums in the same order)."""
    x, layers = workloads.make_workload("b8")
    note(f"exchange stack b8 groups={groups} tile={tile}: 3 forwards")
    runs, info = run_repeated(bl, x, layers, groups=groups, tile=tile)
    assert info["recur_groups"] == groups and info["recur_tile"] == tile
    assert_bitwise_equal(runs, f"groups={groups} tile={tile}")
    err = assert_close(runs[0], oracle_reference(orc, "b8"), f"b8 groups={groups} tile={tile}")
    base, _ = run_stack(bl, x, layers)
    assert np.array_equal(runs[0].view(np.uint32), base.view(np.uint32))
    note(f"exchange stack b8 groups={groups} tile={tile} max abs err {err:.3e} plan {info}")


def test_serial_directions_b256_match_oracle(bl, orc):
    """b256 with four workgroups per one-window tile: 2048 workgroups, twice what the device
    keeps resident, so the two directions run one after the other. The whole output matches
    the oracle and equals the default plan bit for bit."""
    x, layers = workloads.make_workload("b256")
    note("serial directions b256 groups=4 tile=1")
    got, info = run_stack(bl, x, layers, groups=4, tile=1)
    note(f"serial-direction plan {info}")
    assert info["concurrent"] == 0
    err = assert_close(got, oracle_reference(orc, "b256"), "b256 groups=4 tile=1")
    base, _ = run_stack(bl, x, layers)
    assert np.array_equal(got.view(np.uint32), base.view(np.uint32))
    note(f"serial directions b256 max abs err {err:.3e}")


@pytest.mark.parametrize("batch,steps,groups,tile", [(384, 96, 4, 1), (520, 40, 4, 1), (520, 40, 2, 1),
                                                     (1024, 24, 4, 2)])
def test_multi_launch_schedule_matches_oracle(bl, orc, batch, steps, groups, tile):
    """More workgroups per direction than the device keeps resident: each direction's
    recurrence is cut into several launches, run serially, each over its own tiles. Three
    forwards on one plan (each layer of each pass takes its own flag range) agree bit for
    bit, match the oracle and equal the default plan."""
    layers = workloads.make_layers(91)
    x = workloads.make_input(92 + batch, batch, steps)
    note(f"multi-launch batch={batch} steps={steps} groups={groups} tile={tile}: 3 forwards")
    runs, info = run_repeated(bl, x, layers, groups=groups, tile=tile)
    note(f"multi-launch plan {info}")
    assert info["recur_launches"] > 1
    assert_bitwise_equal(runs, f"multi-launch b{batch}")
    err = assert_close(runs[0], orc.stack(x, layers, threads=THREADS), f"multi-launch b{batch}")
    base, _ = run_stack(bl, x, layers)
    assert np.array_equal(runs[0].view(np.uint32), base.view(np.uint32))
    note(f"multi-launch batch={batch} launches={info['recur_launches']} max abs err {err:.3e}")


@pytest.mark.parametrize("name", ["b8", "b32", "b256", "b64_t4096"])
def test_three_part_split_is_as_accurate_as_fp32(bl, orc, name):
    """The accuracy side of the projection rule, rerun: on each workload the rule may split
    (at least 2048 rows), the stack with the three-part split stays within 1.1 times the
    largest error of the stack with FP32 products against the fp64 oracle (the factor of the
    pages' own check); the two-part split does not, and the rule never picks it."""
    x, layers = workloads.make_workload(name)
    ref = oracle_reference(orc, name)
    errs = {}
    for mode in (4, 3, 2):
        got, info = run_stack(bl, x, layers, projection=mode)
        errs[mode] = float(np.max(np.abs(got.astype(np.float64) - ref)))
    note(f"rule check {name}: largest error fp32 {errs[4]:.3e}, three parts {errs[3]:.3e} "
         f"({errs[3] / errs[4]:.3f}x), two parts {errs[2]:.3e} ({errs[2] / errs[4]:.3f}x)")
    assert errs[3] <= 1.1 * errs[4]
    assert errs[2] > 1.1 * errs[4]
    assert bl.schedule(x.shape[0], x.shape[1], 256, 1)["projection"] in (3, 4)


def test_split_projection_batch_invariant(bl):
    """A window's split-precision output is bitwise the same at B = 1 and inside B = 32."""
    x, layers = workloads.make_workload("b32")
    xs = np.ascontiguousarray(x[:, :120])
    y32, _ = run_stack(bl, xs, layers, projection=2)
    y1, _ = run_stack(bl, np.ascontiguousarray(xs[9:10]), layers, projection=2)
    assert np.array_equal(y1[0].view(np.uint32), y32[9].view(np.uint32))


@pytest.mark.parametrize("layer_index", [0, 1])
def test_fp32_projection_rows_independent_of_the_launch(bl, layer_index):
    """The FP32 projection runs one workgroup per CU when few tile rounds are needed (4,000 rows:
    256 tiles) and two when that is faster (40,000 rows: 2,504 tiles); a row's gates are
    bitwise the same either way."""
    layers = workloads.make_layers(77)
    width = 60 if layer_index == 0 else 256
    x = np.tanh(np.random.default_rng(5).standard_normal((40000, width))).astype(np.float32)
    note(f"fp32 projection launch invariance layer={layer_index}")
    out = {}
    for rows in (4000, 40000):
        plan = bl.Plan(layers, rows, 1, projection=4)
        out[rows] = plan.project(layer_index, torch.from_numpy(np.ascontiguousarray(x[:rows])).cuda()).cpu().numpy()
        plan.close()
    assert np.array_equal(out[4000].view(np.uint32), out[40000][:4000].view(np.uint32))


def test_stack_at_the_largest_accepted_size(bl, orc):
    """1023 windows of 4096 steps, the largest batch of that length the 32-bit indexing
    accepts (4,190,208 rows; 1024 windows are refused): the default plan's forward, every
    output finite and within [-1, 1], and the first, a middle and the last window element by
    element against the oracle."""
    batch, steps = 1023, 4096
    layers = workloads.make_layers(4099)
    x = workloads.make_input(4099, batch, steps)
    note(f"largest size batch={batch} steps={steps}")
    plan = bl.Plan(layers, batch, steps)
    y = plan.forward(torch.from_numpy(x).cuda())
    plan.check()
    info = plan.info()
    assert bool(torch.isfinite(y).all()) and float(y.abs().max()) <= 1.0
    sample = [0, 511, 1022]
    ref = orc.stack(x, layers, threads=len(sample), windows=sample)
    for i, w in enumerate(sample):
        err = assert_close(y[w].cpu().numpy(), ref[i], f"largest size window {w}")
        note(f"largest size window {w} max abs err {err:.3e} plan {info}")
    plan.close()
    del y
    torch.cuda.empty_cache()


def test_streamed_stack_past_two_gigabytes_of_input(bl, orc):
    """64 windows of 34,000 steps with streamed gates: the layer inputs exceed 2 GiB, so the
    streamed projection's 32-bit byte offsets pass 2^31. The last window against the oracle;
    the first and the last bitwise equal to the same window run alone."""
    batch, steps = 64, 34000
    layers = workloads.make_layers(34001)
    x = workloads.make_input(34001, batch, steps)
    note(f"streamed past 2 GiB batch={batch} steps={steps}")
    plan = bl.Plan(layers, batch, steps)
    info = plan.info()
    assert info["pipeline"] == 1
    y = plan.forward(torch.from_numpy(x).cuda())
    plan.check()
    plan.close()
    assert bool(torch.isfinite(y).all()) and float(y.abs().max()) <= 1.0
    for w in (0, batch - 1):
        one, _ = run_stack(bl, np.ascontiguousarray(x[w:w + 1]), layers, projection=info["projection"])
        assert np.array_equal(one[0].view(np.uint32), y[w].cpu().numpy().view(np.uint32)), f"window {w}"
    err = assert_close(y[batch - 1].cpu().numpy(), orc.stack(x, layers, windows=[batch - 1])[0], "last window")
    note(f"streamed past 2 GiB last window max abs err {err:.3e}")
    del y
    torch.cuda.empty_cache()


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
    plan.check()  # the report was cleared
    plan.close()


@pytest.mark.parametrize("pipeline,groups", [(1, 4), (2, 1)])
def test_timeout_reaches_the_next_forward_without_check(bl, pipeline, groups):
    """A forward whose waits time out (forced) returns OK when it enqueues; once it has run, the
    next forward on the plan returns BILSTM_TIMEOUT by itself, without bilstm_check, enqueues
    nothing, and clears the report, so the forward after it is accepted again."""
    x, layers = workloads.make_workload("b8")
    xs = torch.from_numpy(np.ascontiguousarray(x[:, :64])).cuda()
    note(f"timeout without check: pipeline={pipeline} groups={groups}")
    plan = bl.Plan(layers, 8, 64, groups=groups, tile=1, pipeline=pipeline, watchdog_us=-1)
    try:
        y = torch.zeros((8, 64, 256), dtype=torch.float32, device="cuda")
        plan.forward(xs, y)
        torch.cuda.synchronize()  # the caller waits on its own stream only
        marker = torch.full_like(y, 7.0)
        with pytest.raises(bl.BilstmError) as e:
            plan.forward(xs, marker)
        assert e.value.name == "BILSTM_TIMEOUT" and "earlier call" in str(e.value)
        torch.cuda.synchronize()
        assert bool(torch.all(marker == 7.0)), "a forward that reported a timeout enqueued work"
        plan.forward(xs, y)  # accepted again
        torch.cuda.synchronize()
        with pytest.raises(bl.BilstmError) as e:
            plan.check()
        assert e.value.name == "BILSTM_TIMEOUT"
    finally:
        plan.close()


def test_check_waits_for_the_plan_only(bl):
    """bilstm_check waits for the plan's last call, not for the device: work pending on another
    stream is still running when it returns."""
    x, layers = workloads.make_workload("b8")
    xs = torch.from_numpy(np.ascontiguousarray(x[:, :100])).cuda()
    plan = bl.Plan(layers, 8, 100)
    try:
        # calibrate torch's spin kernel: cycles per millisecond on this device
        probe = torch.cuda.Stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(probe):
            e0.record()
            torch.cuda._sleep(10_000_000)
            e1.record()
        probe.synchronize()
        per_ms = 10_000_000 / max(e0.elapsed_time(e1), 1e-3)
        note(f"check scope: spin kernel {per_ms:.0f} cycles/ms")
        other = torch.cuda.Stream()
        y = torch.empty((8, 100, 256), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(other):
            torch.cuda._sleep(int(per_ms * 1500))  # about 1.5 s
        t0 = time.perf_counter()
        plan.forward(xs, y)
        plan.check()
        waited = time.perf_counter() - t0
        busy = not other.query()
        other.synchronize()
        note(f"check scope: check returned after {waited * 1e3:.1f} ms; other stream still busy: {busy}")
        assert busy and waited < 1.0
    finally:
        plan.close()


@pytest.mark.parametrize("groups,pipeline", [(1, 2), (1, 4), (1, 3), (4, 1), (2, 1)])
def test_near_wrap_counters_clear_and_stay_bitwise(bl, groups, pipeline):
    """Flags and pass numbers started just below their clear thresholds (test hook): the first
    forward runs with values at the top of their range, the second clears the exchange words
    (groups > 1) or the streamed counters and progress words (pipeline 2-4) and starts from
    zero. Four forwards agree bit for bit with a plan that never came near a wrap."""
    x, layers = workloads.make_workload("b8")
    xs = np.ascontiguousarray(x[:, :150])
    note(f"near wrap groups={groups} pipeline={pipeline}")
    plan = bl.Plan(layers, 8, 150, groups=groups, tile=1, pipeline=pipeline, near_wrap=1)
    xd = torch.from_numpy(xs).cuda()
    try:
        outs, clears = [], []
        for _ in range(4):
            outs.append(plan.forward(xd).cpu().numpy())
            clears.append(plan.info()["clears"])
        plan.check()
    finally:
        plan.close()
    note(f"near wrap groups={groups} pipeline={pipeline}: clears after each forward {clears}")
    assert clears[0] == 0 and clears[1] == 1 and clears[-1] == 1
    base, _ = run_stack(bl, xs, layers, groups=groups, tile=1, pipeline=pipeline)
    for o in outs:
        assert np.array_equal(o.view(np.uint32), base.view(np.uint32))


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


def test_fma_rate_probe(bl):
    """The FMA issue rate behind the recurrence's bound: with two or more waves per SIMD a SIMD
    retires one wave64 FP32 FMA about every two shader clocks (128 per clock per CU, the rate the
    published FP32 vector peak implies); a single wave issues at most every clock."""
    out = {wps: bl.probe_fma_rate(0, wps, 1, 4000) for wps in (1, 2, 4)}
    note(f"fma rate probe: {out}")
    for wps, r in out.items():
        assert 1.0 <= r["clocks_per_fma"] < 16 and 0.5 < r["ghz"] < 4.0
    assert out[2]["clocks_per_fma"] < 3.0


def test_mfma_rate_probe(bl):
    """The matrix-core rates behind the projection's peaks: bf16 32x32x16 MFMAs on zero operands
    near the published dense bf16 peak, FP32 32x32x2 near the FP32 one, and random operands no
    faster than zeros; bad arguments are rejected before any launch."""
    bf16 = bl.probe_mfma_rate(0, 0, 0, 2000)
    fp32 = bl.probe_mfma_rate(1, 0, 0, 500)
    rnd = bl.probe_mfma_rate(0, 2, 0, 2000)
    note(f"mfma rate probe: bf16 zeros {bf16}, fp32 zeros {fp32}, bf16 uniform {rnd}")
    assert 1500 < bf16["tflops"] < 2700 and 100 < fp32["tflops"] < 170
    assert rnd["tflops"] < 1.05 * bf16["tflops"]
    with pytest.raises(bl.BilstmError):
        bl.probe_mfma_rate(2, 0)
    with pytest.raises(bl.BilstmError):
        bl.probe_mfma_rate(0, 3)


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
