"""GPU: streamed gates (each layer's projection beside its own recurrence, published chunk by
chunk through counters the recurrence polls).

The projection's per-row sum and the recurrence do not depend on the order tiles run in, so a
streamed forward must equal the unstreamed one bit for bit, for every batch and sequence
shape (ragged row blocks, sequences shorter than one chunk or than the prefetch ring), over
repeated forwards on one plan (the counters' targets advance per pass), and the oracle bounds
it as it does the default path.
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


def run(bl, x, layers, repeats=1, **kw):
    plan = bl.Plan(layers, x.shape[0], x.shape[1], **kw)
    xd = torch.from_numpy(x).cuda()
    outs = [plan.forward(xd).cpu().numpy() for _ in range(repeats)]
    plan.check()
    info = plan.info()
    plan.close()
    return outs, info


# (batch, steps, tile): one window (chunks of 128 steps), two (64), three and more (32); steps
# below one chunk, below the 8 steps the counters are read ahead, just past a chunk, not a
# whole number of chunks
SHAPES = [(1, 589, 0), (1, 1, 0), (1, 129, 0), (2, 130, 0), (2, 65, 0), (3, 150, 0), (3, 3, 0), (5, 7, 0),
          (4, 33, 0), (4, 17, 0), (8, 200, 0), (8, 97, 2), (8, 64, 4), (32, 150, 0),
          # one-window tiles prefetch 16 steps: sequences just short of, at and past whole rings
          (3, 15, 0), (2, 16, 0), (4, 32, 0), (1, 48, 0),
          # projection grids of 128 and 64 workgroups beside the recurrence
          (64, 70, 0), (96, 40, 0)]


@pytest.mark.parametrize("pipeline", [2, 4, 3, 5])
@pytest.mark.parametrize("batch,steps,tile", SHAPES)
def test_streamed_equals_unstreamed_bitwise(bl, batch, steps, tile, pipeline):
    """pipeline 2: the next layer's projection runs during this layer's recurrence, reading the
    rows it publishes; 4: the same with the four recurrences as one launch; 3: each projection
    after the previous layer's recurrence; 5: as 3, each recurrence after its projection (the
    streamed kernels one at a time)."""
    x = workloads.make_input(40 + batch, batch, steps)
    layers = workloads.make_layers(41)
    note(f"streamed (pipeline={pipeline}) vs unstreamed batch={batch} steps={steps} tile={tile}")
    got, info = run(bl, x, layers, pipeline=pipeline, tile=tile)
    base, binfo = run(bl, x, layers, pipeline=1, slices=1, tile=tile)
    assert info["pipeline"] == 1 and binfo["pipeline"] == 0
    assert info["stream_overlap"] == (0 if pipeline in (3, 5) else 1)
    assert info["stream_serial"] == (1 if pipeline == 5 else 0)
    one_launch = info["concurrent"] == 2 and info["recur_launches"] == 1
    assert info["stream_fused"] == (1 if pipeline == 4 and one_launch else 0)
    assert np.array_equal(got[0].view(np.uint32), base[0].view(np.uint32))


@pytest.mark.parametrize("projection", [2, 3])
@pytest.mark.parametrize("pipeline", [2, 4, 5])
@pytest.mark.parametrize("batch,steps,tile", SHAPES)
def test_streamed_split_equals_unstreamed_split_bitwise(bl, batch, steps, tile, pipeline, projection):
    """The streamed kernel splits its FP32 operands into bf16 parts after the LDS ring, the
    plain split kernel while staging x (W split at plan creation): the same parts, the same
    products in the same order, so the gates, and the stack's output, are bitwise the same, for
    every shape the FP32 streamed path is checked on."""
    x = workloads.make_input(60 + batch, batch, steps)
    layers = workloads.make_layers(61)
    note(f"streamed split projection={projection} pipeline={pipeline} batch={batch} steps={steps} tile={tile}")
    got, info = run(bl, x, layers, pipeline=pipeline, tile=tile, projection=projection)
    base, binfo = run(bl, x, layers, pipeline=1, slices=1, tile=tile, projection=projection)
    assert info["pipeline"] == 1 and binfo["pipeline"] == 0 and info["projection"] == projection
    assert np.array_equal(got[0].view(np.uint32), base[0].view(np.uint32))


def tiles_per_projection_workgroup(info):
    """Most streamed tiles one projection workgroup of a layer holds: chunks of stream_chunk
    steps, windows in groups of 128 / stream_chunk, four 128-column tiles per chunk, direction
    and group (chunk 0 cut `stream_split` times), on the CUs the recurrence leaves."""
    chunk = info["stream_chunk"]
    chunks = -(-info["steps"] // chunk)
    groups = -(-info["batch"] // (128 // chunk))
    tiles = (chunks - 1 + info["stream_split"]) * 2 * groups * 4
    workgroups = max(8, (info["cu_count"] - 2 * info["recur_tiles"] * info["recur_groups"]) // 8 * 8)
    return -(-tiles // workgroups)


# Shapes whose projection workgroups hold 8 tiles or more each: beside the previous layer's
# recurrence they take the tiles whose rows exist first (the walk), then the rest in order.
WALK_SHAPES = [(64, 600), (48, 400), (96, 300), (64, 4096)]


@pytest.mark.parametrize("projection", [4, 3])
@pytest.mark.parametrize("pipeline", [2, 4])
@pytest.mark.parametrize("batch,steps", WALK_SHAPES)
def test_streamed_walk_equals_unstreamed_bitwise(bl, batch, steps, pipeline, projection):
    """The walk changes when tiles are computed, not what they compute: bitwise equal to the
    unstreamed stack, over two forwards on one plan."""
    x = workloads.make_input(80 + batch, batch, steps)
    layers = workloads.make_layers(81)
    note(f"streamed walk pipeline={pipeline} projection={projection} batch={batch} steps={steps}")
    got, info = run(bl, x, layers, repeats=2, pipeline=pipeline, projection=projection)
    assert info["pipeline"] == 1 and info["stream_overlap"] == 1
    assert tiles_per_projection_workgroup(info) >= 8
    base, _ = run(bl, x, layers, pipeline=1, slices=1, projection=projection)
    for g in got:
        assert np.array_equal(g.view(np.uint32), base[0].view(np.uint32))


@pytest.mark.parametrize("batch,steps,forwards,projection", [(64, 600, 60, 4), (64, 600, 60, 3), (64, 4096, 12, 3)])
def test_streamed_walk_many_forwards_are_bit_stable(bl, batch, steps, forwards, projection):
    """Many forwards on one plan whose projection workgroups walk: the walk's choices depend
    on timing, the gates do not, so every forward's output is the first one's, bit for bit
    (compared as integers on the GPU), and the plan reports no error."""
    x = workloads.make_input(70, batch, steps)
    layers = workloads.make_layers(71)
    note(f"streamed walk {forwards} forwards batch={batch} steps={steps} projection={projection}")
    plan = bl.Plan(layers, batch, steps, pipeline=2, projection=projection)
    assert tiles_per_projection_workgroup(plan.info()) >= 8
    xd = torch.from_numpy(x).cuda()
    first = plan.forward(xd).view(torch.int32).clone()
    y = torch.empty((batch, steps, 256), dtype=torch.float32, device="cuda")
    for _ in range(forwards - 1):
        plan.forward(xd, y)
        assert torch.equal(y.view(torch.int32), first)
    plan.check()
    plan.close()


@pytest.mark.parametrize("pipeline", [2, 4, 3])
def test_streamed_repeated_forwards_are_bit_stable(bl, pipeline):
    """Five forwards on one plan: each pass's counters reach the next target exactly once."""
    x, layers = workloads.make_workload("b8")
    xs = np.ascontiguousarray(x[:, :150])
    note(f"streamed repeated forwards b8 t150 x5 pipeline={pipeline}")
    outs, info = run(bl, xs, layers, repeats=5, pipeline=pipeline)
    assert info["pipeline"] == 1
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def test_streamed_matches_oracle(bl, orc):
    x, layers = workloads.make_workload("b8")
    note("streamed b8 against the oracle")
    outs, info = run(bl, x, layers, pipeline=4)
    ref = orc.stack(x, layers, threads=min(16, os.cpu_count() or 1))
    err = np.abs(outs[0].astype(np.float64) - ref)
    assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"max abs err {err.max():.3e}"
    note(f"streamed b8 max abs err {err.max():.3e} chunk {info['stream_chunk']}")


@pytest.mark.parametrize("pipeline", [2, 4, 3])
def test_streamed_phase_times(bl, pipeline):
    x, layers = workloads.make_workload("b8")
    xs = np.ascontiguousarray(x[:, :100])
    note(f"streamed phase times pipeline={pipeline}")
    plan = bl.Plan(layers, 8, 100, pipeline=pipeline)
    xd = torch.from_numpy(xs).cuda()
    ref = plan.forward(xd).cpu().numpy()
    plan.set_phase_events(True)
    got = plan.forward(xd).cpu().numpy()
    t = plan.phase_times()
    plan.check()
    fused = plan.info()["stream_fused"]
    plan.close()
    assert fused == (1 if pipeline == 4 else 0)
    # timing changes nothing in the results
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    rec = t["recurrence_ms"]
    for l in range(4):
        # phase ends from the forward's start: recurrences end in order, each after the
        # projection whose gates it reads, and each launch (or layer's share of the one
        # launch) lasts at most until its end
        assert 0 < t["projection_ms"][l] < rec[l] + 1e-3
        assert l == 0 or rec[l - 1] < rec[l]
        assert 0 < t["recurrence_launch_ms"][l] <= rec[l] + 1e-3
    if fused:
        # the shares of the one launch add up to it and end with the last recurrence
        total = sum(t["recurrence_launch_ms"])
        assert total <= rec[3] + 1e-3
        assert abs((rec[3] - rec[0]) - sum(t["recurrence_launch_ms"][1:])) < 1e-2


@pytest.mark.parametrize("projection", [4, 3])
@pytest.mark.parametrize("pipeline", [2, 4, 3])
def test_streamed_watchdog_reports_timeout_and_grid_drains(bl, pipeline, projection):
    """Counter waits forced to time out from the host (watchdog_us = -1: every wait expects a
    count no pass reaches and gives up on its first poll): the kernels finish and the plan
    reports BILSTM_TIMEOUT; a normal plan afterwards is unaffected. Both streamed projection
    kernels (FP32 and split precision)."""
    x, layers = workloads.make_workload("b8")
    xs = np.ascontiguousarray(x[:, :64])
    note(f"streamed watchdog first-miss pipeline={pipeline} projection={projection}")
    plan = bl.Plan(layers, 8, 64, pipeline=pipeline, watchdog_us=-1, projection=projection)
    plan.forward(torch.from_numpy(xs).cuda())
    with pytest.raises(bl.BilstmError) as e:
        plan.check()
    assert e.value.name == "BILSTM_TIMEOUT"
    plan.check()
    plan.close()
    got, _ = run(bl, xs, layers, pipeline=2)
    base, _ = run(bl, xs, layers, pipeline=1)
    assert np.array_equal(got[0].view(np.uint32), base[0].view(np.uint32))


@pytest.mark.parametrize("projection", [4, 3])
def test_streamed_walk_watchdog_reports_timeout_and_grid_drains(bl, projection):
    """As above on a shape whose projection workgroups walk (48 windows × 400 steps): with every
    wait giving up at once the walk still takes each tile once and every workgroup ends."""
    x = workloads.make_input(90, 48, 400)
    layers = workloads.make_layers(91)
    note(f"streamed walk watchdog first-miss projection={projection}")
    plan = bl.Plan(layers, 48, 400, pipeline=2, watchdog_us=-1, projection=projection)
    assert tiles_per_projection_workgroup(plan.info()) >= 8
    plan.forward(torch.from_numpy(x).cuda())
    with pytest.raises(bl.BilstmError) as e:
        plan.check()
    assert e.value.name == "BILSTM_TIMEOUT"
    plan.check()
    plan.close()
    got, _ = run(bl, x, layers, pipeline=2, projection=projection)
    base, _ = run(bl, x, layers, pipeline=1, slices=1, projection=projection)
    assert np.array_equal(got[0].view(np.uint32), base[0].view(np.uint32))


@pytest.mark.parametrize("pipeline", [0, 1])
def test_forward_follows_the_callers_stream(bl, pipeline):
    # The forward runs in the order of the stream it is given: work queued on that stream
    # before it (a long spin, then new input) is seen by every layer, and work queued after it
    # (a copy of the output) sees the whole stack. Streamed (pipeline 0 = auto) and unstreamed.
    batch, steps = 8, 300
    layers = workloads.make_layers(77)
    x_old = torch.from_numpy(workloads.make_input(78, batch, steps)).cuda()
    x_new = torch.from_numpy(workloads.make_input(79, batch, steps)).cuda()
    note(f"caller's stream: pipeline {pipeline}, batch {batch}, steps {steps}")
    plan = bl.Plan(layers, batch, steps, device=0, pipeline=pipeline)
    try:
        ref = plan.forward(x_new)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()  # default priority
        x = x_old.clone()
        y = torch.zeros_like(ref)
        out = torch.empty_like(ref)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            torch.cuda._sleep(20_000_000)   # keeps the stream busy for milliseconds
            x.copy_(x_new)
            plan.forward(x, y, stream=side)
            out.copy_(y)
        side.synchronize()
        plan.check()
        assert torch.equal(out, ref)
    finally:
        plan.close()
