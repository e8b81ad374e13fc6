"""Host-side tests of the HIP library: it loads, exports every symbol the header declares,
and its packer, schedule and argument checks behave — all without a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bilstm.h")


@pytest.fixture(scope="module")
def bl():
    import bidirectional_lstm_sequence_amd as bl
    if not os.path.exists(bl.LIB_PATH):
        from bidirectional_lstm_sequence_amd import _build
        _build.build()
    bl.library()
    return bl


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:bilstm_status|void|const char\s*\*)\s*(bilstm_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["bilstm_plan_create", "bilstm_forward", "bilstm_destroy", "bilstm_last_error"]:
        assert required in names


def test_library_exports_every_declared_symbol(bl):
    lib = ctypes.CDLL(bl.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in bilstm.h but not exported"
    assert sorted(bl.EXPORTS) == declared_functions()


def test_library_does_not_link_the_oracle(bl):
    with open(bl.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"oracle_stack_window" not in blob and b"liboracle" not in blob


def _interleaved_reference(layer, width):
    """Packed layout written out from its definition: row d*512 + 4j + g <- source row g*128 + j."""
    kpad = (width + 31) // 32 * 32
    w = np.zeros((1024, kpad), np.float32)
    r = np.zeros((2, 512, 128), np.float32)
    b = np.zeros(1024, np.float32)
    for d in range(2):
        for g in range(4):
            for j in range(128):
                w[d * 512 + 4 * j + g, :width] = layer["w"][d, g * 128 + j]
                r[d, 4 * j + g] = layer["r"][d, g * 128 + j]
                b[d * 512 + 4 * j + g] = np.float32(layer["b"][d, 0, g * 128 + j]) + np.float32(layer["b"][d, 1, g * 128 + j])
    return w, r, b


@pytest.mark.parametrize("width", [60, 256])
def test_pack_layer_interleaves_gates_and_folds_bias(bl, width):
    layer = workloads.make_layers(21)[0 if width == 60 else 1]
    w, r, b = bl.pack_layer(layer, width)
    ew, er, eb = _interleaved_reference(layer, width)
    np.testing.assert_array_equal(w, ew)
    np.testing.assert_array_equal(r, er)
    np.testing.assert_array_equal(b, eb)
    # the padding columns are zero
    assert not np.any(w[:, width:])


def test_pack_layer_rejects_wrong_lengths(bl):
    layer = workloads.make_layers(22)[0]
    bad = dict(layer)
    bad["w"] = layer["w"][:, :, :59].copy()
    with pytest.raises(bl.BilstmError) as e:
        bl.pack_layer(bad, 60)
    assert e.value.name == "BILSTM_BUFFER_LENGTH"
    assert "expected" in str(e.value)


@pytest.mark.parametrize("batch", [1, 7, 8, 32, 100, 256, 1000])
@pytest.mark.parametrize("groups", [0, 1, 2, 4, 8, 16])
def test_schedule_fits_resident_capacity(bl, batch, groups):
    cu, per_cu = 256, 1
    try:
        s = bl.schedule(batch, 589, cu, per_cu, groups=groups)
    except bl.BilstmError as e:
        assert e.name == "BILSTM_UNSUPPORTED"
        return
    cap = cu * per_cu
    assert s["recur_tiles"] * s["recur_tile"] >= batch
    assert (s["recur_tiles"] - 1) * s["recur_tile"] < batch
    per_launch = -(-s["recur_tiles"] // s["recur_launches"])
    if s["recur_groups"] > 1:
        # workgroups of a tile wait for each other: every launch must be resident at once
        assert per_launch * s["recur_groups"] <= cap
        if s["concurrent"]:
            assert 2 * s["recur_tiles"] * s["recur_groups"] <= cap
    assert s["recur_threads"] == 4 * (128 // s["recur_groups"])


def test_schedule_default_prefers_small_tiles(bl):
    assert bl.schedule(32, 589, 256, 1)["recur_tile"] == 1
    s = bl.schedule(256, 589, 256, 1)
    assert s["recur_tile"] == 2 and s["recur_tiles"] == 128


def test_schedule_refuses_concurrency_that_cannot_be_resident(bl):
    with pytest.raises(bl.BilstmError) as e:
        bl.schedule(256, 589, 256, 1, groups=4, tile=1, concurrent=1)
    assert e.value.name == "BILSTM_UNSUPPORTED"
    s = bl.schedule(256, 589, 256, 1, groups=4, tile=1)
    assert s["concurrent"] == 0 and s["recur_launches"] == 4


@pytest.mark.parametrize("batch", [1, 2, 5, 8, 31, 32, 64, 100, 256])
@pytest.mark.parametrize("slices", [0, 1, 2, 3, 4, 8])
def test_schedule_slices_cover_the_batch(bl, batch, slices):
    """Slices are whole tiles, cover every window once, and the auto choice slices only when
    the recurrence leaves at least half of the CUs idle (streamed gates off: they replace the
    slices when on)."""
    s = bl.schedule(batch, 589, 256, 1, slices=slices, pipeline=1)
    n, w, tile = s["slices"], s["slice_windows"], s["recur_tile"]
    assert 1 <= n <= max(1, slices if slices else 2)
    assert w % tile == 0 or w == batch
    assert (n - 1) * w < batch <= n * w
    if slices == 0:
        idle_half = 4 * s["recur_tiles"] * s["recur_groups"] <= 256
        assert (n > 1) == (idle_half and batch >= 2 * tile)


def test_schedule_slices_need_single_workgroup_tiles(bl):
    for kwargs in (dict(groups=2), dict(concurrent=1)):
        with pytest.raises(bl.BilstmError) as e:
            bl.schedule(32, 589, 256, 1, slices=4, **kwargs)
        assert e.value.name == "BILSTM_UNSUPPORTED"
        assert bl.schedule(32, 589, 256, 1, **kwargs)["slices"] == 1
    assert bl.schedule(32, 589, 256, 1, pipeline=1)["slices"] == 2
    assert bl.schedule(256, 589, 256, 1)["slices"] == 1


def test_schedule_library_projection_runs_unsliced(bl):
    s = bl.schedule(32, 589, 256, 1, projection=1)
    assert s["projection"] == 1 and s["slices"] == 1
    assert bl.schedule(32, 589, 256, 1)["projection"] == 4
    for mode in (2, 3):  # the own split-precision kernels stream like the FP32 one
        s = bl.schedule(32, 589, 256, 1, projection=mode)
        assert s["projection"] == mode and s["slices"] == 1 and s["pipeline"] == 1
        s = bl.schedule(32, 589, 256, 1, projection=mode, pipeline=1)  # unstreamed: sliced
        assert s["projection"] == mode and s["slices"] == 2 and s["pipeline"] == 0
    with pytest.raises(bl.BilstmError) as e:
        bl.schedule(32, 589, 256, 1, projection=1, slices=2)
    assert e.value.name == "BILSTM_UNSUPPORTED"


@pytest.mark.parametrize("batch,steps,chosen", [
    (1, 589, 4),        # 589 rows: below the rows that amortize the split
    (3, 5, 4),
    (8, 589, 4),        # streamed, the FP32 projection keeps up beside the recurrence
    (32, 589, 4),       # the headline workload
    (48, 589, 4),
    (56, 589, 3),       # streamed, more projection work per step than the free CUs do in FP32
    (64, 4096, 3),      # the long workload
    (128, 589, 3),      # unstreamed: the projection runs between the recurrences
    (256, 589, 3),
    (1024, 24, 3)])
def test_projection_rule(bl, batch, steps, chosen):
    """projection = 0: the three-part split where it amortizes and the projection is on the
    forward's critical path, else FP32; never the two-part split or the vendor GEMM."""
    assert bl.schedule(batch, steps, 256, 1)["projection"] == chosen


@pytest.mark.parametrize("batch,steps", [(32, 589), (64, 4096), (256, 589), (128, 64)])
def test_projection_rule_ignores_the_plans_other_options(bl, batch, steps):
    """The rule depends on the workload and the device only: streaming, slices, the recurrence
    split and the direction mode leave its choice alone, so every plan of a workload computes
    the same gates (the bitwise-equality properties across those options hold)."""
    base = bl.schedule(batch, steps, 256, 1)["projection"]
    for kwargs in (dict(pipeline=1), dict(pipeline=1, slices=2), dict(groups=2), dict(groups=4, tile=1),
                   dict(concurrent=0), dict(tile=4)):
        try:
            s = bl.schedule(batch, steps, 256, 4, **kwargs)
        except bl.BilstmError:
            continue
        assert s["projection"] == base, kwargs


@pytest.mark.parametrize("batch,steps,on,chunk", [(1, 589, 1, 128), (2, 589, 1, 64), (3, 589, 1, 32),
                                                   (7, 589, 1, 32), (8, 589, 1, 32), (16, 589, 1, 32),
                                                   (32, 589, 1, 32), (64, 4096, 1, 32), (64, 589, 1, 32),
                                                   (65, 589, 0, 0), (96, 589, 0, 0), (256, 589, 0, 0)])
def test_schedule_streams_gates_when_the_recurrence_leaves_cus(bl, batch, steps, on, chunk):
    """Auto: streamed gates when the recurrence's grid (one workgroup per window and
    direction) leaves at least half of the 256 CUs to the projection; they replace the batch
    slices. With fewer CUs the streamed projection sets the pace (96 windows: 3.5 ms streamed
    against 1.8 unstreamed)."""
    s = bl.schedule(batch, steps, 256, 1)
    assert s["pipeline"] == on and s["stream_chunk"] == chunk
    if on:
        assert s["slices"] == 1 and s["recur_groups"] == 1 and s["concurrent"] == 2
        assert 2 * 2 * s["recur_tiles"] <= 256
        # a chunk's row block of 128 rows holds whole windows, a whole number of recurrence tiles
        assert 128 % chunk == 0 and (128 // chunk) % s["recur_tile"] == 0 and chunk % 4 == 0


def test_schedule_forced_streaming_checks_its_conditions(bl):
    s = bl.schedule(8, 589, 256, 1, pipeline=2, tile=4)
    assert s["pipeline"] == 1 and s["stream_chunk"] == 32 and s["recur_tile"] == 4
    for batch, chunk in ((1, 128), (2, 64), (3, 32)):  # row blocks of 1, 2 and 4 windows
        assert bl.schedule(batch, 589, 256, 1, pipeline=2)["stream_chunk"] == chunk
    s = bl.schedule(120, 589, 256, 1, pipeline=2)  # 240 + 8 <= 256: allowed when asked for
    assert s["pipeline"] == 1
    for kwargs in (dict(groups=2), dict(projection=1), dict(slices=2)):
        with pytest.raises(bl.BilstmError) as e:
            bl.schedule(32, 589, 256, 1, pipeline=2, **kwargs)
        assert e.value.name == "BILSTM_UNSUPPORTED"
        assert bl.schedule(32, 589, 256, 1, **kwargs)["pipeline"] == 0
    with pytest.raises(bl.BilstmError) as e:
        bl.schedule(256, 589, 256, 1, pipeline=2)  # the recurrence takes every CU
    assert e.value.name == "BILSTM_UNSUPPORTED"
    assert bl.schedule(32, 589, 256, 1, pipeline=1)["pipeline"] == 0


@pytest.mark.parametrize("batch,steps,pipeline,overlap", [
    (32, 589, 0, 1), (16, 589, 0, 1), (64, 4096, 0, 1), (64, 589, 0, 1), (96, 589, 2, 1), (32, 589, 3, 0),
    (64, 4096, 4, 1),
    (8, 589, 2, 1), (1, 589, 2, 1), (32, 589, 1, 0), (8, 589, 0, 1), (4, 589, 0, 1), (1, 589, 0, 1),
    (32, 589, 5, 0), (64, 4096, 5, 0)])
def test_schedule_layer_overlap(bl, batch, steps, pipeline, overlap):
    """Streamed gates overlap the next layer's projection with this layer's recurrence unless
    pipeline = 3 asks for each projection after the previous recurrence (or 5, which also runs
    each recurrence after its projection)."""
    s = bl.schedule(batch, steps, 256, 1, pipeline=pipeline)
    assert s["stream_overlap"] == overlap
    assert s["stream_serial"] == (1 if pipeline == 5 else 0)
    assert s["pipeline"] == (1 if pipeline != 1 else 0)


@pytest.mark.parametrize("batch,steps,kwargs,fused", [
    (32, 589, {}, 0), (8, 589, {}, 0), (64, 4096, {}, 0), (32, 589, dict(pipeline=2), 0),
    (32, 589, dict(pipeline=4), 1), (64, 4096, dict(pipeline=4), 1), (32, 589, dict(pipeline=3), 0),
    (32, 589, dict(pipeline=1), 0), (32, 589, dict(pipeline=4, concurrent=1), 0),
    (32, 589, dict(pipeline=4, concurrent=0), 0), (4, 589, {}, 0), (1, 589, dict(pipeline=4), 1)])
def test_schedule_one_launch_recurrence(bl, batch, steps, kwargs, fused):
    """pipeline = 4 runs the four layers' recurrences as one launch when that launch holds both
    directions of every tile; otherwise streamed gates launch each layer's recurrence."""
    s = bl.schedule(batch, steps, 256, 1, **kwargs)
    assert s["stream_fused"] == fused
    assert not fused or (s["pipeline"] == 1 and s["stream_overlap"] == 1 and s["concurrent"] == 2
                         and s["recur_launches"] == 1)


@pytest.mark.parametrize("batch,steps,cus,split", [
    (32, 589, 256, 2), (8, 589, 256, 4), (64, 4096, 256, 1), (1, 589, 256, 4), (16, 589, 256, 4),
    (32, 589, 128, 1), (96, 589, 256, 1), (4, 589, 256, 4), (256, 589, 256, 0)])
def test_schedule_first_chunk_split(bl, batch, steps, cus, split):
    """The first chunk's tiles are as narrow (128 / split columns) as keeps all of them in the
    first round of the streamed projection's workgroups (the CUs the recurrence leaves)."""
    s = bl.schedule(batch, steps, cus, 1, pipeline=2 if split else 0)
    assert s["stream_split"] == split
    if split:
        groups = -(-batch // (128 // s["stream_chunk"]))
        free = max(8, (cus - 2 * s["recur_tiles"] * s["recur_groups"]) // 8 * 8)
        assert 2 * groups * 4 * split <= free or split == 1
        assert split == 4 or 2 * groups * 4 * split * 2 > free


@pytest.mark.parametrize("kwargs,status", [
    (dict(groups=3), "BILSTM_UNSUPPORTED"), (dict(tile=3), "BILSTM_UNSUPPORTED"),
    (dict(concurrent=5), "BILSTM_INVALID_ARGUMENT"), (dict(slices=9), "BILSTM_INVALID_ARGUMENT"),
    (dict(slices=-1), "BILSTM_INVALID_ARGUMENT"), (dict(projection=5), "BILSTM_INVALID_ARGUMENT"),
    (dict(projection=-1), "BILSTM_INVALID_ARGUMENT"), (dict(pipeline=6), "BILSTM_INVALID_ARGUMENT"),
    (dict(pipeline=-1), "BILSTM_INVALID_ARGUMENT")])
def test_schedule_rejects_bad_options(bl, kwargs, status):
    with pytest.raises(bl.BilstmError) as e:
        bl.schedule(8, 589, 256, 1, **kwargs)
    assert e.value.name == status


def test_plan_create_argument_checks_without_gpu(bl):
    lib = bl.library()
    layers = workloads.make_layers(23)
    keep = []
    arr = (bl.Layer * 4)(*[bl._layer_struct(l, keep) for l in layers])
    h = ctypes.c_void_p()
    assert lib.bilstm_plan_create(0, 0, 589, arr, ctypes.byref(h)) == 1  # batch 0
    assert "batch" in bl.last_error()
    assert lib.bilstm_plan_create(0, 1, 589, None, ctypes.byref(h)) == 1
    # wrong R length on layer 2
    arr[2].r_len = arr[2].r_len - 1
    assert lib.bilstm_plan_create(0, 1, 589, arr, ctypes.byref(h)) == 2
    assert "layer 2 R" in bl.last_error()
    arr[2].r_len = arr[2].r_len + 1
    # more rows than 32-bit indexing allows: batch·steps·1024 must stay below 2^32, so 1024
    # windows of 4096 steps are one row too many and 1023 windows pass the size checks
    assert lib.bilstm_plan_create(0, 1 << 16, 1 << 10, arr, ctypes.byref(h)) == 3
    assert lib.bilstm_plan_create(0, 1024, 4096, arr, ctypes.byref(h)) == 3
    if not _have_gpu():
        assert lib.bilstm_plan_create(0, 1023, 4096, arr, ctypes.byref(h)) == 4
    # with valid arguments and no GPU here, the device check answers
    st = lib.bilstm_plan_create(0, 1, 589, arr, ctypes.byref(h))
    if not _have_gpu():
        assert st == 4 and h.value is None


def test_entry_points_reject_null_plan(bl):
    lib = bl.library()
    assert lib.bilstm_forward(None, None, 0, None, 0, None) == 1
    assert lib.bilstm_check(None) == 1
    lib.bilstm_destroy(None)  # NULL-safe


def test_probes_check_arguments_before_the_device(bl):
    """The measurement probes reject bad arguments with BILSTM_INVALID_ARGUMENT (1) before any
    device call, so these checks run without a GPU."""
    lib = bl.library()
    a, b = ctypes.c_double(), ctypes.c_double()
    assert lib.bilstm_probe_mfma_rate(0, 2, 0, 10, ctypes.byref(a), ctypes.byref(b)) == 1   # kind
    assert lib.bilstm_probe_mfma_rate(0, 0, 3, 10, ctypes.byref(a), ctypes.byref(b)) == 1   # data
    assert lib.bilstm_probe_mfma_rate(0, 0, 0, 0, ctypes.byref(a), ctypes.byref(b)) == 1    # iterations
    assert lib.bilstm_probe_mfma_rate(0, 0, 0, 10, None, ctypes.byref(b)) == 1              # NULL output
    assert lib.bilstm_probe_fma_rate(0, 3, 1, 10, ctypes.byref(a), ctypes.byref(b)) == 1    # waves per SIMD
    assert lib.bilstm_probe_fma_rate(0, 2, 0, 10, ctypes.byref(a), ctypes.byref(b)) == 1    # workgroups


def _have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_heads_create_argument_checks_without_gpu(bl):
    """Length and NULL checks of the heads' constructor come before any device call."""
    lib = bl.library()
    head = workloads.make_heads(3)
    keep = [np.ascontiguousarray(head[k], np.float32) for k in ("w0", "b0", "w1", "b1", "w2", "b2")]
    fields = []
    for a in keep:
        fields += [a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), a.size]
    fields[1] -= 1  # W0 one element short
    hw = bl.HeadWeights(*fields, ctypes.c_float(0.01))
    h = ctypes.c_void_p()
    assert lib.bilstm_heads_create(0, ctypes.byref(hw), ctypes.byref(h)) == 2
    assert "heads_create W0" in bl.last_error() and not h.value
    assert lib.bilstm_heads_create(0, None, ctypes.byref(h)) == 1
    assert lib.bilstm_heads_forward(None, None, 0, None, 0, None) == 1
    lib.bilstm_heads_destroy(None)


def _float32_lstm(bias: bool, seed: int):
    """nn.LSTM(60, 128, 4, bidirectional) in float64 whose parameters hold float32 values, so
    the converter's float32 copy and the module see the same numbers."""
    torch = pytest.importorskip("torch")
    torch.manual_seed(seed)
    net = torch.nn.LSTM(60, 128, num_layers=4, bidirectional=True, batch_first=True, bias=bias,
                        dtype=torch.float64)
    with torch.no_grad():
        for p in net.parameters():
            p.copy_(p.to(torch.float32).to(torch.float64))
    return net


@pytest.mark.parametrize("bias", [True, False])
def test_layers_from_state_dict_match_the_torch_module(oracle_lib, bias):
    # the oracle on converted parameters reproduces the module itself (directions, gate rows
    # i, f, g, o, bias_ih as Wb and bias_hh as Rb, zero biases for bias=False)
    torch = pytest.importorskip("torch")
    import bidirectional_lstm_sequence_amd as bl
    net = _float32_lstm(bias, seed=11)
    layers = bl.layers_from_state_dict(net.state_dict())
    assert [l["w"].shape for l in layers] == [(2, 512, 60)] + [(2, 512, 256)] * 3
    assert all(l["r"].shape == (2, 512, 128) and l["b"].shape == (2, 2, 512) for l in layers)
    assert all(l["w"].dtype == np.float32 for l in layers)
    if not bias:
        assert all(not l["b"].any() for l in layers)
    x = np.random.default_rng(4).standard_normal((2, 9, 60)).astype(np.float32)
    with torch.no_grad():
        ref, _ = net(torch.from_numpy(x.astype(np.float64)))
    got = oracle_lib.stack(x, layers)
    assert np.abs(got - ref.numpy()).max() < 1e-12


def test_layers_from_state_dict_rejects_other_shapes():
    torch = pytest.importorskip("torch")
    import bidirectional_lstm_sequence_amd as bl
    net = torch.nn.LSTM(61, 128, num_layers=4, bidirectional=True, batch_first=True)
    with pytest.raises(ValueError, match="layer 0"):
        bl.layers_from_state_dict(net.state_dict())
    net = torch.nn.LSTM(60, 128, num_layers=3, bidirectional=True, batch_first=True)
    with pytest.raises(KeyError):
        bl.layers_from_state_dict(net.state_dict())
