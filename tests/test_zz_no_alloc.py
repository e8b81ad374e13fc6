"""GPU: bilstm_forward_noalloc, the stack without a plan and without allocation, against a
plan's bilstm_forward on the same inputs (bitwise: the same kernels and packed bits) and
against the oracle (the output tolerance), on two calls in a row, the second smaller, which
reuse the one static scratch array of the device."""

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


def test_forward_noalloc_matches_plan_forward_twice(bl):
    import oracle
    oracle.build(force=False)
    layers = workloads.make_layers(501)
    dev_layers = bl.device_layers(layers)
    cases = [(8, 589), (3, 100)]  # the second call smaller than the first
    inputs = [workloads.make_input(502 + i, b, t) for i, (b, t) in enumerate(cases)]
    xs = [torch.from_numpy(x).cuda() for x in inputs]
    ys = [torch.full((b, t, 256), float("nan"), dtype=torch.float32, device="cuda") for b, t in cases]
    torch.cuda.synchronize()
    for (b, t), xd, y in zip(cases, xs, ys):
        note(f"forward_noalloc batch={b} steps={t}")
        bl.forward_noalloc(dev_layers, xd, y)
    torch.cuda.synchronize()
    for (b, t), x, xd, y in zip(cases, inputs, xs, ys):
        got = y.cpu().numpy()
        with bl.Plan(layers, b, t) as plan:
            ref_plan = plan.forward(xd).cpu().numpy()
            plan.check()
        assert np.array_equal(got.view(np.uint32), ref_plan.view(np.uint32)), f"b{b} t{t}: differs from the plan"
        ref = oracle.stack(x, layers, threads=min(16, os.cpu_count() or 1))
        err = np.abs(got.astype(np.float64) - ref)
        assert np.all(err <= ATOL + RTOL * np.abs(ref)), f"b{b} t{t}: max abs err {err.max():.3e}"
        note(f"forward_noalloc batch={b} steps={t}: bitwise equal to the plan, max abs err {err.max():.3e}")


def test_forward_noalloc_rejects_sizes_beyond_its_scratch(bl):
    layers = bl.device_layers(workloads.make_layers(503))
    b, t = 40, 589  # 23,560 rows: more than the static scratch holds
    x = torch.zeros((b, t, 60), dtype=torch.float32, device="cuda")
    y = torch.zeros((b, t, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(bl.BilstmError) as e:
        bl.forward_noalloc(layers, x, y)
    assert e.value.name == "BILSTM_DIMENSION_OVERFLOW" and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool(torch.all(y == 0)), "a rejected call wrote its output"


def test_forward_noalloc_at_its_largest_size(bl):
    """One window of 23,227 steps: exactly the rows the static scratch holds, bitwise equal to
    a plan's forward."""
    layers = workloads.make_layers(504)
    b, t = 1, 23227
    x = torch.from_numpy(workloads.make_input(505, b, t)).cuda()
    y = torch.full((b, t, 256), float("nan"), dtype=torch.float32, device="cuda")
    note(f"forward_noalloc batch={b} steps={t} (the scratch's limit)")
    bl.forward_noalloc(bl.device_layers(layers), x, y)
    torch.cuda.synchronize()
    with bl.Plan(layers, b, t) as plan:
        ref = plan.forward(x)
        plan.check()
    assert torch.equal(y.view(torch.int32), ref.view(torch.int32))
