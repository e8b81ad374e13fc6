"""GPU parity of the fused segmentation heads (linear0, linear1, classifier after the stack)
against the oracle, element by element on seeded inputs.

Tolerance (allclose form, as for the stack): |gpu - oracle| <= 2e-5 + 1e-4·|oracle|.
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
    bl.library()
    return bl


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def assert_close(got, ref, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside tolerance, max abs err {err.max():.3e}"
    return float(err.max())


@pytest.mark.parametrize("rows", [1, 63, 64, 65, 1000, 4712])
def test_heads_match_oracle(bl, orc, rows):
    """Ragged row counts around the 64-row tile; inputs in [-1, 1] like the stack's output."""
    head = workloads.make_heads(40 + rows)
    y = np.random.default_rng(rows).uniform(-1, 1, size=(rows, 256)).astype(np.float32)
    y[0, :7] = [1.0, -1.0, 0.0, 1.0, -1.0, 1.0, -1.0]
    note(f"heads rows={rows}")
    h = bl.Heads(head)
    out = h.forward(torch.from_numpy(y).cuda()).cpu().numpy()
    h.close()
    ref = orc.heads(y, head)
    err = assert_close(out, ref, f"heads rows={rows}")
    np.testing.assert_allclose(np.exp(out.astype(np.float64)).sum(axis=1), 1.0, rtol=0, atol=1e-5)
    note(f"heads rows={rows} max abs err {err:.3e}")


def test_heads_at_the_long_workload_size(bl, orc):
    """262,144 rows (the 64 x 4096 stack output): sampled rows (both ends and a random set)
    against the oracle, and two runs bitwise equal."""
    rows = 64 * 4096
    head = workloads.make_heads(4096)
    y = np.random.default_rng(4096).uniform(-1, 1, size=(rows, 256)).astype(np.float32)
    note(f"heads rows={rows}")
    h = bl.Heads(head)
    yd = torch.from_numpy(y).cuda()
    out = h.forward(yd).cpu().numpy()
    again = h.forward(yd).cpu().numpy()
    h.close()
    assert np.array_equal(out.view(np.uint32), again.view(np.uint32))
    pick = np.unique(np.concatenate([np.arange(256), np.arange(rows - 256, rows),
                                     np.random.default_rng(7).choice(rows, 2048, replace=False)]))
    ref = orc.heads(np.ascontiguousarray(y[pick]), head)
    err = assert_close(out[pick], ref, f"heads rows={rows} (sampled)")
    note(f"heads rows={rows} sampled {len(pick)} max abs err {err:.3e}")


def test_heads_zero_rows_and_position_invariance(bl):
    """No rows is a no-op; a row's outputs do not depend on where in the batch it sits."""
    head = workloads.make_heads(9)
    y = np.random.default_rng(9).uniform(-1, 1, size=(300, 256)).astype(np.float32)
    h = bl.Heads(head)
    empty = h.forward(torch.zeros((0, 256), device="cuda"))
    assert empty.shape == (0, 7)
    full = h.forward(torch.from_numpy(y).cuda()).cpu().numpy()
    tail = h.forward(torch.from_numpy(np.ascontiguousarray(y[37:])).cuda()).cpu().numpy()
    torch.cuda.synchronize()
    h.close()
    assert np.array_equal(full[37:].view(np.uint32), tail.view(np.uint32))


@pytest.mark.parametrize("name", ["b1", "b8"])
def test_stack_then_heads_match_oracle(bl, orc, name):
    """The stack and the heads on the GPU against the oracle's fp64 stack and heads."""
    x, layers = workloads.make_workload(name)
    head = workloads.make_heads(workloads.WORKLOADS[name].seed)
    note(f"stack+heads {name}")
    plan = bl.Plan(layers, x.shape[0], x.shape[1])
    heads = bl.Heads(head)
    y = plan.forward(torch.from_numpy(x).cuda())
    out = heads.forward(y).cpu().numpy()
    plan.check()
    plan.close()
    heads.close()
    ref_y = orc.stack(x, layers, threads=min(16, os.cpu_count() or 1))
    ref = orc.heads(ref_y.reshape(-1, 256), head).reshape(x.shape[0], x.shape[1], 7)
    err = assert_close(out, ref, f"stack+heads {name}")
    note(f"stack+heads {name} max abs err {err:.3e}")


def test_heads_reject_bad_buffers(bl):
    head = workloads.make_heads(10)
    h = bl.Heads(head)
    with pytest.raises(ValueError):
        h.forward(torch.zeros((4, 255), device="cuda"))
    lib = bl.library()
    import ctypes
    y = torch.zeros((4, 256), device="cuda")
    o = torch.zeros((4, 7), device="cuda")
    st = lib.bilstm_heads_forward(h._h, ctypes.c_void_p(y.data_ptr()), 4 * 256, ctypes.c_void_p(o.data_ptr()),
                                  4 * 7 - 1, None)
    assert st == 2 and "heads_forward output" in bl.last_error()
    st = lib.bilstm_heads_forward(h._h, ctypes.c_void_p(y.data_ptr()), 4 * 256 + 1, ctypes.c_void_p(o.data_ptr()),
                                  4 * 7, None)
    assert st == 2
    h.close()
