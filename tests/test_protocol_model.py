"""CPU model of the publication protocols between concurrently running workgroups (no GPU).

The model (bidirectional_lstm_sequence_amd/csrc/protocol_model.cpp) runs the functions of
protocol.h that the kernels and the plan use — the h exchange's flags, parities and flag-range
reservation with its clear, the chunk counters' targets, signed comparison and clear rule, the
progress words — on std::thread producers and consumers with random delays, and counts every
accepted value that was not its producer's. Covered (the speakrs 0.6.0 page `lstmproj.rs`:
`Exchange` doc, `DirectionLaunch` doc, `clear_state`):
  * flag = layer·T + s + 1 over several layers and passes, with stale words planted before the
    run and left by earlier steps, layers and passes;
  * the flag range reaching 2^32 - 1, the clear and the restart at 0;
  * counters over several passes, starting just below their clear threshold;
  * progress words whose stale values from the previous pass show every step done;
  * a producer that never publishes: its consumers end at the watchdog and every thread ends.
Planted mistakes in copies of protocol.h (no +1 on the flag, no step parity, a target one pass
low, progress compared without its pass number) must each make the model fail.
"""

import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from bidirectional_lstm_sequence_amd import _build


class Result(ctypes.Structure):
    _fields_ = [("accepted", ctypes.c_uint64), ("wrong_values", ctypes.c_uint64), ("timeouts", ctypes.c_uint64),
                ("clears", ctypes.c_uint64), ("passes", ctypes.c_uint64)]


@pytest.fixture(scope="module")
def model():
    if not os.path.exists(_build.MODEL_LIB):
        _build.build_protocol_model()
    lib = ctypes.CDLL(_build.MODEL_LIB)
    i, u32 = ctypes.c_int, ctypes.c_uint32
    R = ctypes.POINTER(Result)
    lib.bilstm_model_exchange.argtypes = [i, i, i, i, i, i, u32, i, i, i, u32, i, u32, R]
    lib.bilstm_model_counters.argtypes = [i, i, i, i, i, u32, i, u32, i, u32, R]
    lib.bilstm_model_progress.argtypes = [i, i, i, i, u32, i, i, u32, R]
    D = ctypes.c_double
    lib.bilstm_model_stream_walk.argtypes = [i, ctypes.POINTER(i), i, i, u32, D, D, D, ctypes.POINTER(i),
                                             ctypes.POINTER(D), ctypes.POINTER(D)]
    for f in (lib.bilstm_model_exchange, lib.bilstm_model_counters, lib.bilstm_model_progress,
              lib.bilstm_model_stream_walk):
        f.restype = ctypes.c_int
    return lib


def run(fn, *args):
    r = Result()
    assert fn(*args, ctypes.byref(r)) == 0
    return r


@pytest.mark.parametrize("groups,tile,seed", [(2, 1, 1), (4, 1, 2), (4, 2, 3), (2, 4, 4)])
def test_exchange_accepts_only_the_producers_words(model, groups, tile, seed):
    # 4 layers x 3 passes of 40 steps; planted stale words with flags below the first pass's
    r = run(model.bilstm_model_exchange, groups, 32, tile, 40, 4, 3, 10_000, 1, -1, 0, 0, 5000, seed)
    others = 32 - 32 // groups
    assert r.wrong_values == 0 and r.timeouts == 0
    assert r.accepted == groups * others * tile * 40 * 4 * 3  # every word of every step, exactly once
    assert r.clears == 0


def test_exchange_across_the_flag_wrap(model):
    # the epoch starts 300 flags below 2^32: the first pass fits, the second clears and restarts
    r = run(model.bilstm_model_exchange, 4, 32, 1, 30, 4, 3, 0xFFFFFFFF - 300, 1, -1, 0, 0, 5000, 11)
    assert r.clears == 1 and r.wrong_values == 0 and r.timeouts == 0
    assert r.accepted == 4 * 24 * 30 * 4 * 3


def test_exchange_silent_member_ends_at_the_watchdog(model):
    # member 1 publishes nothing from step 5 of the first layer on: the others time out once
    # each and stop waiting (running ahead, they may then overwrite words member 1 still waits
    # for, so it may time out too); every thread of every later layer and pass still finishes,
    # and no wrong value is ever accepted
    r = run(model.bilstm_model_exchange, 4, 32, 1, 20, 2, 2, 0, 0, 1, 5, 0, 50, 12)
    assert r.wrong_values == 0
    assert 3 <= r.timeouts <= 4
    assert r.passes == 2


def test_exchange_forced_timeout_skew(model):
    # every wait expects a flag no producer writes: each member gives up once, accepts nothing
    r = run(model.bilstm_model_exchange, 2, 16, 1, 10, 1, 1, 0, 0, -1, 0, 0x80000000, 20, 13)
    assert r.timeouts == 2 and r.accepted == 0


@pytest.mark.parametrize("groups,chunks,split,workers,seed", [(1, 5, 4, 2, 21), (3, 7, 2, 5, 22), (4, 3, 1, 8, 23)])
def test_counters_publish_whole_chunks(model, groups, chunks, split, workers, seed):
    r = run(model.bilstm_model_counters, groups, chunks, split, workers, 5, 0, -1, 0, 5000, seed)
    assert r.wrong_values == 0 and r.timeouts == 0
    assert r.accepted == 5 * 2 * groups * chunks


def test_counters_across_their_clear(model):
    # counters and pass counts start one pass below the clear threshold, with the counters
    # holding what that many passes left: pass 1 and 2 run above it, pass 3 clears
    limit = 0x03FFFFFF
    r = run(model.bilstm_model_counters, 2, 4, 2, 4, 4, limit - 1, -1, 0, 5000, 24)
    assert r.clears == 1 and r.wrong_values == 0 and r.timeouts == 0
    assert r.accepted == 4 * 2 * 2 * 4


def test_counters_missing_tile_ends_at_the_watchdog(model):
    r = run(model.bilstm_model_counters, 2, 4, 1, 3, 2, 0, 9, 0, 50, 25)
    assert r.wrong_values == 0 and r.timeouts == 1 and r.passes == 2


@pytest.mark.parametrize("windows,steps,chunk,every,seed", [(4, 120, 32, 8, 31), (2, 589, 128, 16, 32),
                                                            (5, 37, 8, 4, 33)])
def test_progress_words_ignore_the_previous_pass(model, windows, steps, chunk, every, seed):
    r = run(model.bilstm_model_progress, windows, steps, chunk, every, 9, -1, 5000, seed)
    assert r.wrong_values == 0 and r.timeouts == 0
    assert r.accepted == windows * 2 * ((steps + chunk - 1) // chunk)


def test_progress_missing_window_ends_at_the_watchdog(model):
    r = run(model.bilstm_model_progress, 3, 64, 16, 4, 2, 1, 50, 34)
    assert r.wrong_values == 0 and r.timeouts == 1


# ---- the tile walk of a streamed projection workgroup --------------------------------------

def walk(model, chunks, steps, chunk, lead0, rate, start, tile_time):
    n = len(chunks)
    order, begin, end = (ctypes.c_int * n)(), (ctypes.c_double * n)(), (ctypes.c_double * n)()
    taken = model.bilstm_model_stream_walk(n, (ctypes.c_int * n)(*chunks), steps, chunk, lead0, rate, start,
                                           tile_time, order, begin, end)
    assert taken == n, f"{taken} of {n} tiles taken"
    return list(order), list(begin), list(end)


def need(steps, chunk, c):
    return max(min(c * chunk + chunk, steps), steps - c * chunk)


def test_walk_off_is_consumption_order(model):
    order, _, _ = walk(model, [0, 0, 1, 3, 3, 7], 256, 32, 0, 1.0, 0.0, 5.0)
    assert order == list(range(6))


@pytest.mark.parametrize("seed", range(8))
def test_walk_takes_every_tile_once(model, seed):
    # the walk goes down from the last tile of least need while the previous layer runs, then
    # the rest in consumption order: every tile once, in that shape
    rng = np.random.default_rng(seed)
    for _ in range(40):
        chunk = int(rng.choice([8, 16, 32, 64]))
        steps = int(rng.integers(1, 5000))
        n = int(rng.integers(1, 300))
        chunks = sorted(int(c) for c in rng.integers(0, (steps + chunk - 1) // chunk, n))
        rate = float(rng.uniform(0.5, 5.0))
        order, _, _ = walk(model, chunks, steps, chunk, int(rng.integers(1, 200)), rate,
                           float(rng.uniform(0, steps / rate)), float(rng.uniform(0.5, 100)))
        assert sorted(order) == list(range(n))
        least = min(need(steps, chunk, c) for c in chunks)
        mid = max(k for k in range(n) if need(steps, chunk, chunks[k]) == least)
        if order[0] != 0 or mid == 0:
            # it walked: mid, mid - 1, ..., lo, then 0 .. lo - 1, then mid + 1 .. n - 1
            assert order[0] == mid
            i = 0
            while i < n and order[i] == mid - i:
                i += 1
            lo = mid - i + 1
            assert order == list(range(mid, lo - 1, -1)) + list(range(lo)) + list(range(mid + 1, n))
        else:
            assert order == list(range(n))


@pytest.mark.parametrize("start", [900.0, 1500.0, 1780.0])
def test_walk_keeps_chunk_zero_on_time(model, start):
    # 4096 steps in 32-step chunks, one tile per chunk, the previous layer 1810 time units, a
    # tile 17.6: chunk 0 ends when it would in consumption order, and the next layer, reading
    # chunk c once it has ended, finishes earlier the earlier the workgroup starts
    chunks = list(range(128))
    rate = 4096 / 1810

    def next_layer_end(end):
        t = 1810.0
        for e in end:
            t = max(t, e) + 1810 / 128
        return t

    _, _, plain = walk(model, chunks, 4096, 32, 0, rate, start, 17.6)
    order, _, walked = walk(model, chunks, 4096, 32, 64, rate, start, 17.6)
    assert order[0] == 64
    assert walked[0] <= plain[0] == pytest.approx(1810 + 17.6)
    gain = 1 - next_layer_end(walked) / next_layer_end(plain)
    assert gain > {900.0: 0.08, 1500.0: 0.05, 1780.0: 0.0}[start] - 1e-12
    assert max(walked) <= max(plain)


# ---- planted mistakes: a copy of protocol.h with one rule broken must fail the model ------

MUTANTS = {
    "flag without +1 (zeroed words match step 0)":
        (r"return flag_base \+ static_cast<uint32_t>\(step\) \+ 1u;", "return flag_base + static_cast<uint32_t>(step);"),
    "no step parity (one buffer for every step)":
        (r"return \(\(step & 1\) \* hidden \+ unit\) \* tile \+ b;", "return (0 * hidden + unit) * tile + b;"),
    "counter target one pass low":
        (r"return passes \* static_cast<uint32_t>\(kReadyPerPass\) \+ skew;",
         "return (passes - 1) * static_cast<uint32_t>(kReadyPerPass) + skew;"),
    "progress compared without its pass number":
        (r"return seen >= \(pass_bits \| need\);", "return static_cast<uint32_t>(seen) >= need;"),
    "walk resumes one tile past the walked range":
        (r"if \(w\.next_in_order == w\.lo\) w\.next_in_order = w\.hi;",
         "if (w.next_in_order == w.lo) w.next_in_order = w.hi + 1;"),
    "walk ignores the previous layer's end":
        (r"if \(w\.lo > 0 && static_cast<uint64_t>\(progress\)", "if (w.lo > 0 && true || static_cast<uint64_t>(progress)"),
    "walk starts at the first tile of least need":
        (r"chunk_of\(a - 1\)\) < chunk_need", "chunk_of(a - 1)) <= chunk_need"),
    "walk's lead ignores when the rows were complete":
        (r"const uint32_t from = before > ready_at \? before : ready_at;", "const uint32_t from = before;"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_protocol_mistakes_fail_the_model(tmp_path, name):
    pattern, replacement = MUTANTS[name]
    for f in ("protocol_model.cpp", "protocol.h"):
        shutil.copy(os.path.join(_build.CSRC, f), tmp_path / f)
    header = (tmp_path / "protocol.h").read_text()
    mutated, n = re.subn(pattern, replacement, header)
    assert n == 1, f"mutation {name!r} did not apply"
    (tmp_path / "protocol.h").write_text(mutated)
    exe = _build.build_protocol_model(str(tmp_path / "model_main"), str(tmp_path), main=True)
    res = subprocess.run([exe, "100"], capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"the model did not catch: {name}\n{res.stdout}"


def test_unmutated_model_driver_passes(tmp_path):
    exe = _build.build_protocol_model(str(tmp_path / "model_main"), main=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
