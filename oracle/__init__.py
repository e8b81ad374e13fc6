"""Oracle of the four-layer bidirectional LSTM stack (ctypes wrapper of bilstm_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg use it. The HIP library and its Python binding never import it.

All functions take one window at a time (windows are independent); ``stack`` spreads the
windows of a batch over a thread pool, each thread running the unchanged single-threaded
routine (ctypes releases the GIL during the call).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SOURCES = [os.path.join(_HERE, "bilstm_oracle.c"), os.path.join(_HERE, "lstm_body.inc")]

_libs: dict = {}


def compile_library(source: str, out_path: str) -> str:
    """Compile ``source`` (bilstm_oracle.c or a copy of it) with gcc into ``out_path``."""
    tmp = out_path + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp,
           source, "-lm"]
    subprocess.run(cmd, check=True, cwd=os.path.dirname(os.path.abspath(source)))
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    return compile_library(_SOURCES[0], LIB_PATH)


def build_check(out_path: str) -> str:
    """The oracle with AddressSanitizer and UndefinedBehaviorSanitizer, linked with its
    stand-alone driver (check_main.c), which runs every routine on small shapes."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-o", out_path, os.path.join(_HERE, "check_main.c"), _SOURCES[0], "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    return out_path


def use_library(path: str | None) -> None:
    """Route the functions below to another build of the oracle (None: the default one).

    Only the oracle's own tests use this, to check that deliberately broken copies of the
    oracle fail its pins.
    """
    global _active
    _active = path or LIB_PATH


_active = LIB_PATH


def _load():
    path = _active
    if path in _libs:
        return _libs[path]
    if path == LIB_PATH and not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(path)
    fp = ctypes.POINTER(ctypes.c_float)
    for suffix, real in (("f64", ctypes.c_double), ("f32", ctypes.c_float)):
        rp = ctypes.POINTER(real)
        f = getattr(lib, f"oracle_projection_{suffix}")
        f.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, fp, rp, fp, fp, rp]
        f.restype = ctypes.c_int
        f = getattr(lib, f"oracle_recurrence_{suffix}")
        f.argtypes = [ctypes.c_int, ctypes.c_int, rp, fp, rp]
        f.restype = ctypes.c_int
        f = getattr(lib, f"oracle_stack_window_{suffix}")
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, fp, fp, fp, fp,
                      rp, rp]
        f.restype = ctypes.c_int
        f = getattr(lib, f"oracle_heads_{suffix}")
        f.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_double, fp, rp, fp, fp, fp, fp, fp, fp, rp]
        f.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _real(precision: str):
    if precision == "f64":
        return np.float64, ctypes.c_double
    if precision == "f32":
        return np.float32, ctypes.c_float
    raise ValueError(f"precision must be 'f64' or 'f32', not {precision!r}")


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _flat_layers(layers):
    w_all = np.concatenate([_f32(l["w"]).ravel() for l in layers])
    r_all = np.concatenate([_f32(l["r"]).ravel() for l in layers])
    b_all = np.concatenate([_f32(l["b"]).ravel() for l in layers])
    return w_all, r_all, b_all


def projection(x: np.ndarray, w: np.ndarray, b: np.ndarray, precision: str = "f64") -> np.ndarray:
    """Gate pre-activations ``[rows, 2, 4H]`` of ``x [rows, in]`` (float32 input)."""
    lib = _load()
    dt, ct = _real(precision)
    x = _f32(x)
    w = _f32(w)
    b = _f32(b)
    rows, width = x.shape
    gates = w.shape[1]
    out = np.empty((rows, 2, gates), dtype=dt)
    fn = getattr(lib, f"oracle_projection_{precision}")
    rc = fn(rows, width, gates // 4, _ptr(x, ctypes.c_float), None, _ptr(w, ctypes.c_float),
            _ptr(b, ctypes.c_float), _ptr(out, ct))
    if rc != 0:
        raise RuntimeError(f"oracle_projection failed ({rc})")
    return out


def recurrence(gates: np.ndarray, r: np.ndarray, precision: str = "f64") -> np.ndarray:
    """Both directions' recurrence of one window: ``gates [T, 2, 4H]`` -> ``y [T, 2H]``."""
    lib = _load()
    dt, ct = _real(precision)
    g = np.ascontiguousarray(gates, dtype=dt)
    r = _f32(r)
    steps = g.shape[0]
    hidden = r.shape[2]
    y = np.empty((steps, 2 * hidden), dtype=dt)
    fn = getattr(lib, f"oracle_recurrence_{precision}")
    rc = fn(steps, hidden, _ptr(g, ct), _ptr(r, ctypes.c_float), _ptr(y, ct))
    if rc != 0:
        raise RuntimeError(f"oracle_recurrence failed ({rc})")
    return y


def stack_window(x: np.ndarray, layers, precision: str = "f64", dump_gates: bool = False,
                 _flat=None):
    """The whole stack over one window ``x [T, in0]``; returns ``y [T, 2H]``.

    With ``dump_gates`` also returns each layer's projection output ``[L, T, 2, 4H]``.
    """
    lib = _load()
    dt, ct = _real(precision)
    x = _f32(x)
    steps, in0 = x.shape
    hidden = layers[0]["r"].shape[2]
    nl = len(layers)
    w_all, r_all, b_all = _flat if _flat is not None else _flat_layers(layers)
    y = np.empty((steps, 2 * hidden), dtype=dt)
    dump = np.empty((nl, steps, 2, 4 * hidden), dtype=dt) if dump_gates else None
    fn = getattr(lib, f"oracle_stack_window_{precision}")
    rc = fn(steps, in0, hidden, nl, _ptr(x, ctypes.c_float), _ptr(w_all, ctypes.c_float),
            _ptr(r_all, ctypes.c_float), _ptr(b_all, ctypes.c_float), _ptr(y, ct),
            _ptr(dump, ct) if dump is not None else None)
    if rc != 0:
        raise RuntimeError(f"oracle_stack_window failed ({rc})")
    return (y, dump) if dump_gates else y


def stack(x: np.ndarray, layers, precision: str = "f64", threads: int = 1,
          windows=None) -> np.ndarray:
    """The stack over a batch ``x [B, T, in0]`` -> ``y [len(windows), T, 2H]``.

    ``windows`` selects a subset of window indices (default: all). Windows are dispatched
    over ``threads`` worker threads, each running the single-threaded routine.
    """
    x = _f32(x)
    idx = list(range(x.shape[0])) if windows is None else list(windows)
    flat = _flat_layers(layers)
    if threads <= 1 or len(idx) <= 1:
        outs = [stack_window(x[b], layers, precision, _flat=flat) for b in idx]
    else:
        with ThreadPoolExecutor(max_workers=threads) as pool:
            outs = list(pool.map(lambda b: stack_window(x[b], layers, precision, _flat=flat), idx))
    return np.stack(outs) if outs else np.empty((0,) + (x.shape[1], 2 * layers[0]["r"].shape[2]))


def heads(y: np.ndarray, head: dict, precision: str = "f64") -> np.ndarray:
    """The segmentation heads over ``y [rows, in]`` -> log-probabilities ``[rows, classes]``.

    ``head`` holds float32 ``w0 [in, mid0]``, ``b0 [mid0]``, ``w1 [mid0, mid1]``, ``b1``,
    ``w2 [mid1, classes]``, ``b2`` (row-major [k][n]) and ``slope`` (LeakyReLU). ``y`` may be
    float32 (the library's output) or float64 (the oracle's own stack output).
    """
    lib = _load()
    dt, ct = _real(precision)
    w0, b0, w1, b1, w2, b2 = (_f32(head[k]) for k in ("w0", "b0", "w1", "b1", "w2", "b2"))
    rows, width = y.shape
    mid0, mid1, classes = w0.shape[1], w1.shape[1], w2.shape[1]
    if w0.shape[0] != width or w1.shape[0] != mid0 or w2.shape[0] != mid1:
        raise ValueError("head weight shapes do not chain")
    out = np.empty((rows, classes), dtype=dt)
    fn = getattr(lib, f"oracle_heads_{precision}")
    if y.dtype == np.float32:
        yf, yr = _f32(y), None
    else:
        yf, yr = None, np.ascontiguousarray(y, dtype=dt)
    rc = fn(rows, width, mid0, mid1, classes, float(head["slope"]),
            _ptr(yf, ctypes.c_float) if yf is not None else None,
            _ptr(yr, ct) if yr is not None else None,
            *(_ptr(a, ctypes.c_float) for a in (w0, b0, w1, b1, w2, b2)), _ptr(out, ct))
    if rc != 0:
        raise RuntimeError(f"oracle_heads failed ({rc})")
    return out
