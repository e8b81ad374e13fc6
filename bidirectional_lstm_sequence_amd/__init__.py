"""Python binding of the MI355X bidirectional LSTM stack library (libbilstm_amd.so).

Argument marshalling only: every step of the stack runs in the library's HIP kernels.
PyTorch is used for device memory and streams. The functions mirror include/bilstm.h.

If the library has not been built, importing this package still works (so the host-side
tests can report it), but every call raises ``LibraryMissing``: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

HIDDEN = 128
GATES = 512
FEATURES = 60
WIDTH = 256
LAYERS = 4

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbilstm_amd.so")

STATUS = {0: "BILSTM_OK", 1: "BILSTM_INVALID_ARGUMENT", 2: "BILSTM_BUFFER_LENGTH",
          3: "BILSTM_DIMENSION_OVERFLOW", 4: "BILSTM_UNSUPPORTED", 5: "BILSTM_HIP_ERROR",
          6: "BILSTM_TIMEOUT"}

# every symbol include/bilstm.h declares
EXPORTS = ["bilstm_plan_create", "bilstm_plan_create_ex", "bilstm_forward", "bilstm_project",
           "bilstm_recur", "bilstm_plan_get_info", "bilstm_check", "bilstm_set_phase_events",
           "bilstm_phase_times", "bilstm_destroy", "bilstm_last_error", "bilstm_pack_layer",
           "bilstm_schedule", "bilstm_probe_exchange", "bilstm_heads_create", "bilstm_heads_forward",
           "bilstm_heads_destroy", "bilstm_forward_noalloc", "bilstm_probe_fma_rate",
           "bilstm_probe_mfma_rate"]
HEAD_IN, HEAD_MID, HEAD_CLASSES = 256, 128, 7


class LibraryMissing(RuntimeError):
    pass


class BilstmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class Layer(ctypes.Structure):
    _fields_ = [("w", ctypes.POINTER(ctypes.c_float)), ("w_len", ctypes.c_size_t),
                ("r", ctypes.POINTER(ctypes.c_float)), ("r_len", ctypes.c_size_t),
                ("b", ctypes.POINTER(ctypes.c_float)), ("b_len", ctypes.c_size_t)]


class Options(ctypes.Structure):
    _fields_ = [("recur_groups", ctypes.c_int32), ("recur_tile", ctypes.c_int32),
                ("concurrent", ctypes.c_int32), ("watchdog_us", ctypes.c_int32),
                ("slices", ctypes.c_int32), ("projection", ctypes.c_int32), ("pipeline", ctypes.c_int32),
                ("near_wrap", ctypes.c_int32)]


class HeadWeights(ctypes.Structure):
    _fields_ = [("w0", ctypes.POINTER(ctypes.c_float)), ("w0_len", ctypes.c_size_t),
                ("b0", ctypes.POINTER(ctypes.c_float)), ("b0_len", ctypes.c_size_t),
                ("w1", ctypes.POINTER(ctypes.c_float)), ("w1_len", ctypes.c_size_t),
                ("b1", ctypes.POINTER(ctypes.c_float)), ("b1_len", ctypes.c_size_t),
                ("w2", ctypes.POINTER(ctypes.c_float)), ("w2_len", ctypes.c_size_t),
                ("b2", ctypes.POINTER(ctypes.c_float)), ("b2_len", ctypes.c_size_t),
                ("slope", ctypes.c_float)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_uint32), ("steps", ctypes.c_uint32),
                ("recur_groups", ctypes.c_int32), ("recur_tile", ctypes.c_int32),
                ("recur_tiles", ctypes.c_int32), ("recur_threads", ctypes.c_int32),
                ("recur_launches", ctypes.c_int32), ("concurrent", ctypes.c_int32),
                ("proj_tile_m", ctypes.c_int32), ("proj_tile_n", ctypes.c_int32),
                ("cu_count", ctypes.c_int32), ("recur_capacity", ctypes.c_int32),
                ("device_bytes", ctypes.c_uint64), ("slices", ctypes.c_int32),
                ("slice_windows", ctypes.c_int32), ("projection", ctypes.c_int32),
                ("pipeline", ctypes.c_int32), ("stream_chunk", ctypes.c_int32),
                ("stream_overlap", ctypes.c_int32), ("stream_split", ctypes.c_int32),
                ("stream_fused", ctypes.c_int32), ("stream_serial", ctypes.c_int32),
                ("clears", ctypes.c_uint32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def library():
    """The loaded library; raises LibraryMissing if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    fp = ctypes.POINTER(ctypes.c_float)
    st = ctypes.c_int
    sig = {
        "bilstm_plan_create": ([ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(Layer),
                                ctypes.POINTER(P)], st),
        "bilstm_plan_create_ex": ([ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(Layer),
                                   ctypes.POINTER(Options), ctypes.POINTER(P)], st),
        "bilstm_forward": ([P, P, ctypes.c_size_t, P, ctypes.c_size_t, P], st),
        "bilstm_project": ([P, ctypes.c_int, P, ctypes.c_size_t, P, ctypes.c_size_t, P], st),
        "bilstm_recur": ([P, ctypes.c_int, P, ctypes.c_size_t, P, ctypes.c_size_t, P], st),
        "bilstm_plan_get_info": ([P, ctypes.POINTER(PlanInfo)], st),
        "bilstm_check": ([P], st),
        "bilstm_set_phase_events": ([P, ctypes.c_int], st),
        "bilstm_phase_times": ([P, fp, ctypes.c_size_t], st),
        "bilstm_destroy": ([P], None),
        "bilstm_last_error": ([], ctypes.c_char_p),
        "bilstm_pack_layer": ([ctypes.POINTER(Layer), ctypes.c_uint32, fp, ctypes.c_size_t, fp,
                               ctypes.c_size_t, fp, ctypes.c_size_t], st),
        "bilstm_schedule": ([ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int32, ctypes.c_int32,
                             ctypes.POINTER(Options), ctypes.POINTER(PlanInfo)], st),
        "bilstm_probe_exchange": ([ctypes.c_int, ctypes.c_int, ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32),
                                   ctypes.POINTER(ctypes.c_int32)], st),
        "bilstm_heads_create": ([ctypes.c_int, ctypes.POINTER(HeadWeights), ctypes.POINTER(P)], st),
        "bilstm_heads_forward": ([P, P, ctypes.c_size_t, P, ctypes.c_size_t, P], st),
        "bilstm_heads_destroy": ([P], None),
        "bilstm_forward_noalloc": ([ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(Layer), P,
                                    ctypes.c_size_t, P, ctypes.c_size_t, P], st),
        "bilstm_probe_fma_rate": ([ctypes.c_int, ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)], st),
        "bilstm_probe_mfma_rate": ([ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def last_error() -> str:
    return library().bilstm_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise BilstmError(status, last_error())


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _fptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _layer_struct(layer: dict, keep: list) -> Layer:
    w, r, b = _f32(layer["w"]), _f32(layer["r"]), _f32(layer["b"])
    keep.extend([w, r, b])
    return Layer(_fptr(w), w.size, _fptr(r), r.size, _fptr(b), b.size)


def _options(groups: int, tile: int, concurrent: int, watchdog_us: int = 0, slices: int = 0,
             projection: int = 0, pipeline: int = 0, near_wrap: int = 0) -> Options:
    o = Options()
    o.near_wrap = near_wrap
    o.projection = projection
    o.pipeline = pipeline
    o.recur_groups = groups
    o.recur_tile = tile
    o.concurrent = concurrent
    o.watchdog_us = watchdog_us
    o.slices = slices
    return o


def layers_from_state_dict(state_dict) -> list[dict[str, np.ndarray]]:
    """The four layer dicts ``Plan`` takes, from the parameters of
    ``torch.nn.LSTM(60, 128, num_layers=4, bidirectional=True, batch_first=True)``.

    Per layer k and direction d (``""`` forward, ``"_reverse"``): ``weight_ih_l{k}{d}`` is W,
    ``weight_hh_l{k}{d}`` is R, ``bias_ih_l{k}{d}`` is Wb and ``bias_hh_l{k}{d}`` is Rb (an LSTM
    built with ``bias=False`` gives zero biases). Both use nn.LSTM's gate row order i, f, g, o,
    the order the library takes. Values are copied to float32 on the host; nothing is computed.
    """
    def host(name):
        v = state_dict[name]
        if hasattr(v, "detach"):
            v = v.detach().to("cpu").numpy()
        return np.asarray(v, dtype=np.float32)

    layers = []
    for k in range(LAYERS):
        width = FEATURES if k == 0 else WIDTH
        w, r, b = [], [], []
        for suffix in ("", "_reverse"):
            wk, rk = host(f"weight_ih_l{k}{suffix}"), host(f"weight_hh_l{k}{suffix}")
            if wk.shape != (GATES, width) or rk.shape != (GATES, HIDDEN):
                raise ValueError(f"layer {k}{suffix}: weight_ih {wk.shape} / weight_hh {rk.shape}, expected "
                                 f"({GATES}, {width}) / ({GATES}, {HIDDEN})")
            zero = np.zeros(GATES, np.float32)
            bi = host(f"bias_ih_l{k}{suffix}") if f"bias_ih_l{k}{suffix}" in state_dict else zero
            bh = host(f"bias_hh_l{k}{suffix}") if f"bias_hh_l{k}{suffix}" in state_dict else zero
            if bi.shape != (GATES,) or bh.shape != (GATES,):
                raise ValueError(f"layer {k}{suffix}: biases {bi.shape} / {bh.shape}, expected ({GATES},)")
            w.append(wk)
            r.append(rk)
            b.append(np.stack([bi, bh]))
        layers.append({"w": np.stack(w), "r": np.stack(r), "b": np.stack(b)})
    return layers


def pack_layer(layer: dict, width: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Host-side packer (no GPU): packed W [1024, kpad], R [2, 512, 128], bias [1024]."""
    lib = library()
    keep: list = []
    src = _layer_struct(layer, keep)
    kpad = (width + 31) // 32 * 32
    w = np.zeros((2 * GATES, kpad), np.float32)
    r = np.zeros((2, GATES, HIDDEN), np.float32)
    b = np.zeros((2 * GATES,), np.float32)
    _check(lib.bilstm_pack_layer(ctypes.byref(src), width, _fptr(w), w.size, _fptr(r), r.size,
                                 _fptr(b), b.size))
    return w, r, b


def schedule(batch: int, steps: int, cu_count: int, per_cu: int, groups: int = 0, tile: int = 0,
             concurrent: int = -1, slices: int = 0, projection: int = 0, pipeline: int = 0) -> dict:
    """Host-side recurrence schedule (no GPU)."""
    lib = library()
    info = PlanInfo()
    opt = _options(groups, tile, concurrent, slices=slices, projection=projection, pipeline=pipeline)
    _check(lib.bilstm_schedule(batch, steps, cu_count, per_cu, ctypes.byref(opt), ctypes.byref(info)))
    return info.as_dict()


def probe_exchange(device: int = 0, same_xcd: bool = True, round_trips: int = 2000) -> dict:
    """One-way latency of a flagged 64-bit word between two workgroups (ns) and their XCDs."""
    lib = library()
    ns = ctypes.c_double()
    a = ctypes.c_int32()
    b = ctypes.c_int32()
    _check(lib.bilstm_probe_exchange(device, 1 if same_xcd else 0, round_trips, ctypes.byref(ns),
                                     ctypes.byref(a), ctypes.byref(b)))
    return {"one_way_ns": ns.value, "xcd_a": a.value, "xcd_b": b.value}


def probe_fma_rate(device: int = 0, waves_per_simd: int = 2, workgroups: int = 1, iterations: int = 20000) -> dict:
    """Shader clocks per wave64 FP32 FMA per SIMD, and the shader clock in GHz (see bilstm.h)."""
    lib = library()
    cpf = ctypes.c_double()
    ghz = ctypes.c_double()
    _check(lib.bilstm_probe_fma_rate(device, waves_per_simd, workgroups, iterations, ctypes.byref(cpf),
                                     ctypes.byref(ghz)))
    return {"clocks_per_fma": cpf.value, "ghz": ghz.value}


def probe_mfma_rate(kind: int, data: int, device: int = 0, iterations: int = 20000) -> dict:
    """Matrix-core rate in TFLOP/s: kind 0 bf16 32x32x16, 1 FP32 32x32x2; data 0 zeros, 1 ones,
    2 uniform random operands (see bilstm.h)."""
    lib = library()
    tf = ctypes.c_double()
    ms = ctypes.c_double()
    _check(lib.bilstm_probe_mfma_rate(device, kind, data, iterations, ctypes.byref(tf), ctypes.byref(ms)))
    return {"tflops": tf.value, "ms": ms.value}


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t, name: str, shape: tuple):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


class Plan:
    """A plan for ``batch`` windows of ``steps`` frames (one batch size per plan).

    ``layers`` is a list of four dicts with float32 arrays ``w [2,512,in]``, ``r [2,512,128]``
    and ``b [2,2,512]`` (PyTorch nn.LSTM layout, gate rows i, f, g, o; b = [Wb, Rb]).
    ``groups``, ``tile`` and ``concurrent`` override the plan's recurrence split;
    ``watchdog_us`` bounds each recurrence wait (0 = 2 s); ``slices`` sets how many batch
    slices the forward runs as concurrent chains (0 = auto, 1 = off); ``projection`` picks the
    input projection: 0 the plan's rule (the three-part split where it is accurate and on the
    critical path, else FP32), 1 the vendor GEMM (hipBLASLt), 2 and 3 the library's
    split-precision kernel with two or three bf16 parts, 4 the library's FP32 kernel; ``pipeline`` streams each layer's gates
    from its projection into its recurrence while both run (0 = auto, 1 = off, 2 = on, 3 = on with
    each projection after the previous layer's recurrence, 4 = on with the next layer's projection
    during this layer's recurrence, 5 = as 3 with every kernel after the previous one); ``near_wrap`` = 1 starts the plan's flag epoch and pass
    counters just below the values at which it clears them (a test hook for the clear paths).
    """

    def __init__(self, layers, batch: int, steps: int, device: int = 0, groups: int = 0,
                 tile: int = 0, concurrent: int = -1, watchdog_us: int = 0, slices: int = 0,
                 projection: int = 0, pipeline: int = 0, near_wrap: int = 0):
        if len(layers) != LAYERS:
            raise ValueError(f"expected {LAYERS} layers, got {len(layers)}")
        lib = library()
        keep: list = []
        arr = (Layer * LAYERS)(*[_layer_struct(l, keep) for l in layers])
        opt = _options(groups, tile, concurrent, watchdog_us, slices, projection, pipeline, near_wrap)
        handle = ctypes.c_void_p()
        _check(lib.bilstm_plan_create_ex(device, batch, steps, arr, ctypes.byref(opt), ctypes.byref(handle)))
        self._lib = lib
        self._h = handle
        self.batch = batch
        self.steps = steps
        self.device = device

    @property
    def rows(self) -> int:
        return self.batch * self.steps

    def info(self) -> dict:
        info = PlanInfo()
        _check(self._lib.bilstm_plan_get_info(self._h, ctypes.byref(info)))
        return info.as_dict()

    def forward(self, x, y=None, stream=None):
        """x: [B, T, 60] float32 CUDA tensor; returns y [B, T, 256] (allocated if None)."""
        import torch
        if y is None:
            y = torch.empty((self.batch, self.steps, WIDTH), dtype=torch.float32, device=x.device)
        xp = _dev_ptr(x, "x", (self.batch, self.steps, FEATURES))
        yp = _dev_ptr(y, "y", (self.batch, self.steps, WIDTH))
        _check(self._lib.bilstm_forward(self._h, xp, x.numel(), yp, y.numel(), _stream_handle(stream)))
        return y

    def project(self, layer: int, x, gates=None, stream=None):
        """One layer's projection: x [B·T, in] -> gates [B·T, 1024] (packed gate columns)."""
        import torch
        width = FEATURES if layer == 0 else WIDTH
        if gates is None:
            gates = torch.empty((self.rows, 2 * GATES), dtype=torch.float32, device=x.device)
        xp = _dev_ptr(x, "x", (self.rows, width))
        gp = _dev_ptr(gates, "gates", (self.rows, 2 * GATES))
        _check(self._lib.bilstm_project(self._h, layer, xp, x.numel(), gp, gates.numel(),
                                        _stream_handle(stream)))
        return gates

    def recur(self, layer: int, gates, y=None, stream=None):
        """One layer's recurrence: gates [B·T, 1024] -> y [B, T, 256]."""
        import torch
        if y is None:
            y = torch.empty((self.batch, self.steps, WIDTH), dtype=torch.float32, device=gates.device)
        gp = _dev_ptr(gates, "gates", (self.rows, 2 * GATES))
        yp = _dev_ptr(y, "y", (self.batch, self.steps, WIDTH))
        _check(self._lib.bilstm_recur(self._h, layer, gp, gates.numel(), yp, y.numel(),
                                      _stream_handle(stream)))
        return y

    def check(self) -> None:
        """Wait for the plan's last call; raise BilstmError(BILSTM_TIMEOUT) if a watchdog fired."""
        _check(self._lib.bilstm_check(self._h))

    def set_phase_events(self, enable: bool) -> None:
        _check(self._lib.bilstm_set_phase_events(self._h, 1 if enable else 0))

    def phase_times(self) -> dict:
        """Per-phase milliseconds of the last forward run with phase events on."""
        ms = (ctypes.c_float * 12)()
        _check(self._lib.bilstm_phase_times(self._h, ms, 12))
        return {"projection_ms": [ms[i] for i in range(4)], "recurrence_ms": [ms[4 + i] for i in range(4)],
                "recurrence_launch_ms": [ms[8 + i] for i in range(4)]}

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.bilstm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def device_layers(layers, device="cuda") -> list[dict]:
    """The four layer dicts of ``Plan`` as contiguous float32 tensors on ``device``, for
    ``forward_noalloc`` (a copy; nothing computed)."""
    import torch
    return [{k: torch.from_numpy(_f32(l[k])).to(device) for k in ("w", "r", "b")} for l in layers]


def forward_noalloc(layers, x, y, stream=None, device: int = 0) -> None:
    """The whole stack without a plan and without allocating (bilstm_forward_noalloc).

    ``layers``: four dicts of contiguous float32 device tensors ``w [2,512,in]``, ``r [2,512,128]``,
    ``b [2,2,512]`` (see ``device_layers``); ``x [B,T,60]`` and ``y [B,T,256]`` float32 device
    tensors, ``y`` written. Only marshals pointers: no tensor is created here.
    """
    import torch
    if len(layers) != LAYERS:
        raise ValueError(f"expected {LAYERS} layers, got {len(layers)}")
    batch, steps = int(x.shape[0]), int(x.shape[1])
    arr = (Layer * LAYERS)()
    for k, l in enumerate(layers):
        width = FEATURES if k == 0 else WIDTH
        for name, shape in (("w", (2, GATES, width)), ("r", (2, GATES, HIDDEN)), ("b", (2, 2, GATES))):
            t = l[name]
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
                raise TypeError(f"layer {k} {name} must be a contiguous float32 device tensor")
            if tuple(t.shape) != shape:
                raise ValueError(f"layer {k} {name} has shape {tuple(t.shape)}, expected {shape}")
        arr[k] = Layer(ctypes.cast(l["w"].data_ptr(), ctypes.POINTER(ctypes.c_float)), l["w"].numel(),
                       ctypes.cast(l["r"].data_ptr(), ctypes.POINTER(ctypes.c_float)), l["r"].numel(),
                       ctypes.cast(l["b"].data_ptr(), ctypes.POINTER(ctypes.c_float)), l["b"].numel())
    xp = _dev_ptr(x, "x", (batch, steps, FEATURES))
    yp = _dev_ptr(y, "y", (batch, steps, WIDTH))
    _check(library().bilstm_forward_noalloc(device, batch, steps, arr, xp, x.numel(), yp, y.numel(),
                                            _stream_handle(stream)))


def gate_column(direction: int, unit: int, gate: int) -> int:
    """Column of (direction, hidden unit, gate) in the packed gate buffer: d·512 + 4j + g."""
    return direction * GATES + 4 * unit + gate


class Heads:
    """The segmentation heads after the stack (linear0, linear1, classifier with LeakyReLU and
    log-softmax), fused on the GPU.

    ``head`` holds float32 ``w0 [256, 128]``, ``b0``, ``w1 [128, 128]``, ``b1``, ``w2 [128, 7]``,
    ``b2`` (row-major ``[k, n]``) and ``slope``.
    """

    def __init__(self, head: dict, device: int = 0):
        lib = library()
        keep = [_f32(head[k]) for k in ("w0", "b0", "w1", "b1", "w2", "b2")]
        hw = HeadWeights(*[v for a in keep for v in (_fptr(a), a.size)], ctypes.c_float(head["slope"]))
        handle = ctypes.c_void_p()
        _check(lib.bilstm_heads_create(device, ctypes.byref(hw), ctypes.byref(handle)))
        self._lib = lib
        self._h = handle
        self.device = device

    def forward(self, y, out=None, stream=None):
        """y: [..., 256] float32 CUDA tensor (e.g. the stack's [B, T, 256]); returns [..., 7]."""
        import torch
        rows = y.numel() // HEAD_IN
        if out is None:
            out = torch.empty(tuple(y.shape[:-1]) + (HEAD_CLASSES,), dtype=torch.float32, device=y.device)
        yp = _dev_ptr(y, "y", tuple(y.shape[:-1]) + (HEAD_IN,))
        op = _dev_ptr(out, "out", tuple(y.shape[:-1]) + (HEAD_CLASSES,))
        if rows == 0:
            return out
        _check(self._lib.bilstm_heads_forward(self._h, yp, rows * HEAD_IN, op, rows * HEAD_CLASSES,
                                              _stream_handle(stream)))
        return out

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.bilstm_heads_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
