"""Seeded synthetic inputs for the bidirectional LSTM stack.

This module only draws random numbers. It holds none of the LSTM arithmetic, so both the
oracle tests and the HIP path can take their inputs from it without sharing any of the
method's code.

The stack is the segmentation model's four bidirectional LSTM layers described on the
speakrs 0.6.0 `lstmproj.rs` page (module doc; `PackedLayer` doc): hidden size 128, 512 gate
rows per direction, input width 60 in the first layer and 256 (forward and reverse hidden
states side by side) in the others, inputs cut into 589-frame windows (the same page,
`driver_pin`).

Weights follow PyTorch's `nn.LSTM` layout and default initialisation, U(-1/sqrt(H), 1/sqrt(H)):

* ``w``: float32 ``[2, 4H, in]``, direction 0 forward, 1 reverse, gate rows in blocks i, f, g, o
* ``r``: float32 ``[2, 4H, H]``
* ``b``: float32 ``[2, 2, 4H]``, per direction the input bias (Wb) then the recurrent bias (Rb)

Per layer the draws are taken in the order W, R, Wb, Rb (each covering both directions),
then the input. No data set is involved: every workload here is synthetic.

The segmentation heads that follow the stack (the `segdense.rs` page, `Site` doc: 256 to 128,
128 to 128 and 128 to 7, weights row-major ``[k, n]``) draw from their own stream: ``w0``,
``b0``, ``w1``, ``b1``, ``w2``, ``b2``, each ~ U(-1/sqrt(k), 1/sqrt(k)) (PyTorch's `nn.Linear`
default), with LeakyReLU slope 0.01 (PyTorch's default; the page gives none).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

HIDDEN = 128
FEATURES = 60
LAYERS = 4
FRAMES = 589


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, value distribution and seed."""

    name: str
    batch: int
    steps: int
    seed: int
    input_sigma: float = 1.0
    r_scale: float = 1.0
    zero_every: int = 0  # windows with b % zero_every == 0 get an all-zero input (0 = none)

    @property
    def frames(self) -> int:
        return self.batch * self.steps


# The five workloads. ``b1`` is small enough for the oracle to run whole in seconds;
# ``b32`` is the headline throughput workload.
WORKLOADS = {
    "b1": Workload("b1", 1, FRAMES, seed=1001),
    "b8": Workload("b8", 8, FRAMES, seed=1002),
    "b32": Workload("b32", 32, FRAMES, seed=1003),
    "b256": Workload("b256", 256, FRAMES, seed=1004, zero_every=10),
    "b64_t4096": Workload("b64_t4096", 64, 4096, seed=1005, input_sigma=2.0, r_scale=2.0),
}


def make_layers(seed: int, hidden: int = HIDDEN, features: int = FEATURES, layers: int = LAYERS,
                r_scale: float = 1.0) -> list[dict[str, np.ndarray]]:
    """Draw every layer's W, R and biases from ``seed``.

    ``r_scale`` multiplies the recurrent matrices only (the long-sequence stress workload
    uses 2). The multiplication happens after the float32 cast, so it is exact.
    """
    rng = np.random.default_rng(seed)
    bound = 1.0 / math.sqrt(hidden)
    gates = 4 * hidden
    out = []
    for layer in range(layers):
        width = features if layer == 0 else 2 * hidden
        w = rng.uniform(-bound, bound, size=(2, gates, width)).astype(np.float32)
        r = rng.uniform(-bound, bound, size=(2, gates, hidden)).astype(np.float32)
        wb = rng.uniform(-bound, bound, size=(2, gates)).astype(np.float32)
        rb = rng.uniform(-bound, bound, size=(2, gates)).astype(np.float32)
        if r_scale != 1.0:
            r = (r * np.float32(r_scale)).astype(np.float32)
        b = np.stack([wb, rb], axis=1)  # [2 directions][Wb, Rb][4H]
        out.append({"w": np.ascontiguousarray(w), "r": np.ascontiguousarray(r),
                    "b": np.ascontiguousarray(b)})
    return out


def make_input(seed: int, batch: int, steps: int, features: int = FEATURES,
               sigma: float = 1.0, zero_every: int = 0) -> np.ndarray:
    """Draw a ``[batch, steps, features]`` float32 input ~ N(0, sigma).

    The generator is seeded with ``seed + 1`` so the input stream is independent of the
    weight stream. Windows with ``b % zero_every == 0`` are all-zero when ``zero_every`` > 0.
    """
    rng = np.random.default_rng(seed + 1)
    x = rng.standard_normal(size=(batch, steps, features), dtype=np.float64)
    x = (x * sigma).astype(np.float32)
    if zero_every > 0:
        x[::zero_every] = 0.0
    return np.ascontiguousarray(x)


def make_workload(wl: Workload | str) -> tuple[np.ndarray, list[dict[str, np.ndarray]]]:
    """Input and weights for a named workload."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    layers = make_layers(wl.seed, r_scale=wl.r_scale)
    x = make_input(wl.seed, wl.batch, wl.steps, sigma=wl.input_sigma, zero_every=wl.zero_every)
    return x, layers


def random_layers(seed: int, hidden: int, features: int, layers: int,
                  scale: float | None = None) -> list[dict[str, np.ndarray]]:
    """Weights of arbitrary (small) sizes for oracle pins; same layout as ``make_layers``."""
    rng = np.random.default_rng(seed)
    bound = scale if scale is not None else 1.0 / math.sqrt(hidden)
    gates = 4 * hidden
    out = []
    for layer in range(layers):
        width = features if layer == 0 else 2 * hidden
        out.append({
            "w": rng.uniform(-bound, bound, size=(2, gates, width)).astype(np.float32),
            "r": rng.uniform(-bound, bound, size=(2, gates, hidden)).astype(np.float32),
            "b": rng.uniform(-bound, bound, size=(2, 2, gates)).astype(np.float32),
        })
    return out


HEAD_SIZES = (256, 128, 128, 7)   # stack output, linear0, linear1, classes
LEAKY_SLOPE = 0.01


def make_heads(seed: int, sizes: tuple = HEAD_SIZES, slope: float = LEAKY_SLOPE) -> dict:
    """Draw the heads' weights ``[k, n]`` and biases from ``seed + 2`` (own stream)."""
    rng = np.random.default_rng(seed + 2)
    out: dict = {"slope": slope}
    for i in range(3):
        k, n = sizes[i], sizes[i + 1]
        bound = 1.0 / math.sqrt(k)
        out[f"w{i}"] = np.ascontiguousarray(rng.uniform(-bound, bound, size=(k, n)).astype(np.float32))
        out[f"b{i}"] = np.ascontiguousarray(rng.uniform(-bound, bound, size=(n,)).astype(np.float32))
    return out
