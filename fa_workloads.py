"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random numbers and encodes them; it holds none of the
attention arithmetic.  The oracle and the HIP path both consume what it makes:
the same 16-bit words are uploaded to the device and decoded (exactly) to
float64 for the oracle.

Recipe (one per workload, seed 0 unless ``FA_SEED`` says otherwise):

* ``numpy.random.default_rng(seed)``; Q, K and V drawn in that order as
  float32 standard normals of shape [B, H, N, d] (row-major).
* Workload-specific changes are made in float32 after the draw: "spiky" scales
  round(1% of N) distinct key rows per head by 8 (chosen with ``rng.choice``
  after the three draws, head by head in (b, h) order); "half" multiplies all
  three tensors by 0.5 (standard deviation 0.5).
* The 16-bit encodings round to nearest even: IEEE half via numpy, bfloat16
  by rounding the float32 bit pattern.
* The backward's output gradient dO is a fourth tensor of float32 standard
  normals from ``default_rng([seed, 1])`` (``draw_dout``), encoded the same
  way.
* ``scale`` is float32(1 / sqrt(d)), the value handed to the device; the
  oracle widens that same float32 to float64.

Shapes and value distributions follow the pages' workloads (N=4096, d=128 in
the HBM-traffic and on-chip-budget examples); there is no dataset.
"""

import os
from dataclasses import dataclass

import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str               # "f32" | "f16" | "bf16"
    values: str              # "normal" | "spiky" | "half"
    causal: tuple            # mask settings exercised
    tile: tuple = None       # (block_q, block_k) forced, or None for the default

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def flops(self, causal):
        """4 B H N^2 d (two multiply-adds per score per head dimension over
        the two contractions), halved under the causal mask by convention."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if causal else f


WORKLOADS = {
    # single head, fp32 arithmetic, 64x64 tiles
    "C1": Workload("C1", 1, 1, 256, 64, "f32", "normal", (False, True), (64, 64)),
    # the pages' N=4096, d=128 example shape in fp16, non-causal
    "C2": Workload("C2", 4, 16, 4096, 128, "f16", "normal", (False,)),
    # the same shape in bf16, non-causal: the throughput target row
    "C2b": Workload("C2b", 4, 16, 4096, 128, "bf16", "normal", (False,)),
    # bf16, causal, 1% of key rows x8 to exercise the running-max rescale
    "C3": Workload("C3", 4, 16, 4096, 128, "bf16", "spiky", (True,)),
    # ragged: N not a multiple of any tile
    "C4": Workload("C4", 16, 32, 1000, 64, "bf16", "normal", (False, True)),
    # long context, causal, N(0, 0.5^2)
    "C5": Workload("C5", 1, 32, 32768, 128, "bf16", "half", (True,)),
}


def default_seed():
    return int(os.environ.get("FA_SEED", "0"))


def draw_f32(shape, values="normal", seed=0):
    """Q, K, V as float32 arrays per the recipe in the module docstring."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if values == "spiky":
        B, H, N, _ = shape
        n_rows = int(round(0.01 * N))
        for b in range(B):
            for h in range(H):
                idx = rng.choice(N, n_rows, replace=False)
                k[b, h, idx] *= np.float32(8.0)
    elif values == "half":
        for t in (q, k, v):
            t *= np.float32(0.5)
    elif values != "normal":
        raise ValueError(f"unknown value recipe {values!r}")
    return q, k, v


def draw_dout(shape, seed=0):
    """The output gradient dO for the backward workloads: float32 standard
    normals of ``shape`` from its own generator, ``default_rng([seed, 1])``,
    so that the Q, K, V draws of the same seed are unchanged."""
    return np.random.default_rng([seed, 1]).standard_normal(shape, dtype=np.float32)


def bf16_encode(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs here are finite, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_decode(w):
    """bfloat16 bit patterns (uint16) -> float32, exact."""
    return (np.asarray(w, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def encode(x, dtype):
    """float32 array -> the array of element words handed to the device:
    float32 itself, float16, or bfloat16 words as uint16."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return bf16_encode(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode64(w, dtype):
    """Device element words -> float64, exactly (every fp32/fp16/bf16 value is
    representable in float64)."""
    if dtype == "bf16":
        return bf16_decode(w).astype(np.float64)
    return np.asarray(w).astype(np.float64)


def scale_for(d):
    """The softmax scale handed to the device: float32(1/sqrt(d))."""
    return float(np.float32(1.0 / np.sqrt(np.float64(d))))


def make_words(shape, dtype, values="normal", seed=0):
    """Encoded Q, K, V words for the device only (the oracle decodes the heads
    it needs with ``decode64``)."""
    return tuple(encode(t, dtype) for t in draw_f32(shape, values, seed))


def make(shape, dtype, values="normal", seed=0):
    """Encoded Q, K, V words for the device and their exact float64 values
    for the oracle: returns ``(words, values64)``, each a (q, k, v) tuple."""
    f32 = draw_f32(shape, values, seed)
    words = tuple(encode(t, dtype) for t in f32)
    vals = tuple(decode64(w, dtype) for w in words)
    return words, vals


def make_workload(wl, seed=None):
    """``make`` for a named workload."""
    seed = default_seed() if seed is None else seed
    return make(wl.shape, wl.dtype, wl.values, seed)
