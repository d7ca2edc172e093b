"""Seeded synthetic inputs for the LLM.int8() linear layer.

This module only draws numbers: it holds none of the layer's arithmetic, so the
CPU oracle and the HIP path can both be fed the very same bytes from it.

Shapes follow the BLOOM-176B layer sizes used as stand-ins for the model
workloads that the blog "A Gentle Introduction to 8-bit Matrix Multiplication
for transformers at scale using Hugging Face Transformers, Accelerate and
bitsandbytes" evaluates on (sections "Is it faster than native models?" and
"What does 0 degradation mean?"); no model weights or datasets are used.

Recipe (one workload):
  * X: fp32 draws from N(0, x_sigma^2), clamped to |x| <= 5.75 so that only the
    injected columns can reach the outlier threshold 6, then cast to fp16 (RNE).
  * ``n_out`` columns of X, picked without replacement, have every entry
    replaced by +/-U(out_lo, out_hi) with a random sign (cast to fp16).
  * W: fp32 draws from N(0, w_sigma^2), cast to fp16; math layout [K][N]
    (Y = X @ W, i.e. the transpose of an nn.Linear weight).
  * X and W come from two independent PCG64 streams keyed by (seed, 0) and
    (seed, 1), so X can be drawn without drawing W.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_x", "make_w", "make_inputs", "CLAMP"]

# Largest magnitude a base draw of X may take (an fp16 value, below threshold 6).
CLAMP = 5.75

# Rows (or elements) drawn per chunk: bounds host memory for the 1.6 GB weights.
_CHUNK_ELEMS = 1 << 24


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    x_sigma: float
    w_sigma: float
    n_out: int
    out_lo: float
    out_hi: float
    seed: int
    threshold: float = 6.0

    def as_dict(self):
        return asdict(self)

    @property
    def int_ops(self) -> int:
        """Dense linear-layer operation count 2*M*N*K."""
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 16, 1024, 4096, 1.0, 0.02, 2, 8.0, 20.0, seed=1),
        Workload("decode", 8, 4096, 16384, 1.0, 0.02, 4, 6.5, 40.0, seed=2),
        Workload("qkv_prefill", 2048, 14336, 43008, 1.0, 0.02, 8, 8.0, 60.0, seed=3),
        Workload("mlp_down_prefill", 4096, 57344, 14336, 0.5, 0.01, 16, 8.0, 60.0, seed=4),
        Workload("square_0pct", 8192, 8192, 8192, 1.0, 0.02, 0, 6.0, 100.0, seed=50),
        Workload("square_0.1pct", 8192, 8192, 8192, 1.0, 0.02, 8, 6.0, 100.0, seed=51),
        Workload("square_1pct", 8192, 8192, 8192, 1.0, 0.02, 82, 6.0, 100.0, seed=52),
        # decode batch (8 tokens) through the two BLOOM-176B prefill layers
        # above: the weight stream of the small-M path at K > 4096
        Workload("decode_qkv", 8, 14336, 43008, 1.0, 0.02, 8, 8.0, 60.0, seed=6),
        Workload("decode_mlp_down", 8, 57344, 14336, 0.5, 0.01, 16, 8.0, 60.0, seed=7),
        # a batch of 32 tokens on the decode layer: the weight-bound path for
        # 16 < M <= 64
        Workload("decode_m32", 32, 4096, 16384, 1.0, 0.02, 4, 6.5, 40.0, seed=8),
        # the decode layer with 1 % of its hidden columns outliers (41 of
        # 4096): the fused kernel's path for many outlier columns per wave
        Workload("decode_1pct", 8, 4096, 16384, 1.0, 0.02, 41, 6.5, 40.0, seed=9),
        # batches of 128 and 256 tokens on the decode layer: weight-bound shapes
        # above the streaming kernel's 64 rows
        Workload("decode_m128", 128, 4096, 16384, 1.0, 0.02, 4, 6.5, 40.0, seed=10),
        Workload("decode_m256", 256, 4096, 16384, 1.0, 0.02, 4, 6.5, 40.0, seed=11),
    ]
}


def _normal_fp16(rng: np.random.Generator, shape, sigma: float, clamp: float | None):
    """Fill an fp16 array of ``shape`` with N(0, sigma^2) draws, chunk by chunk."""
    out = np.empty(shape, dtype=np.float16)
    flat = out.reshape(-1)
    for s in range(0, flat.size, _CHUNK_ELEMS):
        e = min(flat.size, s + _CHUNK_ELEMS)
        v = rng.standard_normal(e - s, dtype=np.float32)
        v *= np.float32(sigma)
        if clamp is not None:
            np.clip(v, -clamp, clamp, out=v)
        flat[s:e] = v.astype(np.float16)
    return out


def make_x(M, K, x_sigma, n_out, out_lo, out_hi, seed):
    """Activations X fp16 [M][K] with ``n_out`` injected outlier columns.

    Returns (X, cols) where ``cols`` are the injected column indices, unsorted.
    """
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    X = _normal_fp16(rng, (M, K), x_sigma, CLAMP)
    cols = rng.choice(K, size=n_out, replace=False) if n_out > 0 else np.zeros(0, np.int64)
    if n_out > 0:
        mags = rng.uniform(out_lo, out_hi, size=(M, n_out)).astype(np.float32)
        signs = np.where(rng.integers(0, 2, size=(M, n_out)) == 1, 1.0, -1.0).astype(np.float32)
        X[:, cols] = (mags * signs).astype(np.float16)
    return X, cols


def make_w(K, N, w_sigma, seed):
    """Weights W fp16 [K][N] (math layout, Y = X @ W)."""
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    return _normal_fp16(rng, (K, N), w_sigma, None)


def make_inputs(w: Workload | str, with_w: bool = True):
    """(X, W, cols) for a named workload; W is None when ``with_w`` is False."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    X, cols = make_x(w.M, w.K, w.x_sigma, w.n_out, w.out_lo, w.out_hi, w.seed)
    W = make_w(w.K, w.N, w.w_sigma, w.seed) if with_w else None
    return X, W, cols


def make_small(M, K, N, seed, n_out=0, x_sigma=1.0, w_sigma=0.02, out_lo=8.0, out_hi=20.0):
    """Small ad-hoc case with the same recipe (for ragged-shape parity tests)."""
    X, cols = make_x(M, K, x_sigma, n_out, out_lo, out_hi, seed)
    W = make_w(K, N, w_sigma, seed)
    return X, W, cols
