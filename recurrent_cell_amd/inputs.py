"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module draws random numbers and nothing else: it holds none of the cell's
arithmetic and imports neither the GPU library nor the oracle.

Recipe (numpy PCG64 via ``default_rng``):
  * CfC K-loop: one stream seeded with ``seed``; draw order h0, u, y, W_f, W_g,
    W_h, each drawn in float64 and cast to fp32.  h0, u, y ~ N(0, 1);
    W_q ~ U(-1/sqrt(n_in), 1/sqrt(n_in)); biases zero.  With
    ``bias_scale > 0`` the three bias rows are drawn after W_h from
    U(-bias_scale, bias_scale) (parity cases that exercise the bias path).
  * Batch-axis reduction: row b of a [B, N] array comes from its own stream
    ``default_rng([seed, b]).standard_normal(N, dtype=float32)``, so any row
    can be regenerated alone.
"""
from dataclasses import dataclass

import numpy as np


@dataclass
class CfcInputs:
    u: np.ndarray      # [K, B, n_x] fp32
    y: np.ndarray      # [K, B, C]   fp32
    h0: np.ndarray     # [B, C]      fp32
    W: np.ndarray      # [3, C, n_in] fp32 (heads f, g, h)
    bias: np.ndarray   # [3, C]      fp32

    @property
    def dims(self):
        K, B, n_x = self.u.shape
        C = self.h0.shape[1]
        return dict(B=B, C=C, n_x=n_x, K=K)


def cfc_inputs(B: int, C: int, n_x: int, K: int, seed: int = 0,
               bias_scale: float = 0.0) -> CfcInputs:
    rng = np.random.default_rng(seed)
    n_in = n_x + C
    h0 = rng.standard_normal((B, C)).astype(np.float32)
    u = rng.standard_normal((K, B, n_x)).astype(np.float32)
    y = rng.standard_normal((K, B, C)).astype(np.float32)
    bound = 1.0 / np.sqrt(n_in) if n_in > 0 else 0.0
    W = np.stack([rng.uniform(-bound, bound, (C, n_in)) for _ in range(3)]).astype(np.float32)
    if bias_scale > 0:
        bias = rng.uniform(-bias_scale, bias_scale, (3, C)).astype(np.float32)
    else:
        bias = np.zeros((3, C), np.float32)
    return CfcInputs(u=np.ascontiguousarray(u), y=np.ascontiguousarray(y),
                     h0=np.ascontiguousarray(h0), W=np.ascontiguousarray(W),
                     bias=np.ascontiguousarray(bias))


def reduce_row(seed: int, b: int, N: int) -> np.ndarray:
    """Row b of the batch-axis reduction input: N(0,1) fp32 from stream [seed, b]."""
    return np.random.default_rng([seed, b]).standard_normal(N, dtype=np.float32)


def reduce_rows(B: int, N: int, seed: int = 0) -> np.ndarray:
    out = np.empty((B, N), np.float32)
    for b in range(B):
        out[b] = reduce_row(seed, b, N)
    return out


def normal(shape, seed: int, stream: int = 0) -> np.ndarray:
    """N(0, 1) fp32 array from stream [seed, stream] (extra operands of the
    single-step cases: incoming carry, pre-existing scratch)."""
    return np.random.default_rng([seed, 0x5EED, stream]).standard_normal(shape).astype(np.float32)


def adamw_inputs(sizes, seed: int):
    """Optimizer state for one AdamW step over segments of the given sizes:
    parameters ~ N(0, 0.25), gradients and first moments ~ N(0, 1e-4), second
    moments = squares of N(0, 1e-4) draws (non-negative, as the method keeps
    them), all fp32.  Returns four lists (p, g, m, v)."""
    out = ([], [], [], [])
    for i, n in enumerate(sizes):
        rng = np.random.default_rng([seed, 0xADA, i])
        d = rng.standard_normal((4, n))
        vals = (0.5 * d[0], 1e-2 * d[1], 1e-2 * d[2], (1e-2 * d[3]) ** 2)
        for lst, a in zip(out, vals):
            lst.append(a.astype(np.float32))
    return out


def small_int_rows(B: int, N: int, seed: int = 0, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integers in [lo, hi] stored as fp32: every partial sum of at most 2^20 such
    rows is an integer below 2^24 in magnitude, so fp32 sums of them are exact."""
    rng = np.random.default_rng([seed, 0x1A7])
    return rng.integers(lo, hi + 1, size=(B, N)).astype(np.float32)


# The configurations the library is measured and checked on.
class MlpInputs:
    """Seeded MLP training-step inputs: X [B, dims[0]], T [B, dims[-1]] ~ N(0, 1);
    W_l [dims[l+1], dims[l]] He-uniform U(+-sqrt(6 / dims[l])); b_l zero, or
    U(+-bias_scale) when bias_scale > 0 (parity cases, so that the bias path
    is exercised).  All fp32."""

    def __init__(self, B, dims, seed=0, bias_scale=0.0):
        rng = np.random.default_rng([seed, 0x4D4C50])
        self.dims = list(dims)
        self.X = rng.standard_normal((B, dims[0])).astype(np.float32)
        self.T = rng.standard_normal((B, dims[-1])).astype(np.float32)
        self.W, self.b = [], []
        for l in range(len(dims) - 1):
            bound = np.sqrt(6.0 / dims[l])
            self.W.append(rng.uniform(-bound, bound, (dims[l + 1], dims[l])).astype(np.float32))
        for l in range(len(dims) - 1):
            if bias_scale > 0:
                self.b.append(rng.uniform(-bias_scale, bias_scale, dims[l + 1]).astype(np.float32))
            else:
                self.b.append(np.zeros(dims[l + 1], np.float32))


MLP_DIMS = (48, 256, 256, 128, 51)
MLP_B = 16384

CONFIGS = {
    "tiny": dict(B=4, C=16, n_x=8, K=4),
    "pages": dict(B=32, C=128, n_x=64, K=64),
    "wide": dict(B=256, C=256, n_x=128, K=64),
}
REDUCE_B = (32, 128, 256)
REDUCE_N = (4096, 73728, 1048576, 8388608)
