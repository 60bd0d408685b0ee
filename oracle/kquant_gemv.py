"""Oracle: batched GEMV straight from Q4_K / Q6_K super-blocks (small M).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages (realizar 0.8.4: the note on ``cublas_gemm_threshold`` on the
``cublas_prefill/mod.rs`` page, and the ``q4k_gemv_into`` /
``q6k_gemv_indexed_async`` dispatchers on the ``q6k_gemv_indexed.rs`` page)
send a batch of fewer rows than a threshold (4 by default) to GEMV kernels
that read the K-quant blocks directly, with an fp32 input and an fp32
output, instead of dequantising the weight and running a GEMM.  They print
the dispatchers, not the kernels, so the operation is taken as its plain
definition:

    y[i][j] = sum_k x[i][k] * w[j][k],   w = dequant(qtype, blocks, n, k)

with x fp32 [m][k] row-major, w the fp32 dequantised weight [n][k] (exactly
as ``kquant.dequant``) and y fp32 [m][n] row-major.

Here each product of two fp32 values is exact in float64 (at most 48
significant bits) and the K products are summed in float64, so ``gemv`` is
within about K * 2^-53 of the exact value.  A GPU that accumulates in fp32,
in any order, with fused or separate multiply-adds, is within
``bound`` = gamma_K * sum_k |x[i][k] * w[j][k]| of the exact value, gamma_K
= K u / (1 - K u), u = 2^-24 (the standard bound for a sum of K terms
evaluated in any order).
"""
from __future__ import annotations

import numpy as np

from .kquant import QK_K, dequant

U32 = 2.0 ** -24


def _check(qtype: int, n: int, k: int, x: np.ndarray) -> np.ndarray:
    if k % QK_K != 0:
        raise ValueError("k must be a multiple of 256")
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] != k:
        raise ValueError("x must be fp32 [m][k]")
    return x


def gemv(qtype: int, blocks: np.ndarray, n: int, k: int, x: np.ndarray) -> np.ndarray:
    """float64 [m][n]: y[i][j] = sum_k x[i][k] * dequant(W)[j][k]."""
    x = _check(qtype, n, k, x)
    w = dequant(qtype, blocks, n, k).astype(np.float64)
    return x.astype(np.float64) @ w.T


def gemv_abs(qtype: int, blocks: np.ndarray, n: int, k: int, x: np.ndarray) -> np.ndarray:
    """float64 [m][n]: sum_k |x[i][k] * dequant(W)[j][k]|."""
    x = _check(qtype, n, k, x)
    w = np.abs(dequant(qtype, blocks, n, k).astype(np.float64))
    return np.abs(x.astype(np.float64)) @ w.T


def bound(qtype: int, blocks: np.ndarray, n: int, k: int, x: np.ndarray) -> np.ndarray:
    """Largest |y_fp32 - gemv| for fp32 accumulation in any order."""
    g = k * U32 / (1.0 - k * U32)
    return g * gemv_abs(qtype, blocks, n, k, x)
