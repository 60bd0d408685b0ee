"""Oracle: the FP16 cached-weight GEMM the FP8 path replaced (comparator).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (realizar 0.8.4):
* page ``cublas_prefill/gemm.rs``, ``get_or_cache_fp16_weight`` — on a cache
  miss the K-quant weight is dequantised to an fp32 scratch tensor, which is
  then converted to fp16 (one value per weight, [N][K] row-major) and cached;
* page ``cublas_prefill/gemm.rs``, ``cublas_prefill_hgemm`` — the fp32
  activation [M][K] is converted to fp16, and the GEMM multiplies the fp16
  activation by the transposed fp16 weight with fp32 accumulation and an
  fp32 output [M][N] (no scale factors: alpha 1, beta 0);
* page ``cublas_prefill/mod.rs``, ``F32_TO_F16_PTX`` — the conversion is the
  round-to-nearest-even fp32 -> fp16 conversion (``cvt.rn.f16.f32``), so
  values of magnitude >= 65520 become +-Inf, NaN stays NaN and small values
  round to fp16 subnormals.

Readings (the pages are silent):
* the fp16 activation buffer has pad16(M) rows, rows M.. are zero (the same
  padding as the FP8 activation; only rows < M of the output exist);
* the GEMM may sum in any order in fp32; ``bound`` is the resulting error
  bound against the float64 sum computed here.
"""
from __future__ import annotations

import numpy as np

from . import kquant

U32 = 2.0 ** -24  # unit roundoff of fp32
U64 = 2.0 ** -53  # unit roundoff of float64


def pad_m(m: int) -> int:
    return (m + 15) & ~15


def to_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 with round-to-nearest-even (numpy's conversion)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def pack_weight(qtype: int, blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    """fp16 [n][k]: the fp32 dequantised weight, each value rounded to fp16."""
    return to_f16(kquant.dequant(qtype, blocks, n, k)).reshape(n, k)


def convert_act(x: np.ndarray) -> np.ndarray:
    """fp16 [pad_m(m)][k] of fp32 x [m][k]; pad rows zero."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    out = np.zeros((pad_m(m), k), dtype=np.float16)
    out[:m] = to_f16(x)
    return out


def gemm(a16: np.ndarray, w16: np.ndarray, m: int) -> np.ndarray:
    """float64 y [m][N] = sum_k a[i][k] * w[j][k] over the fp16 values.

    Each product of two fp16 values is exact in float64 (22 significant
    bits); the sum over K is float64, within (K-1) 2^-53 sum|a w| of exact."""
    A = np.asarray(a16, dtype=np.float16)[:m].astype(np.float64)
    Wt = np.asarray(w16, dtype=np.float16).astype(np.float64)
    return A @ Wt.T


def abs_sum(a16: np.ndarray, w16: np.ndarray, m: int) -> np.ndarray:
    """float64 [m][N]: sum_k |a[i][k] * w[j][k]|."""
    A = np.abs(np.asarray(a16, dtype=np.float16)[:m].astype(np.float64))
    Wt = np.abs(np.asarray(w16, dtype=np.float16).astype(np.float64))
    return A @ Wt.T


def bound(a16: np.ndarray, w16: np.ndarray, m: int) -> np.ndarray:
    """Largest |y_gpu - gemm| for an fp32 sum of the exact products in any
    order with a relative error of at most 2u per addition (u = 2^-24:
    round to nearest gives u, a truncating adder inside the matrix core at
    most 2u), plus this oracle's own float64 error:
    (gamma_K(2u) + gamma_K(2^-53)) * sum_k |a w|,
    gamma_K(v) = K v / (1 - K v)."""
    k = np.asarray(w16).shape[1]
    g32 = 2 * k * U32 / (1.0 - 2 * k * U32)
    g64 = k * U64 / (1.0 - k * U64)
    return (g32 + g64) * abs_sum(a16, w16, m)
