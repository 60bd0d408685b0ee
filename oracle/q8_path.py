"""Oracle: the integer path — Q8_1 activation blocks times Q4_K weights.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source (realizar 0.8.4, page ``cublas_prefill/gemm.rs``,
``launch_dp4a_q4k_gemm`` and the ``DP4A_GEMM_PREFILL`` branch of
``cublas_prefill_gemm``): the fp32 activation [M][K] is first quantised to
the Q8_1 format, 36 bytes per 32 values, with one thread-block per 32
values; then a GEMM multiplies the Q4_K weight blocks by those Q8_1 blocks
with 8-bit integer dot products and writes fp32 [M][N].  The pages print
the launches, not the two kernels, so this module takes the plainest
reading of each:

Q8_1 block (the public GGML layout, 36 bytes): f16 ``d``, f16 ``s``, then
32 int8 quants ``q``, for 32 consecutive values x of one activation row:
    a  = max |x_i|                    (fp32; NaN ignored, as the path's absmax)
    d  = RN_f32(a / 127)
    id = RN_f32(1 / d), or 0 when d == 0
    q_i = the integer nearest to RN_f32(x_i * id), halves away from zero,
          clamped to [-127, 127]; a NaN product gives 0
    stored d = f16(d), s = f16(RN_f32(d * sum_i q_i))      (f16: to nearest even)
Blocks are row-major: row i of the activation is blocks i*(K/32) ...

GEMM: the product of the two dequantised tensors,
    y[i][j] = sum_k xq[i][k] * w[j][k]
with xq = f16(d) * q (the Q8_1 value) and w the exact Q4_K value
d4*sc*q4 - dmin*mn (as ``kquant``).  The ``s`` field is part of the format
but not needed by this definition (s is a rounded copy of d*sum q).

``bound`` is the error a GPU evaluation may have: the kernel sums, per
32-value sub-block, the exact integer dot products of the quants times
the weight's scale parts, so cancellation between the two parts of the
Q4_K value is not free; the bound is therefore taken against
T = sum_k |xq| * (|d4*sc*q4| + |dmin*mn|).
"""
from __future__ import annotations

import numpy as np

from . import kquant

QK8 = 32
Q8_1_BYTES = 36
U32 = 2.0 ** -24
U64 = 2.0 ** -53


def _rn32(v: np.ndarray) -> np.ndarray:
    """Round float64 values to fp32 (to nearest even)."""
    with np.errstate(all="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float32)


def quant_q8_1(x: np.ndarray) -> np.ndarray:
    """uint8 [m][K/32][36]: the Q8_1 blocks of fp32 x [m][K] (K % 32 == 0)."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    if k % QK8:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(m, k // QK8, QK8)
    ax = np.abs(xb)
    ax = np.where(np.isnan(ax), np.float32(0), ax)
    a = ax.max(axis=2)                                             # fp32, exact
    with np.errstate(all="ignore"):
        d = _rn32(a.astype(np.float64) / 127.0)                    # correctly rounded quotient
        idv = np.where(d != 0, _rn32(1.0 / d.astype(np.float64)), np.float32(0))
        v = _rn32(xb.astype(np.float64) * idv[..., None].astype(np.float64))  # one fp32 product
        r = np.where(v >= 0, np.floor(v.astype(np.float64) + 0.5), np.ceil(v.astype(np.float64) - 0.5))
        r = np.where(np.isnan(r), 0.0, r)
        q = np.clip(r, -127, 127).astype(np.int64)
        qsum = q.sum(axis=2)
        s32 = _rn32(d.astype(np.float64) * qsum.astype(np.float64))
        d16 = d.astype(np.float16)
        s16 = s32.astype(np.float16)
    out = np.empty((m, k // QK8, Q8_1_BYTES), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(m, k // QK8, 2)
    out[..., 2:4] = s16.view(np.uint8).reshape(m, k // QK8, 2)
    out[..., 4:] = q.astype(np.int8).view(np.uint8)
    return out


def fields(q8: np.ndarray):
    """(d f16 [m][nb], s f16 [m][nb], q int8 [m][nb][32]) of Q8_1 blocks."""
    q8 = np.ascontiguousarray(q8, dtype=np.uint8)
    d = q8[..., 0:2].copy().view(np.float16)[..., 0]
    s = q8[..., 2:4].copy().view(np.float16)[..., 0]
    q = q8[..., 4:].copy().view(np.int8)
    return d, s, q


def dequant_q8_1(q8: np.ndarray) -> np.ndarray:
    """float64 [m][K]: f16(d) * q, exact."""
    d, _, q = fields(q8)
    m, nb = d.shape
    return (d.astype(np.float64)[..., None] * q.astype(np.float64)).reshape(m, nb * QK8)


def weight_exact(blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    """float64 [n][k]: the exact Q4_K values d4*sc*q4 - dmin*mn (each term
    is exact in float64 and so is their difference: they span at most 50
    bits)."""
    d, dmin, sc, mn, q = kquant.q4k_parts(blocks)
    sub = kquant.q4k_subblock_of()
    with np.errstate(all="ignore"):
        w = d[:, None] * sc[:, sub].astype(np.float64) * q.astype(np.float64) \
            - dmin[:, None] * mn[:, sub].astype(np.float64)
    return w.reshape(n, k)


def weight_parts_abs(blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    """float64 [n][k]: |d4*sc*q4| + |dmin*mn| of every Q4_K weight, exact."""
    d, dmin, sc, mn, q = kquant.q4k_parts(blocks)
    sub = kquant.q4k_subblock_of()
    with np.errstate(all="ignore"):
        a = np.abs(d[:, None] * sc[:, sub].astype(np.float64) * q.astype(np.float64)) \
            + np.abs(dmin[:, None] * mn[:, sub].astype(np.float64))
    return a.reshape(n, k)


def gemm(q8: np.ndarray, blocks: np.ndarray, n: int, k: int, rows=None) -> np.ndarray:
    """float64 y [rows][n] = dequant(q8) @ w^T, w the exact Q4_K values
    (each product and the sum in float64)."""
    xq = dequant_q8_1(q8)
    if rows is not None:
        xq = xq[np.asarray(rows)]
    return xq @ weight_exact(blocks, n, k).T


def bound(q8: np.ndarray, blocks: np.ndarray, n: int, k: int, rows=None) -> np.ndarray:
    """Largest |y_gpu - gemm| (Q4_K weights): (gamma_{2K/32+2}(2^-24) +
    gamma_{2K}(2^-53)) * T with T = sum_k |xq| (|d4 sc q4| + |dmin mn|).

    A GPU that forms, per 32-value sub-block, the exact integer sums
    P = sum q4*q8 and S = sum q8, multiplies P by RN(f16(d8) * d4*sc) and S
    by the exact f16(d8) * dmin*mn, and adds the 2K/32 terms into one fp32
    accumulator with fused multiply-adds, makes at most one rounding in the
    scale product and one per accumulation."""
    xq = np.abs(dequant_q8_1(q8))
    if rows is not None:
        xq = xq[np.asarray(rows)]
    t = xq @ weight_parts_abs(blocks, n, k).T
    nterm = 2 * (k // QK8) + 2
    g32 = nterm * U32 / (1.0 - nterm * U32)
    g64 = 2 * k * U64 / (1.0 - 2 * k * U64)  # this oracle's float64 products and sums
    return (g32 + g64) * t
