"""Oracle: absmax, scales, weight packing, activation quantisation, FP8 GEMM.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (realizar 0.8.4):
* page ``cublas_prefill/gemm.rs``, ``get_or_cache_fp8_weight`` — a weight is
  dequantised to fp32, reduced to its absolute maximum, a zero maximum is
  replaced by 1, the quantisation scale is 448/absmax and the dequantisation
  scale absmax/448, and every element is encoded to E4M3 after multiplying by
  the quantisation scale;
* page ``cublas_prefill/gemm.rs``, ``cublas_prefill_fp8_gemm`` — the
  activation (only its m*k real elements) is reduced and encoded the same
  way on the device, M is padded to a multiple of 16, the GEMM computes raw
  FP8 dot products and the output is multiplied by
  (act_absmax/448)*(w_absmax/448); the same FP8 activation serves every
  GEMM that reads the same input;
* page ``cublas_prefill/mod.rs``, ``ABSMAX_REDUCE_PTX`` — absmax is the
  maximum of |x| (a float max that ignores NaN; -0 counts as 0), and
  ``F32_TO_E4M3_DEVICE_SCALED_PTX`` — the device computes 448/absmax and
  absmax/448 with IEEE round-to-nearest division after replacing 0 by 1.

Readings taken (the pages are silent or the build's contract overrides):
* pad rows m..m_pad-1 of the FP8 activation are 0x00;
* the GEMM accumulates and emits fp32 (no fp16 output stage);
* the product is  y = acc * dq_act * dq_w  with acc the exact sum of the
  decoded FP8 products; the GPU may round in any order within ``bound``.
"""
from __future__ import annotations

import numpy as np

from . import e4m3, kquant

FP8_MAX = 448.0


def pad_m(m: int) -> int:
    """M rounded up to a multiple of 16 (the FP8 GEMM's M alignment)."""
    return (m + 15) & ~15


def absmax_bits(x: np.ndarray) -> int:
    """fp32 bit pattern of max |x| over all elements; NaN ignored, -0 is 0.

    Done as an integer max over (bits & 0x7FFFFFFF) of the non-NaN elements;
    for non-negative floats the integer order equals the float order.
    """
    u = e4m3.f32_bits(np.asarray(x, dtype=np.float32).ravel()) & np.uint32(0x7FFFFFFF)
    u = u[u <= np.uint32(0x7F800000)]
    return int(u.max()) if u.size else 0


def absmax(x: np.ndarray) -> np.float32:
    return np.array([absmax_bits(x)], dtype=np.uint32).view(np.float32)[0]


def scales_from_absmax(a) -> tuple[np.float32, np.float32]:
    """(q, dq) = (RN_f32(448/a'), RN_f32(a'/448)), a' = a or 1 when a == 0.

    float64 division followed by one rounding to fp32 equals the correctly
    rounded fp32 quotient (53 >= 2*24 + 2).
    """
    a = np.float32(a)
    ap = np.float32(1.0) if a == 0 else a
    with np.errstate(all="ignore"):
        q = np.float32(np.float64(FP8_MAX) / np.float64(ap))
        dq = np.float32(np.float64(ap) / np.float64(FP8_MAX))
    return q, dq


def pack_weight(qtype: int, blocks: np.ndarray, n: int, k: int):
    """(w_fp8 uint8 [n][k], dq_w f32, absmax f32) for a K-quant weight."""
    w = kquant.dequant(qtype, blocks, n, k)
    a = absmax(w)
    q, dq = scales_from_absmax(a)
    return e4m3.encode_scaled(w, q).reshape(n, k), dq, a


def quant_act(x: np.ndarray):
    """(a_fp8 uint8 [pad_m(m)][k], absmax f32, dq_act f32) for fp32 x [m][k]."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    a = absmax(x)
    q, dq = scales_from_absmax(a)
    out = np.zeros((pad_m(m), k), dtype=np.uint8)
    out[:m] = e4m3.encode_scaled(x, q).reshape(m, k)
    return out, a, dq


def gemm_acc_int(a_fp8: np.ndarray, w_fp8: np.ndarray) -> np.ndarray:
    """Exact acc * 2^18 as float64 [Ma][N] (integer valued).

    Each decoded code times 2^9 is an integer of magnitude <= 229376, so each
    product is below 2^35.6 and any sum over K <= 2^14.3 terms stays below
    2^50 < 2^53: the float64 matmul is exact in any summation order.
    """
    t = e4m3.decode_int_table().astype(np.float64)
    A = t[np.asarray(a_fp8, dtype=np.uint8)]
    W = t[np.asarray(w_fp8, dtype=np.uint8)]
    return A @ W.T


def gemm_abs_int(a_fp8: np.ndarray, w_fp8: np.ndarray) -> np.ndarray:
    """sum_k |a_k w_k| * 2^18 as float64 [Ma][N] (exact, integer valued)."""
    t = np.abs(e4m3.decode_int_table()).astype(np.float64)
    A = t[np.asarray(a_fp8, dtype=np.uint8)]
    W = t[np.asarray(w_fp8, dtype=np.uint8)]
    return A @ W.T


def gemm(a_fp8: np.ndarray, w_fp8: np.ndarray, m: int, dq_act, dq_w) -> np.ndarray:
    """float64 y [m][N] = (sum_k dec(a)dec(w)) * dq_act * dq_w (exact sum)."""
    acc = gemm_acc_int(np.asarray(a_fp8)[:m], w_fp8)
    return acc * 2.0 ** -18 * np.float64(np.float32(dq_act)) * np.float64(np.float32(dq_w))


def bound(a_fp8: np.ndarray, w_fp8: np.ndarray, m: int, dq_act, dq_w,
          rel: float = 2e-3) -> np.ndarray:
    """Per-element tolerance rel * dq_act * dq_w * sum_k |dec(a_k) dec(w_k)|."""
    s = gemm_abs_int(np.asarray(a_fp8)[:m], w_fp8)
    return rel * s * 2.0 ** -18 * np.float64(np.float32(dq_act)) * np.float64(np.float32(dq_w))


def gemm_rows(a_fp8: np.ndarray, w_fp8: np.ndarray, rows, dq_act, dq_w):
    """(y_ref, tol) restricted to the given activation rows (sampled check)."""
    A = np.asarray(a_fp8)[np.asarray(rows)]
    y = gemm_acc_int(A, w_fp8) * 2.0 ** -18 * np.float64(np.float32(dq_act)) * np.float64(np.float32(dq_w))
    tol = bound(A, w_fp8, A.shape[0], dq_act, dq_w)
    return y, tol
