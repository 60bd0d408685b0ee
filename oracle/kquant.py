"""Oracle: Q4_K / Q6_K super-block dequantisation to fp32.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages (realizar 0.8.4, ``cublas_prefill/gemm.rs``: ``launch_dequant_q4k``,
``launch_dequant_q6k``, ``dequant_q4k_to_scratch``, ``dequant_q6k_to_scratch``)
launch generated dequant kernels whose bodies they do not print; they fix
only that a weight [N][K] is stored as N*(K/256) super-blocks of 256 values,
row-major (one launch row per output row, one column per super-block), that
a Q4_K super-block is 144 bytes, and that the result is fp32 [N][K]
row-major.  The field layout and value formula below are the public GGUF
K-quant definitions (reading taken; compatibility with real GGUF files is
parity unpinned because no GGUF file is available).

Q4_K (144 bytes): f16 d | f16 dmin | scales[12] | qs[128].
  Element i (0..255) lies in sub-block j = i // 32.  Its 4-bit quant q is
  the low nibble of qs[32*(i//64) + i%32] for even j, the high nibble for
  odd j.  The 6-bit scale/min (sc_j, m_j) are packed in scales[]:
    j < 4 : sc = scales[j] & 63,  m = scales[j+4] & 63
    j >= 4: sc = (scales[j+4] & 15) | (scales[j-4] >> 6) << 4
            m  = (scales[j+4] >> 4) | (scales[j]   >> 6) << 4
  value = d*sc*q - dmin*m.

Q6_K (210 bytes): ql[128] | qh[64] | scales[16] (int8) | f16 d.
  Element i: half h = i // 128, r = i % 128, part p = r // 32, l = r % 32.
  The low 4 bits come from ql[64h + l + 32*(p & 1)] (low nibble for p < 2,
  high nibble for p >= 2), the high 2 bits from bits 2p..2p+1 of
  qh[32h + l]; q = low | high << 4 (0..63).  The scale is
  scales[8h + l//16 + 2p].  value = d*sc*(q - 32).

Exactness: every product above is exact in fp32 and float64 (Q4_K: d*sc*q
has at most 21 significant bits and dmin*m at most 17; Q6_K: d*sc*(q-32) at
most 24), and the Q4_K difference spans at most 50 bits, so computing in
float64 and rounding once gives the correctly rounded fp32 value; any
evaluation order on the GPU gives that same value.
"""
from __future__ import annotations

import numpy as np

QK_K = 256
Q4_K_BYTES = 144
Q6_K_BYTES = 210


def _f16_at(blocks: np.ndarray, off: int) -> np.ndarray:
    return np.ascontiguousarray(blocks[:, off:off + 2]).view(np.float16)[:, 0].astype(np.float64)


def q4k_scale_min(scales: np.ndarray):
    """(sc, m) int64 arrays [nb, 8] from the 12 packed scale bytes [nb, 12]."""
    s = scales.astype(np.int64)
    sc = np.empty((s.shape[0], 8), dtype=np.int64)
    mn = np.empty((s.shape[0], 8), dtype=np.int64)
    for j in range(8):
        if j < 4:
            sc[:, j] = s[:, j] & 63
            mn[:, j] = s[:, j + 4] & 63
        else:
            sc[:, j] = (s[:, j + 4] & 15) | ((s[:, j - 4] >> 6) << 4)
            mn[:, j] = (s[:, j + 4] >> 4) | ((s[:, j] >> 6) << 4)
    return sc, mn


def q4k_quants(qs: np.ndarray) -> np.ndarray:
    """4-bit quants int64 [nb, 256] in element order from qs [nb, 128]."""
    q = qs.astype(np.int64)
    out = np.empty((q.shape[0], QK_K), dtype=np.int64)
    for i in range(QK_K):
        byte = q[:, 32 * (i // 64) + i % 32]
        out[:, i] = (byte & 15) if (i // 32) % 2 == 0 else (byte >> 4)
    return out


def dequant_q4k_blocks(blocks: np.ndarray) -> np.ndarray:
    """fp32 [nb, 256] from uint8 [nb, 144]."""
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, Q4_K_BYTES)
    d = _f16_at(blocks, 0)[:, None]
    dmin = _f16_at(blocks, 2)[:, None]
    sc, mn = q4k_scale_min(blocks[:, 4:16])
    q = q4k_quants(blocks[:, 16:144])
    sub = np.arange(QK_K) // 32
    with np.errstate(all="ignore"):
        val = d * sc[:, sub].astype(np.float64) * q.astype(np.float64) \
            - dmin * mn[:, sub].astype(np.float64)
    return val.astype(np.float32)


def q4k_parts(blocks: np.ndarray):
    """The fields of Q4_K blocks [nb, 144] as exact numbers: (d, dmin)
    float64 [nb], (sc, mn) int64 [nb, 8] per sub-block, q int64 [nb, 256];
    element i of a block is d*sc[i//32]*q[i] - dmin*mn[i//32]."""
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, Q4_K_BYTES)
    sc, mn = q4k_scale_min(blocks[:, 4:16])
    return _f16_at(blocks, 0), _f16_at(blocks, 2), sc, mn, q4k_quants(blocks[:, 16:144])


def q4k_subblock_of() -> np.ndarray:
    """Sub-block index (0..7) of each of the 256 elements of a super-block."""
    return np.arange(QK_K) // 32


def q6k_quants_scales(blocks: np.ndarray):
    """(q in 0..63, sub-block scale) int64 arrays [nb, 256] in element order."""
    ql = blocks[:, 0:128].astype(np.int64)
    qh = blocks[:, 128:192].astype(np.int64)
    scl = blocks[:, 192:208].view(np.int8).astype(np.int64)
    q = np.empty((blocks.shape[0], QK_K), dtype=np.int64)
    sc = np.empty((blocks.shape[0], QK_K), dtype=np.int64)
    for i in range(QK_K):
        h, r = divmod(i, 128)
        p, l = divmod(r, 32)
        lo_byte = ql[:, 64 * h + l + 32 * (p & 1)]
        lo = (lo_byte & 15) if p < 2 else (lo_byte >> 4)
        hi = (qh[:, 32 * h + l] >> (2 * p)) & 3
        q[:, i] = lo | (hi << 4)
        sc[:, i] = scl[:, 8 * h + l // 16 + 2 * p]
    return q, sc


def dequant_q6k_blocks(blocks: np.ndarray) -> np.ndarray:
    """fp32 [nb, 256] from uint8 [nb, 210]."""
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, Q6_K_BYTES)
    d = _f16_at(blocks, 208)[:, None]
    q, sc = q6k_quants_scales(blocks)
    with np.errstate(all="ignore"):
        val = d * sc.astype(np.float64) * (q - 32).astype(np.float64)
    return val.astype(np.float32)


def dequant(qtype: int, blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    """fp32 [n][k] row-major: row r holds super-blocks r*(k/256) .. +k/256."""
    if k % QK_K != 0:
        raise ValueError("k must be a multiple of 256")
    if qtype == 12:
        flat = dequant_q4k_blocks(blocks)
    elif qtype == 14:
        flat = dequant_q6k_blocks(blocks)
    else:
        raise ValueError(f"unsupported qtype {qtype}")
    if flat.shape[0] != n * (k // QK_K):
        raise ValueError("block count does not match n*(k/256)")
    return flat.reshape(n, k)


def weight_bytes(qtype: int, n: int, k: int) -> int:
    per = {12: Q4_K_BYTES, 14: Q6_K_BYTES}[qtype]
    return n * (k // QK_K) * per
