"""Pins for the oracle's direct K-quant GEMV (CPU only).

Closed forms on blocks built so that every weight is known without the
oracle's dequant (uniform quants, one scale per sub-block or scale group),
indicator inputs that pick one sub-block or scale group, exact linearity in
x, one-hot inputs against the independently pinned dequant, and the fp32
error bound against simulated fp32 accumulation in several orders.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import kquant, kquant_gemv

F16_ONE, F16_HALF, F16_QUARTER = 0x3C00, 0x3800, 0x3400


def _q4k_blocks(nblocks, d=F16_ONE, dmin=0, scales=bytes(12), q=0):
    b = np.zeros((nblocks, 144), dtype=np.uint8)
    b[:, 0:2] = np.array([d], dtype=np.uint16).view(np.uint8)
    b[:, 2:4] = np.array([dmin], dtype=np.uint16).view(np.uint8)
    b[:, 4:16] = np.frombuffer(bytes(scales), dtype=np.uint8)
    b[:, 16:144] = q | (q << 4)  # every 4-bit quant of the block is q
    return b


def _q6k_blocks(nblocks, d=F16_ONE, scales=None):
    b = np.zeros((nblocks, 210), dtype=np.uint8)
    b[:, 0:128] = 0x77   # low 4 bits of every quant: 7
    b[:, 128:192] = 0x55  # high 2 bits of every quant: 1  -> q = 23, q - 32 = -9
    b[:, 192:208] = np.array(scales, dtype=np.int8).view(np.uint8)
    b[:, 208:210] = np.array([d], dtype=np.uint16).view(np.uint8)
    return b


def test_q4k_uniform_rows_closed_form():
    # row j: every weight is d*s*q_j - dmin*t with s = 3, t = 2 in all eight
    # sub-blocks (scale bytes below 16: no high bits), d = 1/2, dmin = 1/4
    n, k = 5, 512
    scales = bytes([3, 3, 3, 3, 2, 2, 2, 2, 3 | (2 << 4), 3 | (2 << 4), 3 | (2 << 4), 3 | (2 << 4)])
    rows = [_q4k_blocks(k // 256, d=F16_HALF, dmin=F16_QUARTER, scales=scales, q=j + 1) for j in range(n)]
    blocks = np.concatenate(rows)
    g = np.random.Generator(np.random.PCG64(5))
    x = g.integers(-8, 9, size=(3, k)).astype(np.float32)
    y = kquant_gemv.gemv(12, blocks, n, k, x)
    w = np.array([0.5 * 3 * (j + 1) - 0.25 * 2 for j in range(n)])
    expect = x.astype(np.float64).sum(axis=1)[:, None] * w[None, :]
    assert y.shape == (3, n)
    np.testing.assert_array_equal(y, expect)


def test_q4k_subblock_order_closed_form():
    # sc_j = 1, 2, 3, 4 for sub-blocks 0..3 (scales[j] & 63) and 5 for 4..7
    # (scales[j+4] & 15, high bits of scales[j-4] zero); m_j = 0; q = 3:
    # sub-block j of a block covers elements 32j..32j+31
    scales = bytes([1, 2, 3, 4, 0, 0, 0, 0, 5, 5, 5, 5])
    sc = [1, 2, 3, 4, 5, 5, 5, 5]
    k = 512
    blocks = _q4k_blocks(k // 256, d=F16_ONE, scales=scales, q=3)
    x = np.zeros((16, k), np.float32)
    for b in range(2):
        for j in range(8):
            x[8 * b + j, 256 * b + 32 * j: 256 * b + 32 * j + 32] = 1.0
    y = kquant_gemv.gemv(12, blocks, 1, k, x)
    expect = np.array([32.0 * sc[j] * 3 for b in range(2) for j in range(8)])[:, None]
    np.testing.assert_array_equal(y, expect)


def test_q6k_scale_group_order_closed_form():
    # q = 23 everywhere, scale group g = g - 8 over elements 16g..16g+15
    # (its scale index 8h + l//16 + 2p equals i // 16), d = 1/2
    scales = [g - 8 for g in range(16)]
    k = 256
    blocks = _q6k_blocks(1, d=F16_HALF, scales=scales)
    x = np.zeros((16, k), np.float32)
    for g in range(16):
        x[g, 16 * g: 16 * g + 16] = 1.0
    y = kquant_gemv.gemv(14, blocks, 1, k, x)
    expect = np.array([16 * 0.5 * (g - 8) * -9.0 for g in range(16)])[:, None]
    np.testing.assert_array_equal(y, expect)


@pytest.mark.parametrize("qtype", [12, 14])
def test_linear_in_x(qtype):
    # integer weights (d = 1, dmin = 0) and small integer inputs: every sum is
    # exact in float64, so y(x1 + x2) == y(x1) + y(x2) bit for bit
    n, k = 7, 768
    g = np.random.Generator(np.random.PCG64(11 + qtype))
    nb = n * (k // 256)
    if qtype == 12:
        blocks = g.integers(0, 256, size=(nb, 144), dtype=np.uint8)
        blocks[:, 0:2] = np.array([F16_ONE], np.uint16).view(np.uint8)
        blocks[:, 2:4] = 0
    else:
        blocks = g.integers(0, 256, size=(nb, 210), dtype=np.uint8)
        blocks[:, 208:210] = np.array([F16_ONE], np.uint16).view(np.uint8)
    x1 = g.integers(-4, 5, size=(3, k)).astype(np.float32)
    x2 = g.integers(-4, 5, size=(3, k)).astype(np.float32)
    y1 = kquant_gemv.gemv(qtype, blocks, n, k, x1)
    y2 = kquant_gemv.gemv(qtype, blocks, n, k, x2)
    y12 = kquant_gemv.gemv(qtype, blocks, n, k, x1 + x2)
    np.testing.assert_array_equal(y12, y1 + y2)
    np.testing.assert_array_equal(kquant_gemv.gemv(qtype, blocks, n, k, 2 * x1), 2 * y1)


@pytest.mark.parametrize("qtype", [12, 14])
def test_one_hot_inputs_select_weight_columns(qtype):
    # x = unit vector e_c gives y[:, j] = w[j][c] (columns of the weight, not rows)
    n, k = 6, 512
    g = np.random.Generator(np.random.PCG64(21 + qtype))
    nb = n * (k // 256)
    per = 144 if qtype == 12 else 210
    blocks = g.integers(0, 256, size=(nb, per), dtype=np.uint8)
    if qtype == 12:
        blocks[:, 0:4] = np.array([0x2E66, 0x2A00], np.uint16).view(np.uint8)
    else:
        blocks[:, 208:210] = np.array([0x2E66], np.uint16).view(np.uint8)
    cols = [0, 1, 31, 32, 255, 256, 300, 511]
    x = np.zeros((len(cols), k), np.float32)
    x[np.arange(len(cols)), cols] = 1.0
    y = kquant_gemv.gemv(qtype, blocks, n, k, x)
    w = kquant.dequant(qtype, blocks, n, k).astype(np.float64)
    np.testing.assert_array_equal(y, w[:, cols].T)


@pytest.mark.parametrize("qtype", [12, 14])
def test_bound_covers_fp32_accumulation(qtype):
    # fp32 sums in three orders (forward, backward, pairwise) stay within the bound
    n, k = 8, 3584
    g = np.random.Generator(np.random.PCG64(31 + qtype))
    nb = n * (k // 256)
    per = 144 if qtype == 12 else 210
    blocks = g.integers(0, 256, size=(nb, per), dtype=np.uint8)
    if qtype == 12:
        blocks[:, 0:4] = np.array([0x2266, 0x1E00], np.uint16).view(np.uint8)
    else:
        blocks[:, 208:210] = np.array([0x2266], np.uint16).view(np.uint8)
    x = g.standard_normal((2, k)).astype(np.float32)
    y = kquant_gemv.gemv(qtype, blocks, n, k, x)
    bd = kquant_gemv.bound(qtype, blocks, n, k, x)
    w = kquant.dequant(qtype, blocks, n, k)
    for i in range(2):
        for j in range(n):
            prods = (x[i].astype(np.float64) * w[j].astype(np.float64)).astype(np.float32)
            fwd = np.float32(0)
            for p in prods:
                fwd = np.float32(fwd + p)
            bwd = np.float32(0)
            for p in prods[::-1]:
                bwd = np.float32(bwd + p)
            pw = prods.copy()
            while pw.size > 1:
                if pw.size % 2:
                    pw = np.append(pw, np.float32(0))
                pw = (pw[0::2] + pw[1::2]).astype(np.float32)
            for s in (fwd, bwd, pw[0]):
                assert abs(float(s) - y[i, j]) <= bd[i, j]
    assert (bd > 0).all()


def test_rejects_bad_shapes():
    blocks = _q4k_blocks(1)
    with pytest.raises(ValueError):
        kquant_gemv.gemv(12, blocks, 1, 300, np.zeros((1, 300), np.float32))
    with pytest.raises(ValueError):
        kquant_gemv.gemv(12, blocks, 1, 256, np.zeros((1, 512), np.float32))


def test_bound_equals_gamma_times_abs_sum_exactly():
    # The bound is gamma_K * sum_k |x_k w_k| with gamma_K = K u / (1 - K u),
    # u = 2^-24.  Here every weight is known in closed form (uniform quants:
    # w = d*s*q_j - dmin*t per row, as in the closed-form test above), so the
    # exact rational value is computed without the oracle's dequant and the
    # float64 result must equal it up to float64 rounding: a bound that is
    # too loose (or too tight) by any factor fails.
    n, k = 4, 768
    scales = bytes([3, 3, 3, 3, 2, 2, 2, 2, 3 | (2 << 4), 3 | (2 << 4), 3 | (2 << 4), 3 | (2 << 4)])
    rows = [_q4k_blocks(k // 256, d=F16_HALF, dmin=F16_QUARTER, scales=scales, q=j) for j in range(n)]
    blocks = np.concatenate(rows)
    g = np.random.Generator(np.random.PCG64(41))
    x = g.standard_normal((2, k)).astype(np.float32)
    bd = kquant_gemv.bound(12, blocks, n, k, x)
    u = Fraction(1, 2 ** 24)
    gamma = k * u / (1 - k * u)
    for i in range(2):
        sx = sum(abs(Fraction(float(v))) for v in x[i])
        for j in range(n):
            wj = Fraction(1, 2) * 3 * j - Fraction(1, 4) * 2  # every weight of row j
            exact = gamma * sx * abs(wj)
            assert abs(Fraction(float(bd[i, j])) - exact) <= exact * Fraction(1, 2 ** 50), (i, j)
    # row 0 has w = -1/2 everywhere: nonzero bound; a zero activation row gives 0
    assert (bd > 0).all()
    assert (kquant_gemv.bound(12, blocks, n, k, np.zeros((1, k), np.float32)) == 0).all()
