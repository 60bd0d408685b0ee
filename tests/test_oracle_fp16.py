"""Pins for the oracle's FP16 cached-weight GEMM comparator (CPU only).

Conversion: hand-derived fp32 -> fp16 pairs (ties, overflow, subnormals,
signed zero) in golden/f16_convert_pins.txt, and torch's independent
float16 conversion on random values of every magnitude.  Weight pack: a
closed-form block whose fp32 value needs fp16 rounding.  GEMM: brute force
over Python Fractions, an identity weight, and the error bound against its
exact rational value.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp16_path, kquant


def test_conversion_golden_pins(golden):
    rows = list(golden("f16_convert_pins.txt"))
    assert len(rows) >= 25
    for a, b in rows:
        x = np.array([int(a, 16)], np.uint32).view(np.float32)
        with np.errstate(all="ignore"):
            got = int(fp16_path.to_f16(x).view(np.uint16)[0])
        assert got == int(b, 16), (a, b, hex(got))


def test_conversion_nan_stays_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    assert np.isnan(fp16_path.to_f16(x)).all()


def test_conversion_matches_torch():
    g = np.random.Generator(np.random.PCG64(77))
    # every magnitude from fp32 subnormals to beyond the fp16 range, both signs
    x = (np.exp2(g.uniform(-150, 17, size=400_000)) * g.choice([-1.0, 1.0], size=400_000)).astype(np.float32)
    with np.errstate(all="ignore"):
        ours = fp16_path.to_f16(x).view(np.uint16)
    theirs = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)


def test_pack_weight_rounds_the_fp32_value():
    # Q4_K block, d = 1 + 2^-10 (0x3C01), dmin = 0, every sub-block scale 63
    # (scale bytes: low 6 bits 63 for j < 4; j >= 4 low nibble 15 plus the top
    # bits 0b11 of scales[j-4]; the mins do not matter with dmin = 0), every
    # quant 15: w = 945 (1 + 2^-10) =
    # 945.9228515625 in fp32, exactly; fp16 has spacing 0.5 in [512, 1024), so
    # the cached value is 946.0.  Quant 1 gives 63.0615234375 -> spacing 2^-5
    # -> 63.0625.
    scales = bytes([0xFF, 0xFF, 0xFF, 0xFF, 0xC0, 0xC0, 0xC0, 0xC0, 0x0F, 0x0F, 0x0F, 0x0F])
    for q, want in ((15, 946.0), (1, 63.0625)):
        blk = np.zeros((1, 144), np.uint8)
        blk[0, 0:2] = np.array([0x3C01], np.uint16).view(np.uint8)
        blk[0, 4:16] = np.frombuffer(scales, np.uint8)
        blk[0, 16:144] = q | (q << 4)
        w32 = kquant.dequant(12, blk, 1, 256)
        assert (w32 == np.float32(63 * q * (1 + 2.0 ** -10))).all()
        w16 = fp16_path.pack_weight(12, blk, 1, 256)
        assert w16.dtype == np.float16 and w16.shape == (1, 256)
        assert (w16 == np.float16(want)).all()


def test_convert_act_pads_with_zero_rows():
    x = np.random.Generator(np.random.PCG64(3)).standard_normal((5, 256)).astype(np.float32)
    a = fp16_path.convert_act(x)
    assert a.shape == (16, 256) and a.dtype == np.float16
    assert (a[5:] == 0).all()
    np.testing.assert_array_equal(a[:5], x.astype(np.float16))


def _fr(v):
    return Fraction(float(v))


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 256, 0), (3, 4, 256, 1), (2, 3, 512, 2)])
def test_gemm_brute_force(m, n, k, seed):
    g = np.random.Generator(np.random.PCG64(100 + seed))
    a = np.zeros((fp16_path.pad_m(m), k), np.float16)
    a[:m] = (g.standard_normal((m, k)) * 30).astype(np.float16)
    w = (g.standard_normal((n, k)) * 1e-2).astype(np.float16)
    y = fp16_path.gemm(a, w, m)
    bd = fp16_path.bound(a, w, m)
    u = Fraction(1, 2 ** 24)
    for i in range(m):
        for j in range(n):
            exact = sum(_fr(a[i, t]) * _fr(w[j, t]) for t in range(k))
            sabs = sum(abs(_fr(a[i, t]) * _fr(w[j, t])) for t in range(k))
            # the oracle's float64 sum is within (K-1) 2^-53 sum|a w| of exact
            assert abs(_fr(y[i, j]) - exact) <= (k - 1) * Fraction(1, 2 ** 53) * sabs
            # the bound is (gamma_K(2u) + gamma_K(2^-53)) sum|a w|, exactly
            want = (2 * k * u / (1 - 2 * k * u) + k * Fraction(1, 2 ** 53) / (1 - k * Fraction(1, 2 ** 53))) * sabs
            assert abs(_fr(bd[i, j]) - want) <= want * Fraction(1, 2 ** 50)


def test_gemm_identity_weight():
    k, n, m = 256, 6, 4
    w = np.zeros((n, k), np.float16)
    w[np.arange(n), np.arange(n)] = 1.0
    a = np.zeros((16, k), np.float16)
    a[:m] = np.random.Generator(np.random.PCG64(8)).standard_normal((m, k)).astype(np.float16)
    np.testing.assert_array_equal(fp16_path.gemm(a, w, m), a[:m, :n].astype(np.float64))


def test_gemm_zero_and_extremes():
    k = 1024
    a = np.full((16, k), 65504.0, np.float16)
    w = np.full((2, k), -65504.0, np.float16)
    y = fp16_path.gemm(a, w, 1)
    assert y[0, 0] == -65504.0 * 65504.0 * k  # exact: 2^32-scale terms, 10 bits of count
    assert (fp16_path.gemm(np.zeros((16, k), np.float16), w, 16) == 0).all()
    assert (fp16_path.bound(np.zeros((16, k), np.float16), w, 16) == 0).all()


def double_rounding_block():
    """A Q4_K block whose sub-block 0 decodes to 37584 + 2^-13 exactly:
    d = 2088 (0x6814), dmin = -2^-13 (0x8800), sc_0 = 2, mn_0 = 1, quants 9.
    fp32 rounds it to 37584.0 (its ulp there is 2^-8), which is halfway
    between the fp16 neighbours 37568 and 37600 (spacing 32): to even gives
    37568 (0x7896).  One rounding straight from the exact value would give
    37600.  The other sub-blocks are 0 - (-2^-13) * 0 = 0."""
    blk = np.zeros((1, 144), np.uint8)
    blk[0, 0:2] = np.array([0x6814], np.uint16).view(np.uint8)
    blk[0, 2:4] = np.array([0x8800], np.uint16).view(np.uint8)
    blk[0, 4] = 2   # sc_0
    blk[0, 8] = 1   # mn_0
    blk[0, 16:48] = 9  # low nibbles of qs[0..31]: sub-block 0
    return blk


def test_pack_weight_rounds_twice_like_the_pages():
    blk = double_rounding_block()
    w32 = kquant.dequant(12, blk, 1, 256)
    assert (w32[0, :32] == np.float32(37584.0)).all() and (w32[0, 32:] == 0).all()
    w16 = fp16_path.pack_weight(12, blk, 1, 256)
    assert (w16[0, :32].view(np.uint16) == 0x7896).all()
    assert float(w16[0, 0]) == 37568.0
