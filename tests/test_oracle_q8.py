"""Pins for the oracle's integer path: Q8_1 activation quantisation and the
Q8_1 x Q4_K GEMM (CPU only).

Q8_1: blocks derived by hand (the scale 127/127 = 1 and 254/127 = 2 make
every quotient exact, so ties away from zero, clamping and NaN handling
show directly), the zero block, and invariants on random data (the largest
element maps to +-127, the dequantised value is within half a step, the
stored s is the f16 of d times the sum of the codes).  GEMM: brute force
over Python Fractions on weights known in closed form (uniform quants) and
on random blocks, and the error bound against its exact rational value.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import q8_path
from tests.test_oracle_kquant import _rn_f32

F16_ONE, F16_HALF, F16_QUARTER = 0x3C00, 0x3800, 0x3400


def _block(vals):
    x = np.zeros((1, 32), np.float32)
    x[0, :len(vals)] = vals
    return x


def _unpack(b):
    d = int(b[0]) | int(b[1]) << 8
    s = int(b[2]) | int(b[3]) << 8
    q = b[4:].view(np.int8).astype(int).tolist()
    return d, s, q


def test_q8_1_scale_one_ties_away_from_zero():
    # amax 127 -> d = 1, 1/d = 1: q = round-half-away(x)
    x = _block([127, 0.5, -0.5, 1.5, 2.5, -2.5, 63.49, -126.6, 0.49999997])
    d, s, q = _unpack(q8_path.quant_q8_1(x)[0, 0])
    assert d == F16_ONE
    assert q[:9] == [127, 1, -1, 2, 3, -3, 63, -127, 0] and q[9:] == [0] * 23
    assert s == 0x5410  # sum 65 = 1.015625 * 2^6


def test_q8_1_scale_two():
    # amax 254 -> d = 2, 1/d = 0.5 (exact): 3 -> 1.5 -> 2, 5 -> 2.5 -> 3, 1 -> 0.5 -> 1
    x = _block([-254, 3, 5, 1, -1, -3, 253, 0.9])
    d, s, q = _unpack(q8_path.quant_q8_1(x)[0, 0])
    assert d == 0x4000
    assert q[:8] == [-127, 2, 3, 1, -1, -2, 127, 0]  # 253 * 0.5 = 126.5 -> 127; 0.45 -> 0
    assert s == 0x4600  # 2 * (-127+2+3+1-1-2+127+0) = 2 * 3 = 6 = 1.5 * 2^2


def test_q8_1_zero_and_nan():
    d, s, q = _unpack(q8_path.quant_q8_1(np.zeros((1, 32), np.float32))[0, 0])
    assert (d, s) == (0, 0) and q == [0] * 32
    # NaN is ignored by the absmax and gives code 0
    x = _block([np.nan, 127, -64])
    d, s, q = _unpack(q8_path.quant_q8_1(x)[0, 0])
    assert d == F16_ONE and q[:3] == [0, 127, -64]
    # a block of NaN only is a zero block
    d, s, q = _unpack(q8_path.quant_q8_1(np.full((1, 32), np.nan, np.float32))[0, 0])
    assert (d, s) == (0, 0) and q == [0] * 32


def test_q8_1_block_layout_row_major():
    # row i, block b: values 32b..32b+31 of row i; every block gets its own scale
    x = np.zeros((2, 96), np.float32)
    x[0, 0], x[0, 32], x[0, 64], x[1, 95] = 127, 254, 508, -127
    q8 = q8_path.quant_q8_1(x)
    assert q8.shape == (2, 3, 36)
    ds = [[_unpack(q8[i, b])[0] for b in range(3)] for i in range(2)]
    assert ds == [[0x3C00, 0x4000, 0x4400], [0, 0, 0x3C00]]
    assert _unpack(q8[1, 2])[2][31] == -127


def test_q8_1_invariants_random():
    g = np.random.Generator(np.random.PCG64(12))
    x = (g.standard_t(3, size=(64, 512)) * np.exp2(g.uniform(-20, 20, size=(64, 1)))).astype(np.float32)
    q8 = q8_path.quant_q8_1(x)
    d16, s16, q = q8_path.fields(q8)
    xb = x.reshape(64, 16, 32)
    amax_idx = np.abs(xb).argmax(axis=2)
    qa = np.take_along_axis(q.astype(int), amax_idx[..., None], axis=2)[..., 0]
    sgn = np.sign(np.take_along_axis(xb, amax_idx[..., None], axis=2)[..., 0])
    assert (qa == 127 * sgn).all()                   # the largest element maps to +-127
    assert (np.abs(q.astype(int)) <= 127).all()
    # |x - d*q| <= d/2 (1 + 2^-20), d the unrounded fp32 scale (here: from the f16 d
    # within f16 precision): check against the fp32 quotient a/127
    d32 = (np.abs(xb).max(axis=2).astype(np.float64) / 127).astype(np.float32).astype(np.float64)
    err = np.abs(xb.astype(np.float64) - d32[..., None] * q)
    assert (err <= d32[..., None] * 0.5 * (1 + 2.0 ** -20)).all()
    # s = f16(RN32(d * sum q))
    for i, b in [(0, 0), (5, 7), (63, 15)]:
        want = _rn_f32(Fraction(float(d32[i, b])) * int(q[i, b].astype(int).sum()))
        assert s16[i, b] == np.float16(want)


def _q4k_uniform(nblocks, d=F16_ONE, dmin=0, scales=bytes(12), q=0):
    b = np.zeros((nblocks, 144), dtype=np.uint8)
    b[:, 0:2] = np.array([d], dtype=np.uint16).view(np.uint8)
    b[:, 2:4] = np.array([dmin], dtype=np.uint16).view(np.uint8)
    b[:, 4:16] = np.frombuffer(bytes(scales), dtype=np.uint8)
    b[:, 16:144] = q | (q << 4)
    return b


def test_gemm_closed_form_weights():
    # row j: every weight is 1/2*3*q_j - 1/4*2 (sc 3, mn 2 in all sub-blocks)
    n, k = 4, 512
    scales = bytes([3, 3, 3, 3, 2, 2, 2, 2, 3 | (2 << 4), 3 | (2 << 4), 3 | (2 << 4), 3 | (2 << 4)])
    blocks = np.concatenate([_q4k_uniform(k // 256, d=F16_HALF, dmin=F16_QUARTER, scales=scales, q=j + 2)
                             for j in range(n)])
    g = np.random.Generator(np.random.PCG64(4))
    x = g.standard_normal((3, k)).astype(np.float32)
    q8 = q8_path.quant_q8_1(x)
    y = q8_path.gemm(q8, blocks, n, k)
    bd = q8_path.bound(q8, blocks, n, k)
    d16, _, q = q8_path.fields(q8)
    for i in range(3):
        xs = sum(Fraction(float(d16[i, b])) * int(q[i, b, t]) for b in range(k // 32) for t in range(32))
        xa = sum(abs(Fraction(float(d16[i, b])) * int(q[i, b, t])) for b in range(k // 32) for t in range(32))
        for j in range(n):
            main, mn = Fraction(1, 2) * 3 * (j + 2), Fraction(1, 4) * 2
            exact = xs * (main - mn)
            assert abs(Fraction(float(y[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
            nterm = 2 * (k // 32) + 2
            u = Fraction(1, 2 ** 24)
            u64 = Fraction(1, 2 ** 53)
            want = (nterm * u / (1 - nterm * u) + 2 * k * u64 / (1 - 2 * k * u64)) * xa * (main + mn)
            assert abs(Fraction(float(bd[i, j])) - want) <= want * Fraction(1, 2 ** 50)


@pytest.mark.parametrize("seed", [0, 1])
def test_gemm_brute_force_random_blocks(seed):
    n, k, m = 3, 256, 2
    blocks = W.q4k_blocks(700 + seed, n, k)
    x = W.act_student_t(710 + seed, m, k)
    q8 = q8_path.quant_q8_1(x)
    y = q8_path.gemm(q8, blocks, n, k)
    d16, _, q = q8_path.fields(q8)
    # the Q4_K fields read straight from the bytes (public layout, as the
    # one-hot pins of the dequantisation fix it)
    for j in range(n):
        raw = blocks[j]
        d4 = Fraction(float(np.frombuffer(raw[0:2].tobytes(), np.float16)[0]))
        dm = Fraction(float(np.frombuffer(raw[2:4].tobytes(), np.float16)[0]))
        s = raw[4:16].astype(int)
        sc = [s[t] & 63 if t < 4 else (s[t + 4] & 15) | ((s[t - 4] >> 6) << 4) for t in range(8)]
        mn = [s[t + 4] & 63 if t < 4 else (s[t + 4] >> 4) | ((s[t] >> 6) << 4) for t in range(8)]
        qs = raw[16:144].astype(int)
        w = []
        for e in range(256):
            byte = qs[32 * (e // 64) + e % 32]
            q4 = byte & 15 if (e // 32) % 2 == 0 else byte >> 4
            w.append(d4 * sc[e // 32] * q4 - dm * mn[e // 32])
        for i in range(m):
            exact = sum(Fraction(float(d16[i, e // 32])) * int(q[i, e // 32, e % 32]) * w[e] for e in range(256))
            mag = sum(abs(Fraction(float(d16[i, e // 32])) * int(q[i, e // 32, e % 32]) * w[e]) for e in range(256))
            assert abs(Fraction(float(y[i, j])) - exact) <= 2 * k * Fraction(1, 2 ** 53) * (mag + abs(exact)) + \
                Fraction(1, 2 ** 90)


def test_rejects_ragged_k():
    with pytest.raises(ValueError):
        q8_path.quant_q8_1(np.zeros((1, 48), np.float32))
