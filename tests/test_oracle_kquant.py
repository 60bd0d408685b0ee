"""Pins for the oracle's Q4_K / Q6_K dequantisation (CPU only).

Layout pins are one-hot blocks whose expected values were worked out by hand
(tests/golden/q4k_layout_pins.txt, q6k_layout_pins.txt).  Rounding is pinned
by comparing with the exact rational value rounded once to fp32 by an
independent exact routine.  Sizes are pinned by the pages' bytes/weight.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import kquant
from tests.conftest import golden_lines


def _q4k_block(d=0x3C00, dmin=0x0000, scales=bytes(12), qs=bytes(128)):
    b = np.zeros(144, dtype=np.uint8)
    b[0:2] = np.array([d], dtype=np.uint16).view(np.uint8)
    b[2:4] = np.array([dmin], dtype=np.uint16).view(np.uint8)
    b[4:16] = np.frombuffer(bytes(scales), dtype=np.uint8)
    b[16:144] = np.frombuffer(bytes(qs), dtype=np.uint8)
    return b[None, :]


def _q6k_block(d=0x3C00, scales=None, ql=None, qh=None):
    b = np.zeros(210, dtype=np.uint8)
    b[0:128] = 0 if ql is None else np.frombuffer(bytes(ql), dtype=np.uint8)
    b[128:192] = 0 if qh is None else np.frombuffer(bytes(qh), dtype=np.uint8)
    b[192:208] = 1 if scales is None else np.array(scales, dtype=np.int8).view(np.uint8)
    b[208:210] = np.array([d], dtype=np.uint16).view(np.uint8)
    return b[None, :]


UNIT_SCALES = bytes([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1])


def test_sizes_match_pages():
    # 144 bytes per 256 weights = 0.5625 bytes per weight
    assert kquant.Q4_K_BYTES / kquant.QK_K == 0.5625
    assert kquant.weight_bytes(W.Q4_K, 256, 512) == 256 * 2 * 144
    assert kquant.weight_bytes(W.Q6_K, 512, 3584) == 512 * 14 * 210
    assert W.q4k_blocks(1, 4, 512).shape == (8, 144)
    assert W.q6k_blocks(1, 4, 512).shape == (8, 210)


@pytest.mark.parametrize("row", list(golden_lines("q4k_layout_pins.txt")))
def test_q4k_golden(row):
    kind = row[0]
    if kind == "quant_position":
        t, i_lo, i_hi = map(int, row[1:])
        qs = bytearray(128)
        qs[t] = 0x21
        got = kquant.dequant_q4k_blocks(_q4k_block(scales=UNIT_SCALES, qs=qs))[0]
        want = np.zeros(256, dtype=np.float32)
        want[i_lo] = 1.0
        want[i_hi] = 2.0
        np.testing.assert_array_equal(got, want)
    elif kind == "scale_fields":
        d, dmin, sc = int(row[1], 16), int(row[2], 16), bytes.fromhex(row[3])
        assert row[4] == ":"
        per_sub = [float(v) for v in row[5:13]]
        got = kquant.dequant_q4k_blocks(_q4k_block(d, dmin, sc, bytes([0x11] * 128)))[0]
        np.testing.assert_array_equal(got, np.repeat(np.array(per_sub, dtype=np.float32), 32))
    else:
        raise AssertionError(kind)


@pytest.mark.parametrize("row", list(golden_lines("q6k_layout_pins.txt")))
def test_q6k_golden(row):
    kind = row[0]
    base = np.full(256, -32.0, dtype=np.float32)
    if kind == "low_bits":
        t, e1, e2 = map(int, row[1:])
        ql = bytearray(128)
        ql[t] = 0x21
        got = kquant.dequant_q6k_blocks(_q6k_block(ql=ql))[0]
        base[e1], base[e2] = -31.0, -30.0
    elif kind == "high_bits":
        u, e16, e32, e48 = map(int, row[1:])
        qh = bytearray(64)
        qh[u] = 0xE4
        got = kquant.dequant_q6k_blocks(_q6k_block(qh=qh))[0]
        base[e16], base[e32], base[e48] = -16.0, 0.0, 16.0
    elif kind == "scale_index":
        s, first, last = map(int, row[1:])
        sc = [1] * 16
        sc[s] = -3
        got = kquant.dequant_q6k_blocks(_q6k_block(scales=sc))[0]
        base[first:last + 1] = 96.0
    elif kind == "uniform":
        d, scb, qlb, qhb = (int(v, 16) for v in row[1:5])
        assert row[5] == ":"
        sc = [np.uint8(scb).view(np.int8)] * 16
        got = kquant.dequant_q6k_blocks(_q6k_block(d=d, scales=sc, ql=bytes([qlb] * 128),
                                                    qh=bytes([qhb] * 64)))[0]
        base[:] = float(row[6])
    else:
        raise AssertionError(kind)
    np.testing.assert_array_equal(got, base)


# ------------------------------------------------------------ exact rounding

def _rn_f32(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even), by search.

    Independent of float64 arithmetic: brackets the value between adjacent
    fp32 numbers and compares exact distances.
    """
    if fr == 0:
        return np.float32(0.0)
    guess = np.float32(float(fr))  # within one fp32 ulp of the exact value
    cands = {guess, np.nextafter(guess, np.float32(np.inf)), np.nextafter(guess, np.float32(-np.inf))}
    best = None
    for c in cands:
        dist = abs(Fraction(float(c)) - fr)
        key = (dist, int(np.array([c], dtype=np.float32).view(np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _f16(bits):
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def test_q4k_is_correctly_rounded():
    blocks = W.q4k_blocks(11, 2, 512)
    got = kquant.dequant_q4k_blocks(blocks)
    for b in range(blocks.shape[0]):
        raw = blocks[b]
        d = _f16(int(raw[0]) | int(raw[1]) << 8)
        dmin = _f16(int(raw[2]) | int(raw[3]) << 8)
        sc = raw[4:16]
        for i in range(0, 256, 7):
            j = i // 32
            if j < 4:
                s, m = int(sc[j]) & 63, int(sc[j + 4]) & 63
            else:
                s = (int(sc[j + 4]) & 15) | ((int(sc[j - 4]) >> 6) << 4)
                m = (int(sc[j + 4]) >> 4) | ((int(sc[j]) >> 6) << 4)
            byte = int(raw[16 + 32 * (i // 64) + i % 32])
            q = byte & 15 if j % 2 == 0 else byte >> 4
            assert got[b, i] == _rn_f32(d * s * q - dmin * m)


def test_q6k_is_exact():
    blocks = W.q6k_blocks(12, 2, 512)
    got = kquant.dequant_q6k_blocks(blocks)
    for b in range(blocks.shape[0]):
        raw = blocks[b]
        d = _f16(int(raw[208]) | int(raw[209]) << 8)
        scl = raw[192:208].view(np.int8)
        for i in range(0, 256, 5):
            h, r = divmod(i, 128)
            p, l = divmod(r, 32)
            lo = int(raw[64 * h + l + 32 * (p & 1)])
            lo = lo & 15 if p < 2 else lo >> 4
            hi = (int(raw[128 + 32 * h + l]) >> (2 * p)) & 3
            exact = d * int(scl[8 * h + l // 16 + 2 * p]) * ((lo | hi << 4) - 32)
            assert Fraction(float(got[b, i])) == exact  # exact in fp32


def test_row_major_block_order():
    # row r of the [n][k] result is made of blocks r*(k/256) .. r*(k/256)+k/256-1
    blocks = W.q4k_blocks(3, 3, 768)
    full = kquant.dequant(W.Q4_K, blocks, 3, 768)
    for r in range(3):
        for c in range(3):
            one = kquant.dequant_q4k_blocks(blocks[r * 3 + c:r * 3 + c + 1])[0]
            np.testing.assert_array_equal(full[r, 256 * c:256 * (c + 1)], one)


def test_rejects_partial_superblocks():
    with pytest.raises(ValueError):
        kquant.dequant(W.Q4_K, W.q4k_blocks(1, 1, 256), 1, 300)
