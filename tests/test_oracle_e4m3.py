"""Pins for the oracle's E4M3 encoder and decoder (CPU only).

The encoder is pinned by hand-derived fixed points (tests/golden), by an
exhaustive sweep of its equivalence classes (scalar reference == vectorised),
by the decode->encode round trip over every code, and by a cross-check with
torch's independent float8_e4m3fn conversion in the normal range.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3
from tests.conftest import golden_lines


def _pins():
    return [(int(a, 16), int(b, 16)) for a, b in golden_lines("e4m3_encode_pins.txt")]


@pytest.mark.parametrize("bits,code", _pins())
def test_golden_scalar(bits, code):
    assert e4m3.encode_bits_scalar(bits) == code


def test_golden_vector():
    pins = _pins()
    u = np.array([p[0] for p in pins], dtype=np.uint32)
    want = np.array([p[1] for p in pins], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3.encode_bits(u), want)


def _class_representatives():
    """One word per (sign, exponent, top-4 fraction bits, sticky class).

    The encoder reads only the sign, the exponent, fraction bits 22..19 and
    whether bits 18..0 are non-zero; sticky representatives cover zero and
    the extremes of the non-zero range.
    """
    s = np.arange(2, dtype=np.uint32)[:, None, None, None]
    e = np.arange(256, dtype=np.uint32)[None, :, None, None]
    top = np.arange(16, dtype=np.uint32)[None, None, :, None]
    st = np.array([0, 1, 0x40000, 0x7FFFF], dtype=np.uint32)[None, None, None, :]
    u = (s << 31) | (e << 23) | (top << 19) | st
    return u.ravel()


def test_vector_equals_scalar_on_every_class():
    u = _class_representatives()
    vec = e4m3.encode_bits(u)
    ref = np.array([e4m3.encode_bits_scalar(int(x)) for x in u], dtype=np.uint8)
    np.testing.assert_array_equal(vec, ref)


def test_never_emits_nan_or_subnormal_or_negative_zero():
    codes = set(e4m3.encode_bits(_class_representatives()).tolist())
    assert 0x7F not in codes and 0xFF not in codes
    assert 0x80 not in codes
    assert not any(0x01 <= c <= 0x07 or 0x81 <= c <= 0x87 for c in codes)


def test_decode_matches_torch_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ov = np.array([e4m3.decode_scalar(b) for b in range(256)])
    nan = np.isnan(tv)
    assert (np.isnan(ov) == nan).all()
    np.testing.assert_array_equal(ov[~nan], tv[~nan])
    # the integer table is the same values times 2^9
    it = e4m3.decode_int_table().astype(np.float64) * 2.0 ** -9
    np.testing.assert_array_equal(it[~nan], tv[~nan])


def test_round_trip_all_finite_codes():
    finite = [b for b in range(256) if (b & 0x7F) != 0x7F]
    assert len(finite) == 254
    vals = np.array([e4m3.decode_scalar(b) for b in finite], dtype=np.float32)
    got = e4m3.encode_bits(e4m3.f32_bits(vals))
    for b, g in zip(finite, got.tolist()):
        flushed = (0x01 <= b <= 0x07) or (0x80 <= b <= 0x87)
        assert g == (0x00 if flushed else b), hex(b)
    assert sum(1 for b in finite if (0x01 <= b <= 0x07) or (0x80 <= b <= 0x87)) == 15


def test_torch_cross_check_normal_range():
    g = np.random.Generator(np.random.PCG64(7))
    mag = np.exp2(g.uniform(-6.0, np.log2(448.0), size=200_000)).astype(np.float32)
    x = np.where(g.integers(0, 2, size=mag.size) == 1, -mag, mag).astype(np.float32)
    ours = e4m3.encode_bits(e4m3.f32_bits(x))
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)


def test_scaled_product_is_single_rounding_and_canonical_nan():
    # x*q with both fp32 is exact in float64, so one cast is one rounding
    x = np.array([1.0000001, 3.3333333], dtype=np.float32)
    q = np.float32(1.1)
    want = np.array([np.float32(x[0]) * q, np.float32(x[1]) * q], dtype=np.float32)
    np.testing.assert_array_equal(e4m3.scaled_product(x, q), want)
    # a NaN result of the scaling multiply is +NaN -> 0x7E, whatever its origin
    x = np.array([np.inf, -np.inf, np.nan, -np.nan, -5.0, 5.0], dtype=np.float32)
    x_bits = e4m3.f32_bits(x).copy()
    x_bits[3] = 0xFFC00000
    x = x_bits.view(np.float32)
    codes = e4m3.encode_scaled(x, 0.0)
    np.testing.assert_array_equal(codes, np.array([0x7E, 0x7E, 0x7E, 0x7E, 0x00, 0x00], dtype=np.uint8))
    codes = e4m3.encode_scaled(x, 1.0)
    np.testing.assert_array_equal(codes, np.array([0x7E, 0xFE, 0x7E, 0x7E, 0xCA, 0x4A], dtype=np.uint8))
