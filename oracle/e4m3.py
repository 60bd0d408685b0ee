"""Oracle: FP32 -> FP8 E4M3 encoding and OCP E4M3FN decoding.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Encoder source: realizar 0.8.4, page ``cublas_prefill/mod.rs``, the inline
kernels ``F32_TO_E4M3_PTX`` (unscaled), ``F32_TO_E4M3_SCALED_PTX`` and
``F32_TO_E4M3_DEVICE_SCALED_PTX`` (which multiply by a scale first).  The
three share one bit-level conversion; stated in words it is:

* split the fp32 word into sign s (bit 31), exponent e (bits 30..23) and
  fraction f (bits 22..0);
* e == 0 (zero or fp32 subnormal) -> 0x00, whatever the sign;
* e == 255 (Inf or NaN) -> s<<7 | 0x7E (the largest finite code, 448);
* rebias: E = e - 127 + 7; E < 1 -> 0x00 (flush decided before rounding,
  so nothing below 2^-6 survives and the sign is dropped);
  E > 15 -> s<<7 | 0x7E;
* keep the top three fraction bits, round to nearest even on bit 19 with
  bits 18..0 as sticky; a carry out of the three bits bumps E, and E > 15
  after the carry saturates to s<<7 | 0x7E;
* pack s<<7 | E<<3 | m.

Reading taken where the listing and the format disagree: the listing would
emit 0x7F / 0xFF for results in (464, 496), which are NaN codes in E4M3FN.
Following the pages' own comment that non-finite and out-of-range values go
to the largest finite value, the oracle saturates E == 15, m == 7 to
s<<7 | 0x7E.  That band cannot be reached on the scaled path
(|x * RN(448/absmax)| <= 448.00003).

Scaled conversion (``F32_TO_E4M3_SCALED_PTX``, ``..._DEVICE_SCALED_PTX``):
the scale is applied as one IEEE fp32 multiply rounded to nearest (no fused
multiply-add).  A NaN produced by that multiply is the positive canonical
NaN, as the pages' target produces for every NaN result of an fp32 multiply;
it therefore encodes to 0x7E.

Decoder: the OCP 8-bit floating point E4M3FN definition (bias 7, no
infinities, S.1111.111 is NaN, subnormals m * 2^-9), which is the format the
pages' encoder targets (bias 7, largest finite 0x7E = 448).
"""
from __future__ import annotations

import numpy as np

MAX_FINITE_CODE = 0x7E
CANONICAL_NAN_BITS = 0x7FC00000


def encode_bits_scalar(u: int) -> int:
    """Encode one fp32 bit pattern (Python int) — the literal reference."""
    u &= 0xFFFFFFFF
    s = u >> 31
    e = (u >> 23) & 0xFF
    f = u & 0x7FFFFF
    if e == 0:
        return 0x00
    if e == 255:
        return (s << 7) | MAX_FINITE_CODE
    E = e - 120
    if E < 1:
        return 0x00
    if E > 15:
        return (s << 7) | MAX_FINITE_CODE
    m3 = f >> 20
    round_bit = (f >> 19) & 1
    sticky = f & 0x7FFFF
    if round_bit and (sticky != 0 or (m3 & 1)):
        m3 += 1
    if m3 == 8:
        m3 = 0
        E += 1
        if E > 15:
            return (s << 7) | MAX_FINITE_CODE
    if E == 15 and m3 == 7:  # 0x7F would be NaN in E4M3FN: saturate
        return (s << 7) | MAX_FINITE_CODE
    return (s << 7) | (E << 3) | m3


def f32_bits(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)


def encode_bits(u: np.ndarray) -> np.ndarray:
    """Vectorised encoder over a uint32 array of fp32 bit patterns.

    Must equal ``encode_bits_scalar`` element by element (pinned
    exhaustively over equivalence classes in the tests).
    """
    u = np.asarray(u, dtype=np.uint32)
    s = (u >> np.uint32(31)).astype(np.int32)
    e = ((u >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32)
    f = (u & np.uint32(0x7FFFFF)).astype(np.int32)
    E = e - 120
    m3 = f >> 20
    rbit = (f >> 19) & 1
    sticky = f & 0x7FFFF
    up = (rbit == 1) & ((sticky != 0) | ((m3 & 1) == 1))
    m3 = m3 + up.astype(np.int32)
    carry = m3 == 8
    m3 = np.where(carry, 0, m3)
    E = E + carry.astype(np.int32)
    packed = (s << 7) | (E << 3) | m3
    sat = (e == 255) | (E > 15) | ((E == 15) & (m3 == 7))
    zero = (e == 0) | ((e - 120) < 1)
    out = np.where(sat, (s << 7) | MAX_FINITE_CODE, packed)
    out = np.where(zero, 0, out)
    return out.astype(np.uint8)


def scaled_product(x: np.ndarray, scale) -> np.ndarray:
    """RN_f32(x * scale) with NaN results replaced by the canonical +NaN."""
    x = np.asarray(x, dtype=np.float32)
    sc = np.float32(scale)
    with np.errstate(all="ignore"):
        y = (x.astype(np.float64) * np.float64(sc)).astype(np.float32)
    y = np.ascontiguousarray(y)
    yb = y.view(np.uint32).copy()
    yb[np.isnan(y)] = CANONICAL_NAN_BITS
    return yb.view(np.float32)


def encode_scaled(x: np.ndarray, scale) -> np.ndarray:
    """E4M3 bytes of RN_f32(x * scale) (the scaled conversion kernels)."""
    return encode_bits(f32_bits(scaled_product(x, scale)))


# ---------------------------------------------------------------- decoding

def decode_scalar(b: int) -> float:
    """OCP E4M3FN decode of one byte to a Python float (NaN for 0x7F/0xFF)."""
    b &= 0xFF
    s = -1.0 if b & 0x80 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def decode_int_table() -> np.ndarray:
    """int64[256]: every code's value times 2^9 (an integer); NaN codes -> 0.

    The GEMM oracle works on these integers so that its sums are exact.
    """
    t = np.zeros(256, dtype=np.int64)
    for b in range(256):
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 15 and m == 7:
            t[b] = 0
            continue
        mag = m if e == 0 else (8 + m) << (e - 1)
        t[b] = -mag if b & 0x80 else mag
    return t


def decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of E4M3FN codes (NaN codes decode to NaN)."""
    codes = np.asarray(codes, dtype=np.uint8)
    v = decode_int_table()[codes].astype(np.float64) * 2.0 ** -9
    nan = ((codes & 0x7F) == 0x7F)
    v[nan] = np.nan
    return v
