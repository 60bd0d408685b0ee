"""Pins for the oracle's absmax, scales, packing, activation quant and GEMM.

GEMM: brute force over Python Fractions on tiny shapes (the decoded values
come from torch's float8_e4m3fn, an independent decoder), an identity-like
weight, and all-zero inputs.  Scales: exact rational rounding.  Absmax:
fixed arrays and the invariant that the absmax element encodes to +-0x7E.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import e4m3, fp8_path, kquant
from tests.test_oracle_kquant import _rn_f32


def test_pad_m():
    assert [fp8_path.pad_m(m) for m in (1, 4, 15, 16, 17, 37, 1000, 2048)] == \
        [16, 16, 16, 16, 32, 48, 1008, 2048]


def test_absmax_fixed_cases():
    f = fp8_path.absmax
    assert f(np.array([-3.0, 2.0, 1.0], np.float32)) == 3.0
    assert f(np.array([-0.0, 0.0], np.float32)) == 0.0
    assert not np.signbit(f(np.array([-0.0], np.float32)))
    assert f(np.array([np.nan, -5.0, 4.0], np.float32)) == 5.0
    assert f(np.array([np.nan, np.nan], np.float32)) == 0.0
    assert f(np.array([1.0, -np.inf], np.float32)) == np.inf
    assert f(np.array([1e-40, -2e-40], np.float32)) == np.float32(2e-40)


@pytest.mark.parametrize("a", [448.0, 1.0, 0.0, 3.0, 1e-3, 7.5e-1, 12345.678, 2.0 ** -20])
def test_scales_exact_rounding(a):
    q, dq = fp8_path.scales_from_absmax(np.float32(a))
    ap = Fraction(float(np.float32(a))) if a != 0 else Fraction(1)
    assert q == _rn_f32(Fraction(448) / ap)
    assert dq == _rn_f32(ap / 448)


def test_scales_special():
    q, dq = fp8_path.scales_from_absmax(np.float32(448.0))
    assert q == 1.0 and dq == 1.0
    q, dq = fp8_path.scales_from_absmax(np.float32(0.0))
    assert q == 448.0 and dq == np.float32(1.0 / 448.0)
    q, dq = fp8_path.scales_from_absmax(np.float32(np.inf))
    assert q == 0.0 and dq == np.inf


def test_absmax_element_encodes_to_max_code():
    g = np.random.Generator(np.random.PCG64(5))
    a = np.exp2(g.uniform(-60, 60, size=20_000)).astype(np.float32)
    qs = np.array([fp8_path.scales_from_absmax(v)[0] for v in a], dtype=np.float32)
    for sgn, code in ((1.0, 0x7E), (-1.0, 0xFE)):
        codes = np.array([e4m3.encode_scaled(np.float32(sgn * v), q)[()] for v, q in zip(a, qs)])
        assert (codes == code).all()
        # and the product never exceeds 448.00004 (so the (464, 496) band is unreachable)
        prod = (sgn * a).astype(np.float64) * qs.astype(np.float64)
        assert np.abs(prod.astype(np.float32)).max() <= np.float32(448.00004)


def test_quant_act_pad_rows_zero_and_scales():
    x = W.act_normal(1, 5, 256)
    a8, amax, dq = fp8_path.quant_act(x)
    assert a8.shape == (16, 256)
    assert (a8[5:] == 0).all()
    assert amax == np.abs(x).max()
    q, dq2 = fp8_path.scales_from_absmax(amax)
    assert dq == dq2
    np.testing.assert_array_equal(a8[:5], e4m3.encode_scaled(x, q))
    # the largest element maps to +-448
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert a8[i] in (0x7E, 0xFE)


def test_quant_act_all_zero():
    a8, amax, dq = fp8_path.quant_act(np.zeros((3, 256), np.float32))
    assert amax == 0.0 and dq == np.float32(1.0 / 448.0)
    assert (a8 == 0).all()


def test_pack_weight_matches_steps():
    blocks = W.q4k_blocks(2, 4, 512)
    w8, dq, a = fp8_path.pack_weight(W.Q4_K, blocks, 4, 512)
    w = kquant.dequant(W.Q4_K, blocks, 4, 512)
    assert a == np.abs(w).max()
    assert dq == _rn_f32(Fraction(float(a)) / 448)
    assert w8.shape == (4, 512) and w8.dtype == np.uint8
    assert set(np.unique(w8[np.abs(w) == a]).tolist()) <= {0x7E, 0xFE}


def test_pack_zero_weight():
    blocks = np.zeros((2, 144), np.uint8)  # d = dmin = 0 -> all weights 0
    w8, dq, a = fp8_path.pack_weight(W.Q4_K, blocks, 1, 512)
    assert a == 0.0 and dq == np.float32(1 / 448) and (w8 == 0).all()


# ------------------------------------------------------------------- GEMM

def _torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 256, 0), (3, 5, 256, 1), (2, 4, 512, 2)])
def test_gemm_brute_force(m, n, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    a8 = g.choice(codes, size=(fp8_path.pad_m(m), k))
    w8 = g.choice(codes, size=(n, k))
    dqa, dqw = np.float32(0.37), np.float32(1.7e-3)
    y = fp8_path.gemm(a8, w8, m, dqa, dqw)
    A, Wd = _torch_decode(a8), _torch_decode(w8)
    for i in range(m):
        for j in range(n):
            s = sum(Fraction(float(A[i, t])) * Fraction(float(Wd[j, t])) for t in range(k))
            exact = s * Fraction(float(dqa)) * Fraction(float(dqw))
            # the oracle's sum is exact; its two scale multiplies round in float64
            assert abs(Fraction(float(y[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 51)
            tol = fp8_path.bound(a8, w8, m, dqa, dqw)
            sabs = sum(abs(Fraction(float(A[i, t])) * Fraction(float(Wd[j, t]))) for t in range(k))
            assert Fraction(float(tol[i, j])) == pytest.approx(
                float(Fraction(2, 1000) * sabs * Fraction(float(dqa)) * Fraction(float(dqw))), rel=1e-12)


def test_gemm_identity_weight():
    # W row j holds 0x38 (1.0) at column j, zeros elsewhere: y[i][j] = dec(a[i][j]) dqa dqw
    k, n, m = 256, 7, 5
    w8 = np.zeros((n, k), np.uint8)
    w8[np.arange(n), np.arange(n)] = 0x38
    g = np.random.Generator(np.random.PCG64(3))
    a8 = g.integers(0, 256, size=(16, k)).astype(np.uint8)
    a8[(a8 & 0x7F) == 0x7F] = 0
    y = fp8_path.gemm(a8, w8, m, 1.0, 1.0)
    np.testing.assert_array_equal(y, _torch_decode(a8[:m, :n]))


def test_gemm_extreme_sum_is_exact():
    # K = 18944 copies of 448*448: the largest sum the configurations can make
    k = 18944
    a8 = np.full((16, k), 0x7E, np.uint8)
    w8 = np.full((2, k), 0xFE, np.uint8)
    y = fp8_path.gemm(a8, w8, 1, 1.0, 1.0)
    assert y[0, 0] == -448.0 * 448.0 * k


def test_gemm_zero_rows_give_zero():
    a8 = np.zeros((16, 256), np.uint8)
    w8 = np.random.Generator(np.random.PCG64(4)).integers(0, 0x7F, size=(3, 256)).astype(np.uint8)
    assert (fp8_path.gemm(a8, w8, 16, 2.0, 3.0) == 0).all()
    assert (fp8_path.bound(a8, w8, 16, 2.0, 3.0) == 0).all()


def test_gemm_rows_selects_rows_of_full_gemm_and_bound():
    # gemm_rows serves every sampled-row GPU check: it must equal the pinned
    # full gemm/bound restricted to the requested rows, in the requested
    # order, for unsorted and repeated rows and for the last real row m-1.
    m, n, k = 37, 6, 512
    g = np.random.Generator(np.random.PCG64(9))
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    a8 = np.zeros((fp8_path.pad_m(m), k), np.uint8)
    a8[:m] = g.choice(codes, size=(m, k))
    w8 = g.choice(codes, size=(n, k))
    dqa, dqw = np.float32(0.011), np.float32(3.7e-4)
    full = fp8_path.gemm(a8, w8, m, dqa, dqw)
    tol_full = fp8_path.bound(a8, w8, m, dqa, dqw)
    rows = [m - 1, 3, 3, 0, 17, m - 1, 20]
    y, tol = fp8_path.gemm_rows(a8, w8, rows, dqa, dqw)
    assert y.shape == (len(rows), n) and tol.shape == (len(rows), n)
    np.testing.assert_array_equal(y, full[rows])
    np.testing.assert_array_equal(tol, tol_full[rows])
    # and a single row against brute force over Fractions (independent decoder)
    A, Wd = _torch_decode(a8), _torch_decode(w8)
    for j in range(n):
        s = sum(Fraction(float(A[m - 1, t])) * Fraction(float(Wd[j, t])) for t in range(k))
        exact = s * Fraction(float(dqa)) * Fraction(float(dqw))
        assert abs(Fraction(float(y[0, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 51)
