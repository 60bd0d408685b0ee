"""GPU parity of the FP8 GEMM that makes the weight codes from the K-quant
blocks inside the kernel (rz_kquant_weight_scale + rz_kquant_fp8_gemm)
against the CPU oracle (needs an MI355X).

The weight scales must be bit-exact (the oracle's absmax of the exact
dequantisation and its correctly rounded 448/a', a'/448).  The output is
checked against the oracle's exact sum over the oracle's packed codes
(oracle.fp8_path.gemm on oracle.fp8_path.pack_weight), within the same
per-element bound as the cached path's GEMM: the codes are the pack's bytes,
so the only freedom is the order of the fp32 accumulation.
"""
import numpy as np
import pytest

import workloads as W
from oracle import fp8_path

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rz():
    import fp8_prefill_gemm_amd as rz
    rz.lib()  # loud failure if the HIP library is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return rz


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(x):
    return np.float32(x).view(np.uint32)


def scales_match(rz, qtype, blocks, n, k):
    q, dq, a = rz.rz_kquant_weight_scale(qtype, dev(blocks), n, k)
    w8, rdq, ra = fp8_path.pack_weight(qtype, blocks, n, k)
    rq, rdq2 = fp8_path.scales_from_absmax(ra)
    assert bits(a) == bits(ra) and bits(q) == bits(rq) and bits(dq) == bits(rdq) == bits(rdq2)
    return q, dq, w8, rdq


def run(rz, qtype, blocks, n, k, x):
    m = x.shape[0]
    print(f"kquant_fp8_gemm qtype={qtype} m={m} n={n} k={k}", flush=True)
    q, dq, w8, rdq = scales_match(rz, qtype, blocks, n, k)
    a8, sc = rz.rz_fp8_quant_act(dev(x))
    r8, _, rdqa = fp8_path.quant_act(x)
    np.testing.assert_array_equal(host(a8), r8)
    y = rz.rz_kquant_fp8_gemm(a8, m, sc, qtype, dev(blocks), n, k, q, dq)
    return host(y), r8, w8, rdqa, rdq, (a8, sc, q, dq)


def check(y, a8, w8, m, dqa, dqw):
    yr = fp8_path.gemm(a8, w8, m, dqa, dqw)
    tol = fp8_path.bound(a8, w8, m, dqa, dqw)
    err = np.abs(y.astype(np.float64) - yr)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} elements out of bound; worst {err[bad].max()} at {np.argwhere(bad)[0]}"
    assert (y[tol == 0] == 0).all()


@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
@pytest.mark.parametrize("n,k", [(8, 256), (128, 512), (1, 256), (384, 2304)])
def test_weight_scale_bit_exact(rz, qtype, n, k):
    scales_match(rz, qtype, W.weight_blocks(qtype, 8100 + n + k, n, k), n, k)


def test_weight_scale_zero_weight(rz):
    # absmax 0 -> a' = 1: q = RN(448), dq = RN(1/448)
    n, k = 64, 512
    blocks = W.weight_blocks(W.Q4_K, 8150, n, k)
    blocks[:] = 0
    q, dq, a = rz.rz_kquant_weight_scale(W.Q4_K, dev(blocks), n, k)
    assert a == 0.0 and q == 448.0 and bits(dq) == bits(np.float32(1.0 / 448.0))


# several tiles in both directions with ragged tails (n and m not multiples
# of 128, m not a multiple of 16), one and several super-blocks; padded
# m >= 512 takes the 256-row tiles (1000 x 4100: 4 x 33 of them, ragged in
# both directions), smaller m the 128-row tiles
@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
@pytest.mark.parametrize("m,n,k", [(16, 256, 512), (1, 64, 256), (37, 200, 768), (130, 129, 512),
                                   (300, 520, 1024), (257, 384, 2304), (600, 1000, 512),
                                   (1000, 520, 768), (496, 260, 256), (1000, 4100, 256)])
def test_parity_shapes(rz, qtype, m, n, k):
    blocks = W.weight_blocks(qtype, 8200 + n + m, n, k)
    x = W.act_student_t(8300 + m + k, m, k)
    y, a8, w8, dqa, dqw, _ = run(rz, qtype, blocks, n, k, x)
    assert y.shape == (m, n)
    check(y, a8, w8, m, dqa, dqw)


@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
def test_matches_cached_path(rz, qtype):
    # the same product through the pack and the FP8 GEMM: both within the
    # bound of the oracle, and within twice that bound of each other
    m, n, k = 512, 640, 1024
    blocks = W.weight_blocks(qtype, 8400 + qtype, n, k)
    x = W.act_normal(8401, m, k)
    y, a8h, w8, dqa, dqw, (a8, sc, q, dq) = run(rz, qtype, blocks, n, k, x)
    w8d, scale, _ = rz.rz_fp8_pack_weight(qtype, dev(blocks), n, k)
    assert bits(scale) == bits(dq)
    np.testing.assert_array_equal(host(w8d), w8)
    yc = host(rz.rz_fp8_gemm(a8, w8d, m, sc, scale))
    tol = fp8_path.bound(a8h, w8, m, dqa, dqw)
    assert (np.abs(y.astype(np.float64) - yc) <= 2 * tol).all()
    check(y, a8h, w8, m, dqa, dqw)


@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
def test_nan_block_scale(rz, qtype):
    # a few blocks with an f16 NaN super-block scale: their weights decode to
    # NaN, which the absmax ignores and the encoder maps to 0x7E (448); the
    # waves that hold them take the encoder with NaN handling, the others
    # the one without
    m, n, k = 520, 300, 768
    blocks = W.weight_blocks(qtype, 8450 + qtype, n, k)
    bb = 144 if qtype == W.Q4_K else 210
    off = 0 if qtype == W.Q4_K else 208
    view = blocks.reshape(-1, bb)
    for b in (0, 7, 3 * (k // 256) + 1, view.shape[0] - 1):
        view[b, off:off + 2] = (0x00, 0x7E)  # f16 NaN, little-endian
    x = W.act_normal(8451, m, k)
    y, a8, w8, dqa, dqw, _ = run(rz, qtype, blocks, n, k, x)
    assert (w8 == 0x7E).any()
    check(y, a8, w8, m, dqa, dqw)


def test_zero_activation_gives_exact_zero(rz):
    m, n, k = 40, 300, 512
    for qtype in (W.Q4_K, W.Q6_K):
        y, *_ = run(rz, qtype, W.weight_blocks(qtype, 8500 + qtype, n, k), n, k, W.act_zero(m, k))
        assert np.array_equal(y, np.zeros((m, n), np.float32))


# full-size weights of the 7B-class FFN at a prefill batch: gate (Q4_K,
# 18944 x 3584) and down (Q6_K, 3584 x 18944), M = 2048, sampled rows
@pytest.mark.parametrize("name,qtype,n,k", [("gate", W.Q4_K, 18944, 3584), ("down", W.Q6_K, 3584, 18944)])
def test_ffn_full_size_sampled(rz, name, qtype, n, k):
    m = 2048
    blocks = W.weight_blocks(qtype, W.seed_for(3, 0, name), n, k)
    x = W.act_silu_gated(W.seed_for(3, 0, "x_down"), m, k) if name == "down" else \
        W.act_student_t(W.seed_for(3, 0, "x_ffn"), m, k)
    print(f"kquant_fp8_gemm full size {name} m={m} n={n} k={k}", flush=True)
    q, dq, w8, rdq = scales_match(rz, qtype, blocks, n, k)
    a8, sc = rz.rz_fp8_quant_act(dev(x))
    r8, _, rdqa = fp8_path.quant_act(x)
    y = rz.rz_kquant_fp8_gemm(a8, m, sc, qtype, dev(blocks), n, k, q, dq)
    rows = np.sort(np.random.default_rng(8600 + qtype).choice(m, 12, replace=False))
    rows[0], rows[-1] = 0, m - 1
    y_s = y[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    yr, tol = fp8_path.gemm_rows(r8, w8, rows, rdqa, rdq)
    err = np.abs(y_s - yr)
    assert (err <= tol).all(), f"{(err > tol).sum()} out of bound"
    assert np.isfinite(y_s).all()


def test_empty_and_stream(rz):
    k, n = 512, 96
    blocks = W.weight_blocks(W.Q4_K, 8701, n, k)
    x = W.act_normal(8702, 3, k)
    q, dq, _ = rz.rz_kquant_weight_scale(W.Q4_K, dev(blocks), n, k)
    a8, sc = rz.rz_fp8_quant_act(dev(x))
    y0 = rz.rz_kquant_fp8_gemm(a8, 0, sc, W.Q4_K, dev(blocks), n, k, q, dq)
    assert tuple(y0.shape) == (0, n)
    bd = dev(blocks)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = rz.rz_kquant_fp8_gemm(a8, 3, sc, W.Q4_K, bd, n, k, q, dq, stream=s)
    s.synchronize()
    w8, rdq, _ = fp8_path.pack_weight(W.Q4_K, blocks, n, k)
    r8, _, rdqa = fp8_path.quant_act(x)
    check(y.cpu().numpy(), r8, w8, 3, rdqa, rdq)
