"""GPU parity of the small-batch GEMV straight from K-quant blocks
(rz_kquant_gemv) against the CPU oracle (needs an MI355X).

Bar: |y - y_ref| <= gamma_K * sum_k |x_k w_k| per element, y_ref the
oracle's float64 sum of exact fp32 products over the dequantised weight
(oracle.kquant_gemv), gamma_K = K u / (1 - K u), u = 2^-24: the bound for
fp32 accumulation in any order.  Zero rows of x give exactly 0.
"""
import numpy as np
import pytest

import workloads as W
from oracle import kquant_gemv

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


def check(qtype, blocks, n, k, x, y):
    ref = kquant_gemv.gemv(qtype, blocks, n, k, x)
    bd = kquant_gemv.bound(qtype, blocks, n, k, x)
    err = np.abs(y.astype(np.float64) - ref)
    bad = err > bd
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} outside the bound; first at "
                           f"{np.argwhere(bad)[0]}, err {err[bad][0]:.3g} > {bd[bad][0]:.3g}")
    return float(np.max(err / np.maximum(bd, 1e-300)))


def run(rz, qtype, blocks, n, k, x):
    print(f"kquant_gemv qtype={qtype} m={x.shape[0]} n={n} k={k}", flush=True)
    return host(rz.rz_kquant_gemv(qtype, dev(blocks), n, k, dev(x)))


# every batch size, ragged n around the rows-per-wave switch, K with a partial
# last step (9 and 14 blocks: the lanes' block loop ends unevenly)
@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("n,k", [(1, 256), (37, 2304), (1000, 512), (4101, 3584)])
def test_parity_shapes(rz, qtype, m, n, k):
    blocks = W.weight_blocks(qtype, 7000 + n + m, n, k)
    x = W.act_normal(7100 + m + k, m, k)
    y = run(rz, qtype, blocks, n, k, x)
    assert y.shape == (m, n)
    check(qtype, blocks, n, k, x, y)


# the small-M edge configuration at full size: K=3584, N=4608, Q4_K, Student-t
# activations with outlier channels, every output checked
@pytest.mark.parametrize("m", [1, 4])
def test_config5_full_size(rz, m):
    n, k = 4608, 3584
    blocks = W.weight_blocks(W.Q4_K, W.seed_for(5, 0, "up"), n, k)
    x = W.act_student_t(W.seed_for(5, 0, "x_ffn") + m, m, k)
    y = run(rz, W.Q4_K, blocks, n, k, x)
    check(W.Q4_K, blocks, n, k, x, y)


# the down projection's weight at a decode-sized batch: Q6_K, K=18944
def test_down_shape_q6k(rz):
    n, k, m = 3584, 18944, 2
    blocks = W.weight_blocks(W.Q6_K, W.seed_for(3, 0, "down"), n, k)
    x = W.act_silu_gated(W.seed_for(3, 0, "x_down"), m, k)
    y = run(rz, W.Q6_K, blocks, n, k, x)
    check(W.Q6_K, blocks, n, k, x, y)


@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
def test_zero_activation_gives_exact_zero(rz, qtype):
    n, k = 300, 1024
    blocks = W.weight_blocks(qtype, 7201, n, k)
    y = run(rz, qtype, blocks, n, k, W.act_zero(3, k))
    assert np.array_equal(y, np.zeros((3, n), np.float32))


@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
def test_nan_row_stays_in_its_row(rz, qtype):
    n, k, m = 129, 512, 3
    blocks = W.weight_blocks(qtype, 7301, n, k)
    x = W.act_normal(7302, m, k)
    x[1, 77] = np.nan
    y = run(rz, qtype, blocks, n, k, x)
    assert np.isnan(y[1]).all()
    clean = x[[0, 2]]
    check(qtype, blocks, n, k, clean, y[[0, 2]])


def test_matches_dequant_then_matmul_exactly_for_one_block(rz):
    # K = 256: every lane sums at most one block, so the result must equal the
    # oracle's sum rounded to fp32 to within the (tiny) bound, and the weight
    # the kernel decodes must be the one rz_dequant_f32 returns
    n, k = 64, 256
    for qtype in (W.Q4_K, W.Q6_K):
        blocks = W.weight_blocks(qtype, 7401 + qtype, n, k)
        w = host(rz.rz_dequant_f32(qtype, dev(blocks), n, k))
        eye = np.zeros((8, k), np.float32)
        cols = [0, 1, 31, 32, 63, 128, 200, 255]
        for i, c in enumerate(cols):
            eye[i, c] = 1.0
        y = run(rz, qtype, blocks, n, k, eye)
        np.testing.assert_array_equal(y, w[:, cols].T)


def test_empty_and_stream(rz):
    k = 512
    blocks = dev(W.weight_blocks(W.Q4_K, 7501, 16, k))
    y = rz.rz_kquant_gemv(W.Q4_K, blocks, 0, k, dev(W.act_normal(1, 2, k)))
    assert tuple(y.shape) == (2, 0)
    s = torch.cuda.Stream()
    x = W.act_normal(7502, 2, k)
    xd = dev(x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = rz.rz_kquant_gemv(W.Q4_K, blocks, 16, k, xd, stream=s)
    s.synchronize()
    check(W.Q4_K, W.weight_blocks(W.Q4_K, 7501, 16, k), 16, k, x, y.cpu().numpy())
