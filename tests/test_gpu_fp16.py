"""GPU parity of the FP16 comparator path against the oracle (needs an MI355X).

The fp16 weight cache and the fp16 activation are compared bit for bit
(including special scales and values that overflow or underflow fp16); the
GEMM element by element against the oracle's float64 sum of the exact fp16
products, within oracle/fp16_path.bound, on every plan the kernel takes
(256x256 interior tiles with whole and half tiles, the 256x256 edge kernel,
128x128 and 64x32 tiles) and on the configurations' shapes.
"""
import numpy as np
import pytest

import workloads as W
from oracle import fp16_path
from tests.test_gpu_special_blocks import random_blocks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rz():
    import fp8_prefill_gemm_amd as rz
    rz.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return rz


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits16(a):
    return np.ascontiguousarray(a).view(np.uint16)


@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
@pytest.mark.parametrize("n,k", [(1, 256), (37, 1280), (256, 3584)])
def test_pack_bit_exact(rz, qtype, n, k):
    blocks = W.weight_blocks(qtype, 2100 + n, n, k)
    got = host(rz.rz_fp16_pack_weight(qtype, dev(blocks), n, k))
    want = fp16_path.pack_weight(qtype, blocks, n, k)
    np.testing.assert_array_equal(bits16(got), bits16(want))


@pytest.mark.parametrize("qtype,mode", [(W.Q4_K, "raw"), (W.Q6_K, "raw"), (W.Q4_K, "finite"), (W.Q6_K, "finite")])
def test_pack_special_scales(rz, qtype, mode):
    # random block bytes: fp16 values that overflow to +-Inf, NaN, subnormals
    n, k = 48, 1024
    blocks = random_blocks(qtype, n, k, 2200 + qtype, mode)
    got = host(rz.rz_fp16_pack_weight(qtype, dev(blocks), n, k))
    with np.errstate(all="ignore"):
        want = fp16_path.pack_weight(qtype, blocks, n, k)
    gn, wn = np.isnan(got), np.isnan(want)
    np.testing.assert_array_equal(gn, wn)
    np.testing.assert_array_equal(bits16(got)[~gn], bits16(want)[~wn])
    assert np.isinf(want).any()


def test_pack_rounds_twice(rz):
    # fp32 first, then fp16 (the pages' fp32 scratch and cvt.rn.f16.f32):
    # 37584 + 2^-13 -> 37584.0 -> 37568 (a single rounding would give 37600)
    from tests.test_oracle_fp16 import double_rounding_block
    blk = np.concatenate([double_rounding_block()] * 3)
    got = host(rz.rz_fp16_pack_weight(W.Q4_K, dev(blk), 1, 768))
    np.testing.assert_array_equal(bits16(got), bits16(fp16_path.pack_weight(W.Q4_K, blk, 1, 768)))
    assert (bits16(got)[0, :32] == 0x7896).all()


@pytest.mark.parametrize("m,k", [(1, 256), (16, 512), (37, 3584), (1000, 3584)])
def test_convert_act_bit_exact(rz, m, k):
    x = W.act_student_t(2300 + m, m, k)
    x[0, :8] = [70000.0, -65520.0, 65519.0, 1e-8, -3e-8, -0.0, np.nan, 1e-40]
    got = host(rz.rz_fp16_convert_act(dev(x)))
    with np.errstate(all="ignore"):
        want = fp16_path.convert_act(x)
    assert got.shape == want.shape == (fp16_path.pad_m(m), k)
    gn, wn = np.isnan(got), np.isnan(want)
    np.testing.assert_array_equal(gn, wn)
    np.testing.assert_array_equal(bits16(got)[~gn], bits16(want)[~wn])


def test_convert_act_overwrites_pad_rows(rz):
    x = W.act_normal(2400, 5, 256)
    out = torch.full((16, 256), 7.0, dtype=torch.float16, device="cuda")
    rz.rz_fp16_convert_act(dev(x), out)
    got = host(out)
    assert (got[5:] == 0).all()
    np.testing.assert_array_equal(bits16(got[:5]), bits16(x.astype(np.float16)))


def check_gemm(y, a16, w16, m, rows=None):
    rows = np.arange(m) if rows is None else np.asarray(rows)
    yr = fp16_path.gemm(a16[rows], w16, len(rows))
    tol = fp16_path.bound(a16[rows], w16, len(rows))
    err = np.abs(y[rows].astype(np.float64) - yr)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} out of bound; worst {err[bad].max()} vs {tol[bad].max()}"
    assert np.isfinite(y[rows]).all()
    return float(np.max(err / np.where(tol > 0, tol, 1)))


def _operands(seed, m, n, k):
    g = np.random.Generator(np.random.PCG64(seed))
    a = np.zeros((fp16_path.pad_m(m), k), np.float16)
    a[:m] = g.standard_normal((m, k)).astype(np.float16)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float16)
    return a, w


@pytest.mark.parametrize("m,n,k", [
    (2048, 2560, 512),    # interior: 80 tiles, all as half tiles
    (2048, 8192, 256),    # interior: 256 whole tiles
    (1000, 1536, 1024),   # interior with the last m-tile overlapping (padded M 1008)
    (2000, 4100, 512),    # interior with ragged N (last n-tile overlapping)
    (160, 65536, 256),    # 256x256 edge kernel (padded M < 256, >= 256 tiles)
    (300, 520, 768),      # 128x128 tiles, ragged
    (16, 256, 512), (1, 64, 256), (37, 200, 768),  # 64x32 tiles (small M)
])
def test_gemm_plans(rz, m, n, k):
    a, w = _operands(2500 + m + n, m, n, k)
    print(f"\n  fp16 gemm m={m} n={n} k={k}", flush=True)
    y = host(rz.rz_fp16_gemm(dev(a), dev(w), m))
    assert y.shape == (m, n)
    rows = None if m * n <= 4_000_000 else np.unique(np.concatenate([[0, 1, m - 2, m - 1],
                                                                      np.random.Generator(np.random.PCG64(m)).choice(m, 60, replace=False)]))
    check_gemm(y, a, w, m, rows)


@pytest.mark.parametrize("m,n", [(2048, 13312), (2000, 13300)])
def test_gemm_quarter_tiles(rz, m, n):
    # 52 tiles per XCD: one round of 32, the 20 left over as 32 half and 16
    # quarter tiles (the fp16 instance of the interior kernel); every row
    # checked, ragged M and N in the second case
    k = 256
    a, w = _operands(2600 + m, m, n, k)
    print(f"\n  fp16 gemm quarter tiles m={m} n={n} k={k}", flush=True)
    y = host(rz.rz_fp16_gemm(dev(a), dev(w), m))
    check_gemm(y, a, w, m)


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_configs_from_blocks(rz, cfg):
    # the whole comparator path from the K-quant blocks, every output row
    groups = W.config_groups(cfg) if cfg != 5 else [W.config_groups(5, m=mm)[0] for mm in W.CFG5_M]
    for grp in groups:
        x = grp.activation()
        a_dev = rz.rz_fp16_convert_act(dev(x))
        a_ref = fp16_path.convert_act(x)
        np.testing.assert_array_equal(bits16(host(a_dev)), bits16(a_ref))
        for gm in grp.gemms:
            blocks = W.weight_blocks(gm.qtype, gm.w_seed, gm.n, gm.k)
            w_dev = rz.rz_fp16_pack_weight(gm.qtype, dev(blocks), gm.n, gm.k)
            w_ref = fp16_path.pack_weight(gm.qtype, blocks, gm.n, gm.k)
            np.testing.assert_array_equal(bits16(host(w_dev)), bits16(w_ref))
            y = host(rz.rz_fp16_gemm(a_dev, w_dev, grp.m))
            r = check_gemm(y, a_ref, w_ref, grp.m)
            print(f"\n  cfg {cfg} {gm.name}: m={grp.m} n={gm.n} k={gm.k} max err/tol={r:.3g}", flush=True)
            del w_dev


def test_gemm_empty_and_identity(rz):
    k, n, m = 512, 300, 5
    w = np.zeros((n, k), np.float16)
    w[np.arange(n), np.arange(n)] = 1.0
    a = np.zeros((16, k), np.float16)
    a[:m] = np.random.Generator(np.random.PCG64(9)).standard_normal((m, k)).astype(np.float16)
    y = host(rz.rz_fp16_gemm(dev(a), dev(w), m))
    np.testing.assert_array_equal(y, a[:m, :n].astype(np.float32))
    assert rz.lib().rz_fp16_gemm(None, None, 0, 7, 256, None, None) == 0
