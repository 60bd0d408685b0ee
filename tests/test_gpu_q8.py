"""GPU parity of the integer path (Q8_1 activation x Q4_K weight) against the
oracle (needs an MI355X).

Q8_1 blocks are compared bit for bit (codes, f16 d and s), including zero,
NaN, +-Inf, huge and tiny blocks; the GEMM element by element against the
oracle's float64 product of the two dequantised tensors, within
oracle/q8_path.bound, on ragged shapes (rows and columns past a 128-wide
workgroup tile, a 64-wide wave tile and a 32-wide MFMA block) and on the
configurations' shapes.
"""
import numpy as np
import pytest

import workloads as W
from oracle import q8_path

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


@pytest.mark.parametrize("m,k,kind", [(1, 256, "normal"), (16, 512, "normal"), (37, 3584, "student_t"),
                                      (1000, 3584, "student_t"), (2048, 3584, "normal"), (64, 18944, "silu")])
def test_quant_bit_exact(rz, m, k, kind):
    x = {"normal": W.act_normal, "student_t": W.act_student_t, "silu": W.act_silu_gated}[kind](3300 + m, m, k)
    got = host(rz.rz_q8_1_quant(dev(x)))
    want = q8_path.quant_q8_1(x)
    assert got.shape == want.shape == (m, k // 32, 36)
    np.testing.assert_array_equal(got, want)


def test_quant_special_blocks(rz):
    m, k = 4, 512
    x = W.act_normal(3400, m, k)
    x[0, 0:32] = 0.0                       # zero block
    x[0, 32:64] = np.nan                   # NaN only: a zero block
    x[0, 64] = np.nan                      # NaN ignored by the absmax, code 0
    x[0, 96] = np.inf                      # Inf absmax: d = Inf, every code 0
    x[0, 128] = -np.inf
    x[1, 0:32] *= 1e30                     # d overflows f16 (Inf in the block)
    x[1, 32:64] *= 1e-30                   # tiny: d is an fp32 subnormal, 1/d overflows
    x[1, 64:96] = 1e-40                    # fp32 subnormal inputs
    x[2, 0:32] = np.linspace(-127, 127, 32).astype(np.float32)  # d = 1: exact halves
    x[2, 32:64] = np.arange(32, dtype=np.float32) - 15.5        # ties away from zero
    got = host(rz.rz_q8_1_quant(dev(x)))
    with np.errstate(all="ignore"):
        want = q8_path.quant_q8_1(x)
    # bytes equal, except that a NaN s only has to be a NaN
    gs, ws_ = got[..., 2:4].copy().view(np.float16), want[..., 2:4].copy().view(np.float16)
    np.testing.assert_array_equal(np.isnan(gs), np.isnan(ws_))
    keep = ~np.isnan(ws_)[..., 0]
    np.testing.assert_array_equal(got[..., :2], want[..., :2])
    np.testing.assert_array_equal(got[..., 4:], want[..., 4:])
    np.testing.assert_array_equal(got[keep][:, 2:4], want[keep][:, 2:4])


def check(y, q8, blocks, n, k, rows=None):
    m = y.shape[0]
    rows = np.arange(m) if rows is None else np.asarray(rows)
    yr = q8_path.gemm(q8, blocks, n, k, rows=rows)
    tol = q8_path.bound(q8, blocks, n, k, rows=rows)
    err = np.abs(y[rows].astype(np.float64) - yr)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} out of bound; worst {err[bad].max()} vs {tol[bad].max()}"
    assert np.isfinite(y[rows]).all()
    return float(np.max(err / np.where(tol > 0, tol, 1)))


@pytest.mark.parametrize("m,n,k", [(1, 1, 256), (16, 256, 512), (33, 65, 256), (100, 200, 768), (130, 300, 1280),
                                   (512, 512, 3584), (37, 4608, 3584), (1000, 1000, 2304)])
def test_gemm_shapes(rz, m, n, k):
    x = W.act_student_t(3500 + m + n, m, k)
    blocks = W.q4k_blocks(3600 + n, n, k)
    q8 = q8_path.quant_q8_1(x)
    print(f"\n  q8 x q4k m={m} n={n} k={k}", flush=True)
    y = host(rz.rz_q8_q4k_gemm(dev(q8), m, dev(blocks), n, k))
    assert y.shape == (m, n)
    r = check(y, q8, blocks, n, k)
    print(f"  max err/tol={r:.3g}", flush=True)


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_configs_from_activation(rz, cfg):
    # quantise on the GPU, compare the blocks, then the GEMM, every row
    groups = W.config_groups(cfg) if cfg != 5 else [W.config_groups(5, m=mm)[0] for mm in W.CFG5_M]
    for grp in groups:
        x = grp.activation()
        q8_dev = rz.rz_q8_1_quant(dev(x))
        q8 = q8_path.quant_q8_1(x)
        np.testing.assert_array_equal(host(q8_dev), q8)
        for gm in grp.gemms:
            if gm.qtype != W.Q4_K:
                continue  # the integer path takes Q4_K weights
            blocks = W.weight_blocks(gm.qtype, gm.w_seed, gm.n, gm.k)
            y = host(rz.rz_q8_q4k_gemm(q8_dev, grp.m, dev(blocks), gm.n, gm.k))
            r = check(y, q8, blocks, gm.n, gm.k)
            print(f"\n  cfg {cfg} {gm.name}: m={grp.m} n={gm.n} k={gm.k} max err/tol={r:.3g}", flush=True)


def test_config3_gate_sampled_rows(rz):
    # the FFN gate at full size: 2048 x 18944 x 3584, rows sampled (with the last 40)
    grp = W.config_groups(3)[0]
    gm = grp.gemms[0]
    x = grp.activation()
    blocks = W.weight_blocks(gm.qtype, gm.w_seed, gm.n, gm.k)
    q8_dev = rz.rz_q8_1_quant(dev(x))
    y = host(rz.rz_q8_q4k_gemm(q8_dev, grp.m, dev(blocks), gm.n, gm.k))
    q8 = q8_path.quant_q8_1(x)
    np.testing.assert_array_equal(host(q8_dev), q8)
    g = np.random.Generator(np.random.PCG64(5))
    rows = np.unique(np.concatenate([g.choice(grp.m, 24, replace=False), np.arange(grp.m - 40, grp.m)]))
    r = check(y, q8, blocks, gm.n, gm.k, rows)
    print(f"\n  gate M=2048: rows={len(rows)} max err/tol={r:.3g}", flush=True)


def test_zero_activation_gives_zero(rz):
    m, n, k = 40, 300, 512
    blocks = W.q4k_blocks(3700, n, k)
    q8 = rz.rz_q8_1_quant(dev(np.zeros((m, k), np.float32)))
    y = host(rz.rz_q8_q4k_gemm(q8, m, dev(blocks), n, k))
    assert (y == 0).all()


def test_empty_and_rejects(rz):
    lib = rz.lib()
    assert lib.rz_q8_q4k_gemm(None, 0, None, 5, 256, None, None) == 0
    assert lib.rz_q8_1_quant(None, 0, 256, None, None) == 0
    assert lib.rz_q8_1_bytes(3, 512) == 3 * 16 * 36
    with pytest.raises(rz.RzError):
        rz.rz_q8_q4k_gemm(torch.zeros(64, dtype=torch.uint8, device="cuda"), 1,
                          torch.zeros(144, dtype=torch.uint8, device="cuda"), 1, 300)
