"""End-to-end parity of the path on the workload configurations (GPU).

Each group quantises its activation once and reuses it for every GEMM that
reads it (Q/K/V; gate/up), as the path prescribes: either one GEMM call per
weight, or (the way bench.py runs the FFN step) every weight of the step
packed by one rz_fp8_pack_weights call and the GEMMs on one activation run
by one rz_fp8_gemm_group call.  Packed bytes, scales and
activation codes are compared bit for bit with the oracle; GEMM outputs are
compared element by element on every row (configurations 1, 2, 3 and 5) or
on sampled rows (the 4096-row layers of configuration 4; the oracle computes
those rows exactly); all 196 weights of configuration 4 are checked against
the oracle's recorded hashes.
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
    rz.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return rz


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_group(rz, grp, rows=None, check_bytes=True):
    print(f"\n  group m={grp.m} k={grp.k} act={grp.act_kind} gemms={[g.name for g in grp.gemms]}", flush=True)
    x = grp.activation()
    ws = rz.workspace("cuda")
    a8, sc = rz.rz_fp8_quant_act(dev(x), ws=ws)
    r8, ra, rdq = fp8_path.quant_act(x)
    torch.cuda.synchronize()
    sch = sc.cpu().numpy()
    assert sch[0] == ra and sch[1] == rdq
    np.testing.assert_array_equal(a8.cpu().numpy(), r8)
    for gm in grp.gemms:
        blocks = W.weight_blocks(gm.qtype, gm.w_seed, gm.n, gm.k)
        w8, wsc, wam = rz.rz_fp8_pack_weight(gm.qtype, dev(blocks), gm.n, gm.k, ws=ws)
        rw8, rwdq, rwa = fp8_path.pack_weight(gm.qtype, blocks, gm.n, gm.k)
        assert np.float32(wam) == rwa and np.float32(wsc) == rwdq, gm.name
        if check_bytes:
            np.testing.assert_array_equal(w8.cpu().numpy(), rw8)
        y = rz.rz_fp8_gemm(a8, w8, grp.m, sc, wsc)
        torch.cuda.synchronize()
        sel = np.arange(grp.m) if rows is None else np.asarray(rows)
        y_s = y[torch.from_numpy(sel).cuda()].cpu().numpy().astype(np.float64)
        yr, tol = fp8_path.gemm_rows(r8, rw8, sel, rdq, rwdq)
        err = np.abs(y_s - yr)
        assert (err <= tol).all(), f"{gm.name}: {(err > tol).sum()} out of bound"
        assert np.isfinite(y_s).all()
        print(f"    {gm.name}: N={gm.n} K={gm.k} rows={len(sel)} max err/tol="
              f"{np.max(err / np.where(tol > 0, tol, 1)):.3g}", flush=True)
        del w8, y


def check_rows(name, y, r8, rw8, rdq, rwdq, sel):
    y_s = y[torch.from_numpy(np.asarray(sel)).cuda()].cpu().numpy().astype(np.float64)
    yr, tol = fp8_path.gemm_rows(r8, rw8, np.asarray(sel), rdq, rwdq)
    err = np.abs(y_s - yr)
    assert (err <= tol).all(), f"{name}: {(err > tol).sum()} out of bound"
    assert np.isfinite(y_s).all()
    print(f"    {name}: rows={len(sel)} max err/tol={np.max(err / np.where(tol > 0, tol, 1)):.3g}", flush=True)


def run_step(rz, groups, rows=None):
    """The groups' weights packed in one call; per group one activation
    quantisation and one grouped GEMM call; every result against the oracle."""
    ws = rz.workspace("cuda")
    gemms = [gm for grp in groups for gm in grp.gemms]
    print(f"\n  step: {[(gm.name, gm.n, gm.k) for gm in gemms]}", flush=True)
    blocks = {gm.name: W.weight_blocks(gm.qtype, gm.w_seed, gm.n, gm.k) for gm in gemms}
    packed = rz.rz_fp8_pack_weights([(gm.qtype, dev(blocks[gm.name]), gm.n, gm.k, None) for gm in gemms], ws=ws)
    packed = dict(zip([gm.name for gm in gemms], packed))
    for grp in groups:
        x = grp.activation()
        a8, sc = rz.rz_fp8_quant_act(dev(x), ws=ws)
        r8, ra, rdq = fp8_path.quant_act(x)
        ys = rz.rz_fp8_gemm_group(a8, grp.m, sc, [(packed[gm.name][0], packed[gm.name][1]) for gm in grp.gemms])
        torch.cuda.synchronize()
        sch = sc.cpu().numpy()
        assert sch[0] == ra and sch[1] == rdq
        np.testing.assert_array_equal(a8.cpu().numpy(), r8)
        sel = np.arange(grp.m) if rows is None else rows(grp)
        for gm, y in zip(grp.gemms, ys):
            w8, wsc, wam = packed[gm.name]
            rw8, rwdq, rwa = fp8_path.pack_weight(gm.qtype, blocks[gm.name], gm.n, gm.k)
            assert np.float32(wam) == rwa and np.float32(wsc) == rwdq, gm.name
            np.testing.assert_array_equal(w8.cpu().numpy(), rw8)
            check_rows(gm.name, y, r8, rw8, rdq, rwdq, sel)
        del ys


def test_config1(rz):
    for grp in W.config_groups(1):
        run_group(rz, grp)


def test_config2_attention_qkv(rz):
    for grp in W.config_groups(2):
        run_group(rz, grp)


@pytest.mark.parametrize("m", W.CFG5_M)
def test_config5_small_m(rz, m):
    for grp in W.config_groups(5, m=m):
        run_group(rz, grp)


def test_config5_zero_activation(rz):
    for m in W.CFG5_M:
        grp = W.config_groups(5, m=m)[0]
        grp.act_kind = "zero"
        run_group(rz, grp)


def _sample_rows(m, count=64, seed=0):
    g = np.random.Generator(np.random.PCG64(seed))
    rows = set(g.choice(m, size=count - 4, replace=False).tolist()) | {0, 1, m - 2, m - 1}
    return sorted(rows)


def test_config3_ffn_full_size(rz):
    # every output row of gate, up and down against the oracle's exact sums
    for grp in W.config_groups(3):
        run_group(rz, grp)


@pytest.mark.parametrize("layer", [0, W.CFG4_LAYERS - 1])
def test_config4_layer(rz, layer):
    for grp in W.config_groups(4, layer=layer):
        run_group(rz, grp, rows=_sample_rows(grp.m, seed=grp.act_seed))


def test_config3_bench_step(rz):
    # the FFN step exactly as bench.py launches it: gate, up and down packed in
    # one call (one launch set), gate and up in one grouped GEMM launch; every
    # output row checked
    run_step(rz, W.config_groups(3))


def test_config4_all_weights_pack_golden(rz, golden):
    # all 196 weights of the 28-layer sweep packed by one rz_fp8_pack_weights
    # call; the codes (SHA-256), absmax and scale of every one equal the
    # oracle's, as tests/golden/make_cfg4_pack_golden.py recorded them
    import hashlib
    want = {(int(f[0]), f[1]): f for f in golden("cfg4_pack_sha256.txt")}
    assert len(want) == 7 * W.CFG4_LAYERS
    specs, blocks = [], []
    for layer in range(W.CFG4_LAYERS):
        for grp in W.config_groups(4, layer=layer):
            for gm in grp.gemms:
                specs.append((layer, gm))
                blocks.append(dev(W.weight_blocks(gm.qtype, gm.w_seed, gm.n, gm.k)))
    print(f"\n  packing {len(specs)} weights in one call", flush=True)
    outs = rz.rz_fp8_pack_weights([(gm.qtype, b, gm.n, gm.k, None) for (_, gm), b in zip(specs, blocks)])
    torch.cuda.synchronize()
    del blocks
    for (layer, gm), (w8, scale, amax) in zip(specs, outs):
        f = want[(layer, gm.name)]
        assert (int(f[2]), int(f[3]), int(f[4])) == (gm.qtype, gm.n, gm.k)
        assert hashlib.sha256(w8.cpu().numpy().tobytes()).hexdigest() == f[5], (layer, gm.name)
        assert f"{int(np.float32(amax).view(np.uint32)):08x}" == f[6], (layer, gm.name, amax)
        assert f"{int(np.float32(scale).view(np.uint32)):08x}" == f[7], (layer, gm.name, scale)
    print(f"  {len(specs)} weights: codes, absmax and scales equal the oracle's", flush=True)


def test_config2_grouped(rz):
    run_step(rz, W.config_groups(2))


def test_config4_layer_grouped(rz):
    # q+k+v in one launch (288 tiles at M=4096), gate+up in one launch
    run_step(rz, W.config_groups(4, layer=1), rows=lambda grp: _sample_rows(grp.m, seed=grp.act_seed + 2))
