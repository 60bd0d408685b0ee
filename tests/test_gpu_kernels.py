"""GPU parity of each kernel against the CPU oracle (needs an MI355X).

Bit-exact: E4M3 codes, dequantised fp32 weights, absmax and scales.
GEMM: |y - y_ref| <= 2e-3 * dq_act * dq_w * sum_k |dec(a_k) dec(w_k)| per
element, y_ref the oracle's exact sum times the two scales.
"""
import numpy as np
import pytest

import workloads as W
from oracle import e4m3, fp8_path, kquant

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


def f32_from_bits(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


# ------------------------------------------------------------------ encoder

def test_encode_golden_and_classes(rz):
    from tests.test_oracle_e4m3 import _class_representatives, _pins
    pins = _pins()
    xb = np.array([p[0] for p in pins] + list(_class_representatives()), dtype=np.uint32)
    x = f32_from_bits(xb)
    got = host(rz.rz_e4m3_encode(dev(x), 1.0))
    np.testing.assert_array_equal(got, e4m3.encode_scaled(x, 1.0))
    # the golden codes themselves (scale 1 makes every NaN positive)
    for (bits, code), g in zip(pins, got[:len(pins)]):
        if ((bits >> 23) & 0xFF) == 0xFF and (bits & 0x7FFFFF):
            assert g == 0x7E
        else:
            assert g == code, hex(bits)


@pytest.mark.parametrize("count", [0, 1, 15, 16, 17, 1000, 65536 + 7])
@pytest.mark.parametrize("scale", [1.0, 448.0 / 3.75, 1e-3, 3.0e4, 0.0])
def test_encode_random_scaled(rz, count, scale):
    g = np.random.Generator(np.random.PCG64(count + 17))
    x = (g.standard_normal(count) * np.exp2(g.integers(-20, 20, count))).astype(np.float32)
    if count > 8:
        x[:4] = [np.inf, -np.inf, np.nan, -0.0]
    got = host(rz.rz_e4m3_encode(dev(x), scale))
    np.testing.assert_array_equal(got, e4m3.encode_scaled(x, scale))


def test_scales_bit_exact(rz):
    g = np.random.Generator(np.random.PCG64(99))
    a = np.exp2(g.uniform(-149, 127, 200_000)).astype(np.float32)
    a[:6] = [0.0, 448.0, 1.0, np.inf, 1e-45, 3.4e38]
    q, dq = rz.rz_fp8_scales(dev(a))
    q, dq = host(q), host(dq)
    ref = [fp8_path.scales_from_absmax(v) for v in a]
    np.testing.assert_array_equal(q, np.array([r[0] for r in ref], np.float32))
    np.testing.assert_array_equal(dq, np.array([r[1] for r in ref], np.float32))


# ------------------------------------------------------------------ absmax

@pytest.mark.parametrize("count", [0, 1, 3, 17, 1000, 1 << 20, (1 << 22) + 3])
def test_absmax(rz, count):
    g = np.random.Generator(np.random.PCG64(count))
    x = g.standard_normal(count).astype(np.float32)
    if count >= 17:
        x[5] = np.nan
        x[count // 2] = -37.5  # the maximum, negative, mid-tensor
        x[3] = -0.0
    out = host(rz.rz_absmax_f32(dev(x)))
    assert out[0].view(np.uint32) == np.uint32(fp8_path.absmax_bits(x))


def test_absmax_specials(rz):
    for x in ([np.nan, np.nan], [-0.0], [1.0, -np.inf, np.nan], [1e-40, -3e-41]):
        x = np.array(x, np.float32)
        out = host(rz.rz_absmax_f32(dev(x)))
        assert out[0].view(np.uint32) == np.uint32(fp8_path.absmax_bits(x))


# ------------------------------------------------------------------ dequant

SHAPES = [(1, 256), (3, 768), (256, 512), (37, 1280), (130, 3584)]


@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
@pytest.mark.parametrize("n,k", SHAPES)
def test_dequant_bit_exact(rz, qtype, n, k):
    blocks = W.weight_blocks(qtype, 500 + n, n, k)
    got = host(rz.rz_dequant_f32(qtype, dev(blocks), n, k))
    want = kquant.dequant(qtype, blocks, n, k)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_dequant_golden_layout_blocks(rz):
    # the hand-pinned one-hot blocks go through the GPU unchanged
    from tests.test_oracle_kquant import UNIT_SCALES, _q4k_block, _q6k_block
    q4 = []
    for t in (0, 31, 32, 100, 127):
        qs = bytearray(128)
        qs[t] = 0x21
        q4.append(_q4k_block(scales=UNIT_SCALES, qs=qs))
    q4 = np.concatenate(q4)
    got = host(rz.rz_dequant_f32(W.Q4_K, dev(q4), q4.shape[0], 256))
    np.testing.assert_array_equal(got, kquant.dequant_q4k_blocks(q4))
    q6 = []
    for t in (0, 40, 100):
        ql = bytearray(128)
        ql[t] = 0x21
        q6.append(_q6k_block(ql=ql))
    q6.append(_q6k_block(scales=[-128] * 16, ql=bytes([0xFF] * 128), qh=bytes([0xFF] * 64)))
    q6 = np.concatenate(q6)
    got = host(rz.rz_dequant_f32(W.Q6_K, dev(q6), q6.shape[0], 256))
    np.testing.assert_array_equal(got, kquant.dequant_q6k_blocks(q6))


# ------------------------------------------------------------------ pack

@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
@pytest.mark.parametrize("n,k", SHAPES + [(512, 3584)])
def test_pack_bit_exact(rz, qtype, n, k):
    blocks = W.weight_blocks(qtype, 900 + n, n, k)
    w8, scale, amax = rz.rz_fp8_pack_weight(qtype, dev(blocks), n, k)
    r8, rdq, ra = fp8_path.pack_weight(qtype, blocks, n, k)
    assert np.float32(amax).view(np.uint32) == ra.view(np.uint32)
    assert np.float32(scale).view(np.uint32) == rdq.view(np.uint32)
    np.testing.assert_array_equal(host(w8), r8)


def test_pack_weights_batch(rz):
    # one call, mixed formats and shapes (including an all-zero weight): every
    # weight bit-exact against the oracle, the same as its own single call
    specs = [(W.Q4_K, 64, 512), (W.Q6_K, 37, 1280), (W.Q4_K, 512, 3584), (W.Q6_K, 1, 256), (W.Q4_K, 3, 768)]
    blocks = [W.weight_blocks(q, 1300 + i, n, k) for i, (q, n, k) in enumerate(specs)]
    blocks[3][:] = 0
    print(f"pack_weights batch of {len(specs)}", flush=True)
    outs = rz.rz_fp8_pack_weights([(q, dev(b), n, k, None) for (q, n, k), b in zip(specs, blocks)])
    for (q, n, k), b, (w8, scale, amax) in zip(specs, blocks, outs):
        r8, rdq, ra = fp8_path.pack_weight(q, b, n, k)
        assert np.float32(amax).view(np.uint32) == ra.view(np.uint32)
        assert np.float32(scale).view(np.uint32) == rdq.view(np.uint32)
        np.testing.assert_array_equal(host(w8), r8)
        s8, sscale, samax = rz.rz_fp8_pack_weight(q, dev(b), n, k)
        assert (sscale, samax) == (scale, amax)
        np.testing.assert_array_equal(host(s8), host(w8))


def test_pack_weights_sets_split_by_partial_keys(rz):
    # a 15360x3584 Q4_K weight takes 1680 pass-1 workgroups and a 7680x3584
    # Q6_K one 840: the first five weights (7560 partial keys, mixed types)
    # share one launch per pass, the sixth needs its own (a launch's partial
    # keys are capped at 8192)
    specs = [(W.Q4_K, 15360, 3584), (W.Q6_K, 7680, 3584)] + [(W.Q4_K, 15360, 3584)] * 4
    blocks = [W.weight_blocks(q, 1500 + i, n, k) for i, (q, n, k) in enumerate(specs)]
    print("pack_weights: six large weights in two launch sets", flush=True)
    outs = rz.rz_fp8_pack_weights([(q, dev(b), n, k, None) for (q, n, k), b in zip(specs, blocks)])
    for (q, n, k), b, (w8, scale, amax) in zip(specs, blocks, outs):
        r8, rdq, ra = fp8_path.pack_weight(q, b, n, k)
        assert np.float32(scale) == rdq and np.float32(amax) == ra
        np.testing.assert_array_equal(host(w8), r8)


def test_pack_weights_many(rz):
    # more weights than the first allocation of host scale slots (256), twice
    cnt = 300
    blocks = [W.weight_blocks(W.Q4_K if i % 3 else W.Q6_K, 1400 + i, 2, 256) for i in range(cnt)]
    qts = [W.Q4_K if i % 3 else W.Q6_K for i in range(cnt)]
    for rep in range(2):
        print(f"pack_weights batch of {cnt}, pass {rep}", flush=True)
        outs = rz.rz_fp8_pack_weights([(q, dev(b), 2, 256, None) for q, b in zip(qts, blocks)])
        for q, b, (w8, scale, amax) in zip(qts, blocks, outs):
            r8, rdq, ra = fp8_path.pack_weight(q, b, 2, 256)
            assert np.float32(scale) == rdq and np.float32(amax) == ra
            np.testing.assert_array_equal(host(w8), r8)


def test_pack_zero_weight(rz):
    blocks = np.zeros((4 * 2, 144), np.uint8)
    w8, scale, amax = rz.rz_fp8_pack_weight(W.Q4_K, dev(blocks), 4, 512)
    assert amax == 0.0 and np.float32(scale) == np.float32(1 / 448)
    assert (host(w8) == 0).all()


def test_pack_reuses_workspace(rz):
    ws = rz.workspace("cuda")
    for seed, (n, k) in enumerate([(64, 512), (8, 256), (300, 1024)]):
        blocks = W.q6k_blocks(seed, n, k)
        w8, scale, amax = rz.rz_fp8_pack_weight(W.Q6_K, dev(blocks), n, k, ws=ws)
        r8, rdq, ra = fp8_path.pack_weight(W.Q6_K, blocks, n, k)
        assert np.float32(scale) == rdq and np.float32(amax) == ra
        np.testing.assert_array_equal(host(w8), r8)


def test_pack_waits_behind_a_busy_stream(rz):
    # the pack's host wait polls for its scales and, after the first
    # millisecond, also queries the stream once a millisecond: a pack queued
    # behind ~20 ms of other work on a side stream still returns its scales
    # (and codes) bit-exact
    blocks = W.weight_blocks(W.Q4_K, 1700, 512, 3584)
    b = dev(blocks)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print("pack behind a 20 ms spin on a side stream", flush=True)
    with torch.cuda.stream(side):
        torch.cuda._sleep(int(40e6))  # ~40M cycles: well over 1 ms at any clock
        w8, scale, amax = rz.rz_fp8_pack_weight(W.Q4_K, b, 512, 3584, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    r8, rdq, ra = fp8_path.pack_weight(W.Q4_K, blocks, 512, 3584)
    assert np.float32(amax).view(np.uint32) == ra.view(np.uint32)
    assert np.float32(scale).view(np.uint32) == rdq.view(np.uint32)
    np.testing.assert_array_equal(host(w8), r8)


def test_quant_and_pack_share_a_workspace_in_turn(rz):
    # Quantisations and packs of different sizes (1 and 2048 pass-1
    # workgroups, a pack set of 3 weights) alternate on one workspace: each
    # writes the partial keys and scale records it reads, so none sees
    # another's leftovers, and every result matches the oracle bit for bit.
    ws = rz.workspace("cuda")
    g = np.random.Generator(np.random.PCG64(41))
    for m, k in [(1, 256), (2048, 3584), (3, 512), (2048, 3584), (1, 256)]:
        x = W.act_student_t(int(g.integers(1 << 30)), m, k)
        a8, sc = rz.rz_fp8_quant_act(dev(x), ws=ws)
        r8, ra, rdq = fp8_path.quant_act(x)
        sc = host(sc)
        assert sc[0].view(np.uint32) == ra.view(np.uint32) and sc[1].view(np.uint32) == rdq.view(np.uint32)
        np.testing.assert_array_equal(host(a8), r8)
        packs = [(W.Q4_K, W.q4k_blocks(m + 1, 64, 512), 64, 512), (W.Q6_K, W.q6k_blocks(m + 2, 32, 768), 32, 768),
                 (W.Q4_K, W.q4k_blocks(m + 3, 300, 256), 300, 256)]
        outs = rz.rz_fp8_pack_weights([(qt, dev(b), n, kk, None) for qt, b, n, kk in packs], ws=ws)
        for (qt, b, n, kk), (w8, scale, amax) in zip(packs, outs):
            r8w, rdqw, raw = fp8_path.pack_weight(qt, b, n, kk)
            assert np.float32(scale) == rdqw and np.float32(amax) == raw
            np.testing.assert_array_equal(host(w8), r8w)


# ------------------------------------------------------------------ activation

@pytest.mark.parametrize("m,k,kind", [(16, 512, "normal"), (1, 3584, "student_t"),
                                      (4, 3584, "student_t"), (37, 3584, "student_t"),
                                      (1000, 3584, "student_t"), (512, 3584, "normal"),
                                      (33, 256, "silu"), (5, 3584, "zero")])
def test_quant_act_bit_exact(rz, m, k, kind):
    x = W.Group(m, k, kind, 700 + m).activation()
    a8, sc = rz.rz_fp8_quant_act(dev(x))
    r8, ra, rdq = fp8_path.quant_act(x)
    sc = host(sc)
    assert sc[0].view(np.uint32) == ra.view(np.uint32)
    assert sc[1].view(np.uint32) == rdq.view(np.uint32)
    np.testing.assert_array_equal(host(a8), r8)


def test_quant_act_empty(rz):
    a8, sc = rz.rz_fp8_quant_act(torch.zeros((0, 512), device="cuda"))
    assert a8.shape == (0, 512)
    sc = host(sc)
    assert sc[0] == 0.0 and sc[1] == np.float32(1 / 448)
    # and through the C ABI with real buffers: nothing but the scales is written
    x = torch.ones((1, 512), device="cuda")
    a8 = torch.full((16, 512), 7, dtype=torch.uint8, device="cuda")
    sc = torch.full((4,), -1.0, device="cuda")
    ws = rz.workspace("cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert rz.lib().rz_fp8_quant_act(x.data_ptr(), 0, 512, a8.data_ptr(), sc.data_ptr(),
                                     ws.data_ptr(), st) == 0
    assert (host(a8) == 7).all()
    sc = host(sc)
    assert sc[0] == 0.0 and sc[1] == np.float32(1 / 448)


def test_quant_act_nonfinite(rz):
    x = W.act_normal(5, 3, 256)
    x[0, 0], x[1, 7], x[2, 9] = np.nan, np.inf, -3.0
    a8, sc = rz.rz_fp8_quant_act(dev(x))
    r8, ra, rdq = fp8_path.quant_act(x)
    sc = host(sc)
    assert sc[0] == np.inf and ra == np.inf and sc[1] == rdq
    np.testing.assert_array_equal(host(a8), r8)


def test_quant_act_overwrites_pad_rows(rz):
    x = W.act_normal(6, 20, 512)
    a8 = torch.full((32, 512), 0x5A, dtype=torch.uint8, device="cuda")
    rz.rz_fp8_quant_act(dev(x), a_fp8=a8)
    got = host(a8)
    assert (got[20:] == 0).all()
    np.testing.assert_array_equal(got, fp8_path.quant_act(x)[0])


# ------------------------------------------------------------------ GEMM

def check_gemm(y, a8, w8, m, dqa, dqw):
    yr = fp8_path.gemm(a8, w8, m, dqa, dqw)
    tol = fp8_path.bound(a8, w8, m, dqa, dqw)
    err = np.abs(y.astype(np.float64) - yr)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} elements out of bound; worst {err[bad].max()} at {np.argwhere(bad)[0]}"
    assert (y[tol == 0] == 0).all()


@pytest.mark.parametrize("m,n,k", [
    (16, 256, 512),      # config 1
    (1, 64, 256), (4, 96, 512), (37, 200, 768), (17, 258, 256),  # ragged n, n % 4 != 0
    (300, 130, 1024), (600, 520, 512),   # medium plan, ragged tiles
    (512, 1024, 512), (1000, 640, 256),
])
def test_gemm_random_codes(rz, m, n, k):
    g = np.random.Generator(np.random.PCG64(m * 7 + n))
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    mp = fp8_path.pad_m(m)
    a8 = g.choice(codes, size=(mp, k))
    a8[m:] = 0
    w8 = g.choice(codes, size=(n, k))
    sc = np.array([1.0, 0.0123, 0, 0], np.float32)
    wdq = np.float32(0.00731)
    y = host(rz.rz_fp8_gemm(dev(a8), dev(w8), m, dev(sc), float(wdq)))
    assert y.shape == (m, n)
    check_gemm(y, a8, w8, m, sc[1], wdq)


def test_gemm_large_plan_full(rz):
    # a shape that takes the 256x256 plan, checked in full
    m, n, k = 2048, 8192, 256
    bn, bm, _, wgs = rz.rz_fp8_gemm_plan(m, n, k)
    assert (bn, bm) == (256, 256)
    g = np.random.Generator(np.random.PCG64(1))
    a8 = g.integers(0, 0x7F, size=(m, k)).astype(np.uint8) | (g.integers(0, 2, size=(m, k)) << 7).astype(np.uint8)
    w8 = g.integers(0, 0x7F, size=(n, k)).astype(np.uint8)
    sc = np.array([1.0, 0.5, 0, 0], np.float32)
    y = host(rz.rz_fp8_gemm(dev(a8), dev(w8), m, dev(sc), 0.25))
    check_gemm(y, a8, w8, m, sc[1], np.float32(0.25))


def _codes(g, shape):
    a = g.integers(0, 0x7F, size=shape).astype(np.uint8)
    return a | (g.integers(0, 2, size=shape) << 7).astype(np.uint8)


# The persistent interior kernel (256 CUs, 32 per XCD): XCD x runs a
# contiguous run of Tx tiles, R = Tx // 32 whole rounds and the L tiles left
# over as 2L half tiles when R > 0 or 2L <= 32, else as L whole tiles.
@pytest.mark.parametrize("m,n,k,full", [
    (2048, 2560, 1536, True),    # 80 tiles, 10 per XCD: all as half tiles
    (2040, 2560, 1024, True),    # same with M padded to 2048: rows >= M dropped
    (2048, 2560, 768, True),     # half tiles only, 6 K-steps
    (2048, 3584, 1024, True),    # 112 tiles: 28 half tiles per XCD
    (2048, 10240, 1024, False),  # 320 tiles: one whole round + 8 tiles per XCD as halves
    (2048, 8960, 512, False),    # 280 tiles: 35 per XCD, one round + 3 tiles as halves
    (4096, 4096, 512, False),    # 256 tiles: exactly one round
    (4096, 4608, 1024, False),   # 288 tiles: one round + 4 tiles per XCD as halves
    (4096, 3584, 1024, False),   # 224 tiles, 28 per XCD: no round, the 56 halves would not fit one: whole
    (768, 25600, 512, False),    # 300 tiles, 37 or 38 per XCD: one round + halves
    (2040, 3584, 4864, False),   # 112 tiles as half tiles with long K, rows >= M dropped
    # padded M not a multiple of 256: the last m-tile (half) is moved up to
    # end at the last activation row and overlaps the one before it
    (2000, 18944, 512, False),   # 2 rounds + halves; last tile at 1744, half at 1872
    (1900, 2560, 1024, True),    # halves only (the last at 1776)
    (300, 16384, 512, False),    # 128 tiles: halves at 0, 128 and 176
    (300, 18944, 512, False),    # 148 tiles, 18 or 19 per XCD: whole tiles, the last m-tile at 48
    (600, 25600, 512, False),    # 300 tiles, one round + halves, the last m-tile at 352
    (1000, 65536, 512, False),   # 4 whole rounds, nothing left over, the last m-tile at 752
    # N not a multiple of 256: the last n-tile starts at N - 256
    (2048, 2500, 1024, True),    # halves only; last n-tile at 2244
    (2000, 18900, 512, False),   # ragged M and N: 2 rounds + halves, last tile at (1744, 18644)
    (768, 25700, 512, False),    # 303 tiles, one round + halves, the last n-tile at 25444
    (1000, 40000, 512, False),   # 2 rounds + halves, ragged M and N
    # 52 tiles per XCD: one round, the 20 left over as 32 halves + 16 quarters
    (2048, 13312, 512, True),
    (2000, 13300, 512, False),   # ragged M and N: the last m-tile at 1744, its quarters up to 1936
    (1000, 26624, 512, False),   # 4 m-tiles, the last at 752: quarters clamped to end at 1008
])
def test_gemm_interior_plans(rz, m, n, k, full):
    mp = fp8_path.pad_m(m)
    bn, bm, threads, wgs = rz.rz_fp8_gemm_plan(m, n, k)
    assert (bn, bm, threads) == (256, 256, 256)
    assert wgs == torch.cuda.get_device_properties(0).multi_processor_count  # one per CU
    assert rz.rz_fp8_gemm_workspace_bytes(m, n, k) == 0
    g = np.random.Generator(np.random.PCG64(m + n + k))
    a8, w8 = _codes(g, (mp, k)), _codes(g, (n, k))
    a8[m:] = 0
    sc = np.array([1.0, 0.03, 0, 0], np.float32)
    wdq = np.float32(0.011)
    A, Wd, S = dev(a8), dev(w8), dev(sc)
    # sampled rows include a band over the last 300 rows (overlapping tiles)
    rows = np.arange(m) if full else np.unique(np.concatenate(
        [[0, 1, m - 1], g.choice(m, 61, replace=False), np.arange(max(0, m - 300), m, 7)]))
    yr, tol = fp8_path.gemm_rows(a8, w8, rows, sc[1], wdq)
    for _ in range(2):  # twice in a row: nothing carried over between calls
        y = host(rz.rz_fp8_gemm(A, Wd, m, S, float(wdq)))
        assert y.shape == (m, n)
        err = np.abs(y[rows].astype(np.float64) - yr)
        assert (err <= tol).all(), f"{(err > tol).sum()} out of bound"


@pytest.mark.parametrize("m,n,k", [
    (200, 65636, 512),   # padded M < 256 with 257 tiles: 256x256 tiles crossing M_pad and N
    (129, 65400, 768),   # M_pad 144, last tile 120 columns wide
])
def test_gemm_large_edge(rz, m, n, k):
    bn, bm, threads, wgs = rz.rz_fp8_gemm_plan(m, n, k)
    mp = fp8_path.pad_m(m)
    assert (bn, bm, threads, wgs) == (256, 256, 256, -(-n // 256))
    assert rz.rz_fp8_gemm_workspace_bytes(m, n, k) == 0
    g = np.random.Generator(np.random.PCG64(m * 7 + n))
    a8, w8 = _codes(g, (mp, k)), _codes(g, (n, k))
    a8[m:] = 0
    sc = np.array([1.0, 0.02, 0, 0], np.float32)
    wdq = np.float32(0.013)
    rows = np.unique(np.concatenate([[0, m - 1], g.choice(m, 40, replace=False)]))
    yr, tol = fp8_path.gemm_rows(a8, w8, rows, sc[1], wdq)
    y = host(rz.rz_fp8_gemm(dev(a8), dev(w8), m, dev(sc), float(wdq)))
    err = np.abs(y[rows].astype(np.float64) - yr)
    assert (err <= tol).all(), f"{(err > tol).sum()} out of bound"


@pytest.mark.parametrize("m,n,k", [
    (1, 4608, 3584),     # one row per wave, last 1 KB chunk of K half used
    (3, 200, 768),       # three activation rows, K shorter than one pass
    (3, 1000, 18944),    # five passes over K
    (2, 17, 256),        # last workgroup with one row; lanes past K read zero
])
def test_gemm_gemv(rz, m, n, k):
    bn, bm, threads, wgs = rz.rz_fp8_gemm_plan(m, n, k)
    assert (bn, bm, threads, wgs) == (4, 16, 256, -(-n // 4))
    assert rz.rz_fp8_gemm_workspace_bytes(m, n, k) == 0
    g = np.random.Generator(np.random.PCG64(m * 11 + n + k))
    a8 = _codes(g, (16, k))
    a8[m:] = 0
    w8 = _codes(g, (n, k))
    sc = np.array([1.0, 0.019, 0, 0], np.float32)
    wdq = np.float32(0.0083)
    y = host(rz.rz_fp8_gemm(dev(a8), dev(w8), m, dev(sc), float(wdq)))
    assert y.shape == (m, n)
    check_gemm(y, a8, w8, m, sc[1], wdq)


@pytest.mark.parametrize("m,n,k", [
    (4, 4608, 3584),     # one activation block, 288 workgroups, 7 K-steps per wave
    (16, 200, 768),      # ragged last block of weight rows, 1-2 K-steps per wave
    (37, 200, 2816),     # three activation blocks (M_pad 48)
    (48, 4608, 3584),    # three full blocks
    (64, 258, 256),      # four blocks, n % 4 != 0, waves without K-steps
    (17, 1000, 18944),   # two blocks, 37 K-steps per wave in register chunks
    (16, 256, 512),      # configuration 1 shape
])
def test_gemm_skinny(rz, m, n, k):
    bn, bm, threads, wgs = rz.rz_fp8_gemm_plan(m, n, k)
    mp = fp8_path.pad_m(m)
    assert (bn, bm, threads, wgs) == (16, mp, 256, -(-n // 16))
    assert rz.rz_fp8_gemm_workspace_bytes(m, n, k) == 0
    g = np.random.Generator(np.random.PCG64(m * 5 + n + k))
    a8 = _codes(g, (mp, k))
    a8[m:] = 0
    w8 = _codes(g, (n, k))
    sc = np.array([1.0, 0.017, 0, 0], np.float32)
    wdq = np.float32(0.0071)
    y = host(rz.rz_fp8_gemm(dev(a8), dev(w8), m, dev(sc), float(wdq)))
    assert y.shape == (m, n)
    check_gemm(y, a8, w8, m, sc[1], wdq)


@pytest.mark.parametrize("m,n,k,full", [
    (80, 200, 768, True),      # 64x32 tiles, 3 K chunks of 1 pair, ragged m and n
    (65, 1000, 2816, True),    # 64x32 tiles, 10 uneven chunks
    (96, 4608, 3584, False),   # 64x32 tiles, 2 chunks of 7 pairs
    (300, 520, 2048, True),    # 64x32 tiles, 5 uneven chunks
    (600, 1000, 3584, False),  # 128x128 tiles, 6 uneven chunks, ragged m and n
    (512, 3584, 3584, False),  # 128x128 tiles in 2 chunks
    (4096, 512, 3584, False),  # 128x128 tiles in 2 chunks
])
def test_gemm_edge_split_plans(rz, m, n, k, full):
    from tests.test_abi import _edge_plan
    bn, bm, wgs, need = _edge_plan(m, n, k)
    assert rz.rz_fp8_gemm_plan(m, n, k)[:2] == (bn, bm) and rz.rz_fp8_gemm_plan(m, n, k)[3] == wgs
    assert rz.rz_fp8_gemm_workspace_bytes(m, n, k) == need > 0
    g = np.random.Generator(np.random.PCG64(m * 3 + n + k))
    mp = fp8_path.pad_m(m)
    a8 = _codes(g, (mp, k))
    a8[m:] = 0
    w8 = _codes(g, (n, k))
    sc = np.array([1.0, 0.021, 0, 0], np.float32)
    wdq = np.float32(0.0093)
    A, Wd, S = dev(a8), dev(w8), dev(sc)
    rows = np.arange(m) if full else np.unique(np.concatenate([[0, 1, m - 1], g.choice(m, 45, replace=False)]))
    yr, tol = fp8_path.gemm_rows(a8, w8, rows, sc[1], wdq)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    # split K twice in a row on one workspace, then whole tiles without one
    for use_ws in (ws, ws, None):
        y = host(rz.rz_fp8_gemm(A, Wd, m, S, float(wdq), ws=use_ws))
        err = np.abs(y[rows].astype(np.float64) - yr)
        assert (err <= tol).all(), f"{(err > tol).sum()} out of bound (ws={use_ws is not None})"
    tiles = -(-mp // bm) * -(-n // bn)
    assert (host(ws[:4 * tiles]) == 0).all()  # arrival counters left at zero for the next call


def test_gemm_split_shapes_share_one_workspace(rz):
    # split-K shapes of different tile counts in turn on one workspace: the
    # counters sit in a region of fixed size, so one shape's partial sums
    # never land where the next shape keeps its counters
    shapes = [(2048, 512, 3584),   # 128x128 tiles: 64 tiles in 4 chunks
              (512, 3584, 3584),   # 112 tiles in 2 chunks
              (512, 512, 3584),    # 64x32 tiles: 128 tiles in 4 chunks
              (80, 200, 768),      # 64x32 tiles: 12 tiles in 3 chunks
              (2048, 512, 3584)]
    need = max(rz.rz_fp8_gemm_workspace_bytes(m, n, k) for m, n, k in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (m, n, k) in enumerate(shapes):
        assert rz.rz_fp8_gemm_workspace_bytes(m, n, k) > 0
        g = np.random.Generator(np.random.PCG64(31 * i + m + n))
        mp = fp8_path.pad_m(m)
        a8 = _codes(g, (mp, k))
        a8[m:] = 0
        w8 = _codes(g, (n, k))
        sc = np.array([1.0, 0.018, 0, 0], np.float32)
        wdq = np.float32(0.0077)
        rows = np.unique(np.concatenate([[0, m - 1], g.choice(m, min(m, 40), replace=False)]))
        yr, tol = fp8_path.gemm_rows(a8, w8, rows, sc[1], wdq)
        y = host(rz.rz_fp8_gemm(dev(a8), dev(w8), m, dev(sc), float(wdq), ws=ws))
        err = np.abs(y[rows].astype(np.float64) - yr)
        assert (err <= tol).all(), f"shape {(m, n, k)}: {(err > tol).sum()} out of bound"
        assert (host(ws[:1024]) == 0).all()  # every counter back at zero


def test_gemm_split_on_two_streams(rz):
    # split-K GEMMs issued alternately on two streams through the binding's
    # default workspace: each stream gets its own zero-filled workspace, so
    # their counters and partial sums never mix
    shapes = [(512, 3584, 3584), (80, 200, 768)]  # 128x128 in 2 chunks; 64x32 in 3 chunks
    cur = torch.cuda.current_stream()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for m, n, k in shapes:
        assert rz.rz_fp8_gemm_workspace_bytes(m, n, k) > 0
        g = np.random.Generator(np.random.PCG64(m + 5 * n + k))
        mp = fp8_path.pad_m(m)
        cases = []
        for si in range(2):
            a8 = _codes(g, (mp, k))
            a8[m:] = 0
            w8 = _codes(g, (n, k))
            sc = np.array([1.0, 0.017 + 0.001 * si, 0, 0], np.float32)
            cases.append((a8, w8, sc, dev(a8), dev(w8), dev(sc)))
        for st in streams:
            st.wait_stream(cur)  # inputs uploaded on the current stream
        outs = [[], []]
        for rep in range(3):
            for si, st in enumerate(streams):
                _, _, _, A, Wd, S = cases[si]
                with torch.cuda.stream(st):
                    outs[si].append(rz.rz_fp8_gemm(A, Wd, m, S, 0.0081, stream=st))
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, m - 1], g.choice(m, min(m, 40), replace=False)]))
        for si in range(2):
            a8, w8, sc = cases[si][:3]
            yr, tol = fp8_path.gemm_rows(a8, w8, rows, sc[1], np.float32(0.0081))
            for y in outs[si]:
                err = np.abs(y.cpu().numpy()[rows].astype(np.float64) - yr)
                assert (err <= tol).all(), f"shape {(m, n, k)} stream {si}: {(err > tol).sum()} out of bound"


@pytest.mark.parametrize("m,k,ns", [
    (2048, 1024, (18944, 18944)),    # gate/up widths: one launch of 1184 tiles (4 rounds, halves, quarters)
    (4096, 512, (3584, 512, 512)),   # q/k/v widths at M=4096: 288 tiles, one round + half tiles
    (2000, 512, (2560, 1024, 256)),  # ragged M, groups of 10, 4 and 1 n-tiles
    (4096, 512, (1024, 0, 512, 2048)),  # a skipped (zero-width) GEMM
])
def test_gemm_group_one_launch(rz, m, k, ns):
    # the grouped launch computes every element exactly as a single call's
    # interior kernel does; the widths here take the interior plan on their own
    # too, except where noted, and some rows are checked against the oracle
    g = np.random.Generator(np.random.PCG64(m + k + len(ns)))
    mp = fp8_path.pad_m(m)
    a8 = _codes(g, (mp, k))
    a8[m:] = 0
    ws_ = [_codes(g, (n, k)) for n in ns]
    scales = [0.25 + 0.125 * i for i in range(len(ns))]
    sc = np.array([1.0, 0.5, 0, 0], np.float32)
    A, S = dev(a8), dev(sc)
    print(f"gemm_group m={m} k={k} ns={ns}", flush=True)
    ys = rz.rz_fp8_gemm_group(A, m, S, [(dev(w), s) for w, s in zip(ws_, scales)])
    rows = np.unique(np.concatenate([[0, 1, m - 2, m - 1], g.integers(0, m, 12)]))
    for w, s, y in zip(ws_, scales, ys):
        n = w.shape[0]
        assert tuple(y.shape) == (m, n)
        if n == 0:
            continue
        got = host(y)
        single = host(rz.rz_fp8_gemm(A, dev(w), m, S, s))
        if rz.rz_fp8_gemm_plan(m, n, k)[:2] == (256, 256):
            np.testing.assert_array_equal(got, single)
        check_gemm(got[rows], a8[rows], w, len(rows), sc[1], np.float32(s))


def test_gemm_group_falls_back_to_single_calls(rz):
    # widths that are not multiples of 256, and a small M: one call per GEMM,
    # the same results as those calls
    for m, k, ns in ((2048, 512, (2500, 512)), (64, 512, (1024, 768)), (512, 3584, (3584, 512, 512))):
        g = np.random.Generator(np.random.PCG64(m * 3 + k))
        a8 = _codes(g, (fp8_path.pad_m(m), k))
        a8[m:] = 0
        ws_ = [_codes(g, (n, k)) for n in ns]
        sc = np.array([1.0, 0.75, 0, 0], np.float32)
        A, S = dev(a8), dev(sc)
        print(f"gemm_group fallback m={m} k={k} ns={ns}", flush=True)
        ys = rz.rz_fp8_gemm_group(A, m, S, [(dev(w), 0.5) for w in ws_])
        for w, y in zip(ws_, ys):
            np.testing.assert_array_equal(host(y), host(rz.rz_fp8_gemm(A, dev(w), m, S, 0.5)))


def test_gemm_identity_weight(rz):
    k, n, m = 512, 64, 37
    w8 = np.zeros((n, k), np.uint8)
    w8[np.arange(n), 3 * np.arange(n)] = 0x38
    g = np.random.Generator(np.random.PCG64(3))
    a8 = g.integers(0, 0x7F, size=(48, k)).astype(np.uint8)
    sc = np.array([1.0, 1.0, 0, 0], np.float32)
    y = host(rz.rz_fp8_gemm(dev(a8), dev(w8), m, dev(sc), 1.0))
    np.testing.assert_array_equal(y, e4m3.decode(a8[:m, 3 * np.arange(n)]).astype(np.float32))


def test_gemm_extreme_accumulation(rz):
    # K = 18944 products of 448 * -448: the largest sum the workloads allow
    k = 18944
    a8 = np.full((16, k), 0x7E, np.uint8)
    w8 = np.full((32, k), 0xFE, np.uint8)
    sc = np.array([1.0, 1.0, 0, 0], np.float32)
    y = host(rz.rz_fp8_gemm(dev(a8), dev(w8), 3, dev(sc), 1.0))
    assert (y == np.float32(-448.0 * 448.0 * k)).all()


def test_gemm_zero_activation_gives_zero(rz):
    w8, scale, _ = rz.rz_fp8_pack_weight(W.Q4_K, dev(W.q4k_blocks(1, 64, 3584)), 64, 3584)
    x = np.zeros((37, 3584), np.float32)
    a8, sc = rz.rz_fp8_quant_act(dev(x))
    y = host(rz.rz_fp8_gemm(a8, w8, 37, sc, scale))
    assert (y == 0).all() and not np.signbit(y).any()
