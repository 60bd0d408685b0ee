"""C ABI contract of librz_fp8.so, checked without a GPU.

The library must load, export every function include/rz_fp8.h declares, and
reject bad arguments before any HIP call (so these run on a CPU-only host).
The pointers used here are fake addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import fp8_prefill_gemm_amd as rz

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rz_fp8.h")

RZ_OK, RZ_ERR_NULL, RZ_ERR_QTYPE, RZ_ERR_SHAPE, RZ_ERR_ALIGN, RZ_ERR_HIP, RZ_ERR_VALUE = 0, -1, -2, -3, -4, -5, -6
P = 0x7F0000001000      # fake, 16-byte aligned, never dereferenced
P2 = 0x7F0000002000
P3 = 0x7F0000003000
BAD = 0x7F0000001004     # 4-byte but not 16-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rz_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rz.lib_path()):
        pytest.skip("librz_fp8.so not built")
    return rz.lib()


def test_exports_every_declared_symbol(L):
    decl = declared_functions()
    assert len(decl) >= 15
    for name in decl:
        assert hasattr(L, name), name
    assert set(decl) == set(rz.EXPORTED)


def test_sizes(L):
    assert L.rz_block_bytes(12) == 144 and L.rz_block_bytes(14) == 210 and L.rz_block_bytes(2) == 0
    assert L.rz_weight_bytes(12, 18944, 3584) == 18944 * 14 * 144
    assert L.rz_weight_bytes(14, 3584, 18944) == 3584 * 74 * 210
    assert L.rz_weight_bytes(12, 4, 300) == 0
    assert [L.rz_pad_m(m) for m in (0, 1, 4, 16, 17, 37, 1000, 2048)] == [0, 16, 16, 16, 32, 48, 1008, 2048]
    assert L.rz_workspace_bytes() >= 8192 + 16
    assert L.rz_version().decode().startswith("rz_fp8")
    assert L.rz_status_string(-3).decode() == "invalid shape"


def _err(L):
    return L.rz_last_error_string().decode()


def test_pack_validation(L):
    f = L.rz_fp8_pack_weight
    host = ctypes.c_float()
    h = ctypes.addressof(host)
    assert f(12, None, 4, 256, P2, h, None, P3, None) == RZ_ERR_NULL
    assert f(12, P, 4, 256, None, h, None, P3, None) == RZ_ERR_NULL
    assert f(12, P, 4, 256, P2, None, None, P3, None) == RZ_ERR_NULL
    assert f(12, P, 4, 256, P2, h, None, None, None) == RZ_ERR_NULL
    assert f(2, P, 4, 256, P2, h, None, P3, None) == RZ_ERR_QTYPE
    assert "unsupported qtype" in _err(L)
    assert f(12, P, 4, 300, P2, h, None, P3, None) == RZ_ERR_SHAPE
    assert f(14, P, 4, 0, P2, h, None, P3, None) == RZ_ERR_SHAPE
    assert f(12, P, 0, 256, P2, h, None, P3, None) == RZ_ERR_SHAPE
    assert f(12, P, 1 << 30, 1 << 20, P2, h, None, P3, None) == RZ_ERR_SHAPE
    assert f(12, BAD, 4, 256, P2, h, None, P3, None) == RZ_ERR_ALIGN
    assert f(12, P, 4, 256, BAD, h, None, P3, None) == RZ_ERR_ALIGN
    assert host.value == 0.0  # outputs untouched on error


def test_pack_weights_validation(L):
    arr = lambda ct, vals: (ct * len(vals))(*vals)
    V = ctypes.c_void_p

    def f(cnt, q, b, n, k, o, sc=True, ws=P3):
        scale = (ctypes.c_float * max(cnt, 1))()
        return L.rz_fp8_pack_weights(cnt, q, b, n, k, o, scale if sc else None, None, ws, None)
    q = arr(ctypes.c_int, [12, 14])
    b = arr(V, [P, P2])
    n = arr(ctypes.c_uint32, [8, 4])
    k = arr(ctypes.c_uint32, [256, 512])
    o = arr(V, [P2, P])
    assert f(0, None, None, None, None, None) == RZ_OK
    assert f(2, None, b, n, k, o) == RZ_ERR_NULL
    assert f(2, q, b, n, k, o, sc=False) == RZ_ERR_NULL
    assert f(2, q, b, n, k, o, ws=None) == RZ_ERR_NULL
    assert f(2, q, arr(V, [P, None]), n, k, o) == RZ_ERR_NULL
    assert "weight 1" in _err(L)
    assert f(2, arr(ctypes.c_int, [12, 3]), b, n, k, o) == RZ_ERR_QTYPE
    assert f(2, q, b, n, arr(ctypes.c_uint32, [256, 300]), o) == RZ_ERR_SHAPE
    assert f(2, q, b, arr(ctypes.c_uint32, [0, 4]), k, o) == RZ_ERR_SHAPE
    assert "weight 0" in _err(L)
    assert f(2, q, arr(V, [P, BAD]), n, k, o) == RZ_ERR_ALIGN
    assert f(2, q, b, n, k, o, ws=BAD) == RZ_ERR_ALIGN


def test_quant_act_validation(L):
    f = L.rz_fp8_quant_act
    assert f(None, 4, 256, P2, P3, P, None) == RZ_ERR_NULL
    assert f(P, 4, 256, None, P3, P, None) == RZ_ERR_NULL
    assert f(P, 4, 256, P2, None, P, None) == RZ_ERR_NULL
    assert f(P, 4, 256, P2, P3, None, None) == RZ_ERR_NULL
    assert f(P, 4, 100, P2, P3, P, None) == RZ_ERR_SHAPE
    assert f(P, 4, 0, P2, P3, P, None) == RZ_ERR_SHAPE
    assert f(BAD, 4, 256, P2, P3, P, None) == RZ_ERR_ALIGN
    assert f(P, 4, 256, BAD, P3, P, None) == RZ_ERR_ALIGN
    assert f(P, 4, 256, P2, P3 + 2, P, None) == RZ_ERR_ALIGN
    assert f(None, 0, 256, None, None, P, None) == RZ_ERR_NULL  # the scale output is always written


def test_gemm_validation(L):
    def f(a, w, m, n, k, sc, ws_, y, ws=None, wsb=0):
        return L.rz_fp8_gemm(a, w, m, n, k, sc, ws_, y, ws, wsb, None)
    assert f(None, P2, 4, 8, 256, P3, 1.0, P) == RZ_ERR_NULL
    assert f(P, None, 4, 8, 256, P3, 1.0, P) == RZ_ERR_NULL
    assert f(P, P2, 4, 8, 256, None, 1.0, P) == RZ_ERR_NULL
    assert f(P, P2, 4, 8, 256, P3, 1.0, None) == RZ_ERR_NULL
    assert f(P, P2, 4, 8, 255, P3, 1.0, P) == RZ_ERR_SHAPE
    assert f(P, P2, 4, 8, 0, P3, 1.0, P) == RZ_ERR_SHAPE
    assert f(P, P2, 4, 8, 1 << 24, P3, 1.0, P) == RZ_ERR_SHAPE
    assert f(P, P2, 1 << 20, 1 << 20, 256, P3, 1.0, P) == RZ_ERR_SHAPE
    assert f(BAD, P2, 4, 8, 256, P3, 1.0, P) == RZ_ERR_ALIGN
    assert f(P, P2, 4, 8, 256, P3, 1.0, BAD) == RZ_ERR_ALIGN
    assert f(P, P2, 4, 8, 256, P3, 1.0, P, BAD, 1024) == RZ_ERR_ALIGN
    assert f(P, P2, 4, 8, 256, P3, float("nan"), P) == RZ_ERR_VALUE
    assert f(P, P2, 4, 8, 256, P3, float("inf"), P) == RZ_ERR_VALUE
    # empty products are no-ops that touch nothing (no device needed)
    assert f(P, P2, 0, 8, 256, P3, 1.0, P) == RZ_OK
    assert f(P, P2, 4, 0, 256, P3, 1.0, P) == RZ_OK
    assert f(None, None, 0, 8, 256, None, 1.0, None) == RZ_OK
    assert f(None, None, 0, 8, 255, None, 1.0, None) == RZ_ERR_SHAPE


def test_kquant_gemv_validation(L):
    def f(q, b, n, k, x, m, y):
        return L.rz_kquant_gemv(q, b, n, k, x, m, y, None)
    assert f(12, None, 8, 256, P2, 1, P3) == RZ_ERR_NULL
    assert f(14, P, 8, 256, None, 1, P3) == RZ_ERR_NULL
    assert f(12, P, 8, 256, P2, 1, None) == RZ_ERR_NULL
    assert f(2, P, 8, 256, P2, 1, P3) == RZ_ERR_QTYPE
    assert f(12, P, 8, 300, P2, 1, P3) == RZ_ERR_SHAPE
    assert f(12, P, 8, 0, P2, 1, P3) == RZ_ERR_SHAPE
    assert f(12, P, 8, 256, P2, 9, P3) == RZ_ERR_SHAPE
    assert "exceeds 8" in _err(L)
    assert f(12, P, 1 << 30, 1 << 10, P2, 1, P3) == RZ_ERR_SHAPE
    assert f(12, BAD, 8, 256, P2, 1, P3) == RZ_ERR_ALIGN
    assert f(14, P, 8, 256, BAD, 1, P3) == RZ_ERR_ALIGN
    assert f(14, P, 8, 256, P2, 1, BAD) == RZ_ERR_ALIGN
    # empty products are no-ops that touch nothing (no device needed)
    assert f(12, None, 8, 256, None, 0, None) == RZ_OK
    assert f(14, None, 0, 256, None, 4, None) == RZ_OK
    assert f(12, None, 0, 255, None, 4, None) == RZ_ERR_SHAPE


def test_kquant_fp8_gemm_validation(L):
    def f(a, m, sc, q, b, n, k, wq, wdq, y):
        return L.rz_kquant_fp8_gemm(a, m, sc, q, b, n, k, wq, wdq, y, None)
    assert f(None, 4, P3, 12, P2, 8, 256, 1.0, 1.0, P) == RZ_ERR_NULL
    assert f(P, 4, None, 12, P2, 8, 256, 1.0, 1.0, P) == RZ_ERR_NULL
    assert f(P, 4, P3, 14, None, 8, 256, 1.0, 1.0, P) == RZ_ERR_NULL
    assert f(P, 4, P3, 12, P2, 8, 256, 1.0, 1.0, None) == RZ_ERR_NULL
    assert f(P, 4, P3, 3, P2, 8, 256, 1.0, 1.0, P) == RZ_ERR_QTYPE
    assert f(P, 4, P3, 12, P2, 8, 300, 1.0, 1.0, P) == RZ_ERR_SHAPE
    assert f(P, 4, P3, 12, P2, 8, 1 << 24, 1.0, 1.0, P) == RZ_ERR_SHAPE
    assert f(P, 1 << 20, P3, 12, P2, 1 << 20, 256, 1.0, 1.0, P) == RZ_ERR_SHAPE
    assert f(BAD, 4, P3, 12, P2, 8, 256, 1.0, 1.0, P) == RZ_ERR_ALIGN
    assert f(P, 4, P3, 14, BAD, 8, 256, 1.0, 1.0, P) == RZ_ERR_ALIGN
    assert f(P, 4, P3, 12, P2, 8, 256, 1.0, 1.0, BAD) == RZ_ERR_ALIGN
    assert f(P, 4, P3, 12, P2, 8, 256, float("nan"), 1.0, P) == RZ_ERR_VALUE
    assert f(P, 4, P3, 12, P2, 8, 256, 1.0, float("inf"), P) == RZ_ERR_VALUE
    # empty products are no-ops that touch nothing (no device needed)
    assert f(None, 0, None, 12, None, 8, 256, 1.0, 1.0, None) == RZ_OK
    assert f(None, 4, None, 14, None, 0, 256, 1.0, 1.0, None) == RZ_OK
    assert f(None, 0, None, 12, None, 8, 255, 1.0, 1.0, None) == RZ_ERR_SHAPE


def test_route_kquant_gemv(L):
    # GEMV route for 1..4 rows, the FP8 path above; host only
    assert [L.rz_route_kquant_gemv(m) for m in (0, 1, 2, 3, 4, 5, 8, 16, 2048)] == [0, 1, 1, 1, 1, 0, 0, 0, 0]
    assert [rz.rz_route_kquant_gemv(m) for m in (1, 4, 5)] == [True, True, False]


def test_kquant_weight_scale_validation(L):
    q, dq = ctypes.c_float(), ctypes.c_float()
    aq, adq = ctypes.addressof(q), ctypes.addressof(dq)

    def f(qt, b, n, k, wq, wdq, ws):
        return L.rz_kquant_weight_scale(qt, b, n, k, wq, wdq, None, ws, None)
    assert f(12, None, 8, 256, aq, adq, P) == RZ_ERR_NULL
    assert f(12, P, 8, 256, None, adq, P) == RZ_ERR_NULL
    assert f(12, P, 8, 256, aq, None, P) == RZ_ERR_NULL
    assert f(12, P, 8, 256, aq, adq, None) == RZ_ERR_NULL
    assert f(5, P, 8, 256, aq, adq, P) == RZ_ERR_QTYPE
    assert f(14, P, 8, 100, aq, adq, P) == RZ_ERR_SHAPE
    assert f(14, P, 0, 256, aq, adq, P) == RZ_ERR_SHAPE
    assert f(12, BAD, 8, 256, aq, adq, P) == RZ_ERR_ALIGN
    assert f(12, P, 8, 256, aq, adq, BAD) == RZ_ERR_ALIGN


def test_gemm_group_validation(L):
    V = ctypes.c_void_p
    arr = lambda ct, vals: (ct * len(vals))(*vals)

    def f(a, m, k, sc, cnt, w, n, s, y):
        return L.rz_fp8_gemm_group(a, m, k, sc, cnt, w, n, s, y, None, 0, None)
    w = arr(V, [P, P2])
    n = arr(ctypes.c_uint32, [256, 512])
    s = arr(ctypes.c_float, [1.0, 2.0])
    y = arr(V, [P3, P])
    assert f(P, 4, 256, P3, 0, None, None, None, None) == RZ_OK
    assert f(P, 0, 256, P3, 2, w, n, s, y) == RZ_OK
    assert f(P, 4, 256, P3, 5, w, n, s, y) == RZ_ERR_SHAPE
    assert f(P, 4, 300, P3, 2, w, n, s, y) == RZ_ERR_SHAPE
    assert f(None, 4, 256, P3, 2, w, n, s, y) == RZ_ERR_NULL
    assert f(P, 4, 256, None, 2, w, n, s, y) == RZ_ERR_NULL
    assert f(P, 4, 256, P3, 2, None, n, s, y) == RZ_ERR_NULL
    assert f(P, 4, 256, P3, 2, arr(V, [P, None]), n, s, y) == RZ_ERR_NULL
    assert "gemm 1" in _err(L)
    assert f(BAD, 4, 256, P3, 2, w, n, s, y) == RZ_ERR_ALIGN
    assert f(P, 4, 256, P3, 2, w, n, s, arr(V, [P3, BAD])) == RZ_ERR_ALIGN
    assert f(P, 4, 256, P3, 2, w, n, arr(ctypes.c_float, [1.0, float("nan")]), y) == RZ_ERR_VALUE
    # zero-width GEMMs are skipped: nothing to launch, no device needed
    assert f(P, 4, 256, P3, 2, arr(V, [None, None]), arr(ctypes.c_uint32, [0, 0]), s,
             arr(V, [None, None])) == RZ_OK


def test_gemm_workspace_sizes(L):
    # the GEMV and skinny kernels (padded M <= 64) need none; split-K with 64x32 tiles:
    # 1 KB of arrival counters (256, whatever the shape) + 12 tiles x 2 chunks of 64x32 fp32
    assert L.rz_fp8_gemm_workspace_bytes(16, 256, 512) == 0
    assert L.rz_fp8_gemm_workspace_bytes(80, 256, 512) == 1024 + 12 * 2 * 64 * 32 * 4
    assert L.rz_fp8_gemm_workspace_bytes(0, 256, 512) == 0
    assert L.rz_fp8_gemm_workspace_bytes(2048, 256, 300) == 0
    # interior-tile plans need none; the 128x128 split needs counters + 2 chunks of 112 tiles
    assert L.rz_fp8_gemm_workspace_bytes(2048, 18944, 3584) == 0
    assert L.rz_fp8_gemm_workspace_bytes(2048, 3584, 18944) == 0
    assert L.rz_fp8_gemm_workspace_bytes(512, 3584, 3584) == 1024 + 112 * 2 * 128 * 128 * 4


def test_diagnostics_validation(L):
    assert L.rz_dequant_f32(12, None, 4, 256, P, None) == RZ_ERR_NULL
    assert L.rz_dequant_f32(3, P, 4, 256, P2, None) == RZ_ERR_QTYPE
    assert L.rz_dequant_f32(14, P, 4, 512 + 16, P2, None) == RZ_ERR_SHAPE
    assert L.rz_dequant_f32(14, BAD, 4, 512, P2, None) == RZ_ERR_ALIGN
    assert L.rz_absmax_f32(None, 4, P2, P3, None) == RZ_ERR_NULL
    assert L.rz_absmax_f32(BAD, 4, P2, P3, None) == RZ_ERR_ALIGN
    assert L.rz_absmax_f32(P, (1 << 36) + 1, P2, P3, None) == RZ_ERR_SHAPE
    assert L.rz_e4m3_encode(P, 4, 1.0, None, None) == RZ_ERR_NULL
    assert L.rz_e4m3_encode(None, 0, 1.0, None, None) == RZ_OK
    assert L.rz_e4m3_encode(P, 4, 1.0, BAD, None) == RZ_ERR_ALIGN
    assert L.rz_fp8_scales(None, 4, P2, P3, None) == RZ_ERR_NULL
    assert L.rz_fp8_scales(P, 0, P2, P3, None) == RZ_OK
    out = (ctypes.c_int32 * 4)()
    assert L.rz_fp8_gemm_plan(2048, 18944, 3584, ctypes.cast(out, ctypes.c_void_p)) == RZ_OK
    assert out[0] * out[1] > 0 and out[2] % 64 == 0 and out[3] > 0
    assert L.rz_fp8_gemm_plan(16, 256, 300, ctypes.cast(out, ctypes.c_void_p)) == RZ_ERR_SHAPE


def test_plans_cover_shapes(L):
    # every workload shape gets a plan whose tiles cover the output
    for m, n, k in [(16, 256, 512), (512, 3584, 3584), (512, 512, 3584), (2048, 18944, 3584),
                    (2048, 3584, 18944), (4096, 18944, 3584), (1, 4608, 3584), (1000, 4608, 3584),
                    (2000, 18900, 3584), (200, 65636, 512)]:
        bn, bm, threads, wgs = rz.rz_fp8_gemm_plan(m, n, k)
        mp = rz.rz_pad_m(m)
        tiles = -(-mp // bm) * -(-n // bn)
        interior = (bn, bm) == (256, 256) and mp >= 256 and 256 <= n < 1 << 21 and k >= 512 and tiles >= 64
        if interior:
            assert wgs == 256  # persistent: one workgroup per CU
        else:
            assert (bn, bm, wgs) == _edge_plan(m, n, k)[:3]
            assert wgs >= tiles
        assert threads in (64, 128, 256, 512)


def _edge_plan(m, n, k, cus=256):
    """(BN, BM, workgroups, workspace bytes) of a plan that is not interior
    (256 CUs): the GEMV kernel (4 weight rows per workgroup) when M <= 3;
    the skinny kernel (16 weight rows per workgroup) when M_pad <= 64; 256x256 tiles from 256 tiles on, unsplit; else 128x128 tiles
    split into s = min(256 // tiles, pairs // 2) K chunks if M_pad >= 128 and
    that gives >= 128 workgroups; else 64x32 tiles in s = min(512 // tiles,
    pairs) chunks.  A split rounds the tiles up to a multiple of 8 (XCDs);
    its workspace is a fixed 1 KB of arrival counters (up to 256 tiles) and
    the partial sums."""
    mp = -(-m // 16) * 16
    pairs = k // 256
    if m <= 3:
        return 4, mp, -(-n // 4), 0
    if mp <= 64:
        return 16, mp, -(-n // 16), 0

    def tiles(bn, bm):
        return -(-mp // bm) * -(-n // bn)

    if tiles(256, 256) >= 256:
        return 256, 256, tiles(256, 256), 0
    t = tiles(128, 128)
    s = max(1, min(256 // t, pairs // 2))
    if mp >= 128 and t * s >= 128:
        bn, bm = 128, 128
    else:
        bn, bm = 64, 32
        t = tiles(64, 32)
        s = max(1, min(512 // t, pairs))
    if s == 1:
        return bn, bm, t, 0
    return bn, bm, 8 * -(-t // 8) * s, 1024 + t * s * bn * bm * 4  # 256 counters, then the partials


def _interior_items(T, W):
    """Per-workgroup item lists of the persistent interior kernel, as the
    kernel builds them: XCD x (workgroups w with w % 8 == x, j = w // 8)
    takes a contiguous run of Tx tiles; R = Tx // W whole rounds (tile
    r*W + j), the L left over as 2L half tiles when R > 0 or 2L <= W (else
    whole, one per workgroup j < L); when W < 2L <= 1.5 W the halves beyond
    the first W are split into quarters, one per workgroup; halves and
    quarters handed out odd workgroups first, an odd one running its
    quarter, or else its first half, before its whole tiles.
    -> {(x, j): [("w", tile) | ("h", tile, half) | ("q", tile, half, quarter)]}"""
    out = {}
    tall, trem = divmod(T, 8)
    for x in range(8):
        first = x * tall + min(x, trem)
        tx = tall + (1 if x < trem else 0)
        r, l = divmod(tx, W)
        halves = r > 0 or 2 * l <= W
        h = 2 * l if halves else 0
        nq = 0
        if h > W and 2 * (h - W) <= W:
            nq, h = 2 * (h - W), W
        for j in range(W):
            hr = j // 2 if j % 2 else W // 2 + j // 2
            items = []
            hh = h + hr // 2
            quarter = ("q", first + r * W + hh // 2, hh % 2, hr % 2) if hr < nq else None
            early_q = j % 2 == 1 and quarter is not None
            early = j % 2 == 1 and hr < h and not early_q
            if early_q:
                items.append(quarter)
            if early:
                items.append(("h", first + r * W + hr // 2, hr % 2))
            items += [("w", first + i * W + j) for i in range(r)]
            if not halves and j < l:
                items.append(("w", first + r * W + j))
            for q in range(hr + (W if early else 0), h, W):
                items.append(("h", first + r * W + q // 2, q % 2))
            if quarter is not None and not early_q:
                items.append(quarter)
            out[(x, j)] = items
    return out


def _interior_group_m(tiles_m, tiles_n, W):
    """Group height of the interior kernel's tile order, as its launch picks
    it: 8 (or tiles_m if fewer); when an XCD's run fits one round, the height
    of 4, 2, 1 below that which gives the run fewer distinct m- plus n-tiles."""
    gm = min(tiles_m, 8)
    tx = -(-tiles_m * tiles_n // 8)
    if tx <= W:
        cost = gm + -(-tx // gm)
        for a in (4, 2, 1):
            if a < gm and a + -(-tx // a) < cost:
                gm, cost = a, a + -(-tx // a)
    return gm


def _grouped_origin(t, tiles_m, tiles_n, gm_full):
    """(n-tile, m-tile) of tile t in the grouped order: groups of gm_full
    m-tiles (the last may be shorter), m fastest inside a group."""
    gidx, tin = divmod(t, gm_full * tiles_n)
    first_m = gidx * gm_full
    gm = min(tiles_m - first_m, gm_full)
    return tin // gm, first_m + tin % gm


@pytest.mark.parametrize("tiles_m,tiles_n,W,want", [(8, 14, 32, 4), (16, 14, 32, 4), (8, 148, 32, 8),
                                                   (4, 18, 32, 4), (8, 74, 32, 8), (3, 100, 32, 3),
                                                   (16, 148, 32, 8), (8, 14, 38, 4), (1, 64, 32, 1)])
def test_interior_group_height(tiles_m, tiles_n, W, want):
    gm = _interior_group_m(tiles_m, tiles_n, W)
    assert gm == want
    T = tiles_m * tiles_n
    origins = [_grouped_origin(t, tiles_m, tiles_n, gm) for t in range(T)]
    assert sorted(origins) == [(n, m) for n in range(tiles_n) for m in range(tiles_m)]
    # distinct m- and n-tiles of each XCD's run: never more than with groups of 8
    tall, trem = divmod(T, 8)
    for x in range(8):
        first = x * tall + min(x, trem)
        run = range(first, first + tall + (1 if x < trem else 0))
        def spread(g):
            o = [_grouped_origin(t, tiles_m, tiles_n, g) for t in run]
            return len({n for n, _ in o}) + len({m for _, m in o})
        if -(-T // 8) <= W:
            assert spread(gm) <= spread(min(tiles_m, 8)) + 1


def test_interior_plan_examples(L):
    # the persistent interior kernel: one workgroup per CU (256 without a device)
    for m, n, k in [(2048, 18944, 3584), (2048, 3584, 18944), (4096, 18944, 3584), (768, 25600, 512),
                    (2048, 37888, 3584)]:
        assert rz.rz_fp8_gemm_plan(m, n, k)[:4] == (256, 256, 256, 256)


@pytest.mark.parametrize("tiles_m,tiles_n", [(8, 74), (8, 148), (8, 14), (16, 14), (16, 148), (3, 100), (2, 74),
                                             (1, 64), (8, 32), (5, 13)])
@pytest.mark.parametrize("W", [32, 2, 3, 31, 38])  # workgroups per XCD: CUs / 8 (32 on MI355X; odd when harvested)
def test_interior_schedule_covers_tiles_once(tiles_m, tiles_n, W):
    T = tiles_m * tiles_n
    items = _interior_items(T, W)
    seen = {}
    for lst in items.values():
        for it in lst:
            key = (it[1],) + tuple(it[2:])
            seen[key] = seen.get(key, 0) + 1
    assert all(v == 1 for v in seen.values())
    for t in range(T):  # whole, or both halves, each half whole or as its two quarters
        halves = [((t, hf) in seen) + ((t, hf, 0) in seen and (t, hf, 1) in seen) for hf in (0, 1)]
        assert ((t,) in seen) != (halves == [1, 1])
        assert halves in ([0, 0], [1, 1])
        for hf in (0, 1):
            assert ((t, hf, 0) in seen) == ((t, hf, 1) in seen)
            assert not ((t, hf) in seen and (t, hf, 0) in seen)
    # load in quarter-tile units: at most one tile above the average
    size = {"w": 4, "h": 2, "q": 1}
    load = {wj: sum(size[it[0]] for it in lst) for wj, lst in items.items()}
    assert max(load.values()) <= -(-4 * T // (8 * W)) + 4
    # no workgroup runs two halves where quarters can take the excess
    tall, trem = divmod(T, 8)
    for (x, j), lst in items.items():
        tx = tall + (1 if x < trem else 0)
        r, l = divmod(tx, W)
        if r > 0 and 2 * l <= W + W // 2:
            assert sum(it[0] == "h" for it in lst) <= 1 and sum(it[0] == "q" for it in lst) <= 1
    # with whole rounds, every odd workgroup that has a quarter runs it first,
    # else its first half
    for (x, j), lst in items.items():
        if j % 2 and any(it[0] == "w" for it in lst):
            if any(it[0] == "q" for it in lst):
                assert lst[0][0] == "q"
            elif any(it[0] == "h" for it in lst):
                assert lst[0][0] == "h"



def test_binding_refuses_host_tensors(L):
    import torch
    with pytest.raises(ValueError):
        rz.rz_fp8_quant_act(torch.zeros(4, 256))
