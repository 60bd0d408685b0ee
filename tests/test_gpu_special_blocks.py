"""Weight-path parity on K-quant blocks with arbitrary bytes (GPU).

The workload generators draw every f16 block scale from U[1e-3, 2e-2], so
the GPU's weight kernels would otherwise only meet positive normal scales.
Here the dequantisation and the pack (single and batched, and the
scale-only pass of the K-quant GEMM) run on blocks whose bytes are all
random, so d and dmin take every f16 pattern (negative, zero, subnormal,
+-Inf, NaN), and on blocks whose scales come from a list of finite special
values plus NaN.  Results must equal the oracle bit for bit: dequantised
values (a NaN only needs to be a NaN), absmax, scale and every E4M3 code.
This covers the pages' float max that ignores NaN and propagates Inf
(mod.rs page, ABSMAX_REDUCE_PTX), the Inf-absmax scales (q = 0, dq = Inf),
and the NaN/Inf products of the scaled conversion (F32_TO_E4M3_SCALED_PTX).
"""
import numpy as np
import pytest

import workloads as W
from oracle import fp8_path, kquant

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# f16 bit patterns: +-0, subnormals, smallest/largest normal, negative
# normals, a few ordinary magnitudes, and quiet NaNs of both signs
FINITE_SPECIAL_F16 = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x83FF, 0x0400, 0x8400, 0x7BFF, 0xFBFF,
                      0x3C00, 0xBC00, 0x2E66, 0xA2E6, 0x1400, 0x9400]
NAN_F16 = [0x7E00, 0xFE00, 0x7C01]


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


def _scale_offsets(qtype):
    return (0, 2) if qtype == W.Q4_K else (208,)


def random_blocks(qtype, n, k, seed, mode):
    """uint8 [n*(k/256)][block] with random bytes.

    mode "raw": every byte uniform (f16 scales of any pattern: one in 32 is
    NaN) and one block in 32 given a +-Inf scale, which random bytes almost
    never produce; "finite": scales drawn from FINITE_SPECIAL_F16, with one
    block in 64 given a NaN scale (so the absmax stays finite)."""
    per = W.BLOCK_BYTES[qtype]
    nb = n * (k // 256)
    g = np.random.Generator(np.random.PCG64(seed))
    b = g.integers(0, 256, size=(nb, per), dtype=np.uint8)
    if mode == "raw":
        for off in _scale_offsets(qtype):
            rows = np.flatnonzero(g.random(nb) < 1 / 32)
            pats = np.where(g.random(rows.size) < 0.5, 0x7C00, 0xFC00).astype(np.uint16)
            b[rows, off:off + 2] = pats.view(np.uint8).reshape(rows.size, 2)
    if mode == "finite":
        for off in _scale_offsets(qtype):
            pats = np.array(FINITE_SPECIAL_F16, np.uint16)[g.integers(0, len(FINITE_SPECIAL_F16), size=nb)]
            nan_rows = g.random(nb) < 1 / 64
            pats[nan_rows] = np.array(NAN_F16, np.uint16)[g.integers(0, len(NAN_F16), size=int(nan_rows.sum()))]
            b[:, off:off + 2] = pats.view(np.uint8).reshape(nb, 2)
    return b


def assert_same_f32(got, want):
    """Bit-equal, except that a NaN only has to meet a NaN."""
    gn, wn = np.isnan(got), np.isnan(want)
    np.testing.assert_array_equal(gn, wn)
    np.testing.assert_array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32))


CASES = [(W.Q4_K, 64, 1024, "raw"), (W.Q6_K, 64, 1024, "raw"), (W.Q4_K, 37, 3584, "finite"),
         (W.Q6_K, 37, 3584, "finite"), (W.Q4_K, 300, 512, "finite"), (W.Q6_K, 130, 768, "finite")]


@pytest.mark.parametrize("qtype,n,k,mode", CASES)
def test_dequant_special_scales(rz, qtype, n, k, mode):
    blocks = random_blocks(qtype, n, k, 7000 + n + qtype, mode)
    print(f"\n  dequant qtype={qtype} n={n} k={k} mode={mode}", flush=True)
    got = host(rz.rz_dequant_f32(qtype, dev(blocks), n, k))
    with np.errstate(all="ignore"):
        want = kquant.dequant(qtype, blocks, n, k)
    if mode == "raw":
        assert np.isnan(want).any() and np.isinf(want).any()  # the special cases are present
    assert_same_f32(got, want)


def _check_pack(qtype, blocks, n, k, w8, scale, amax):
    with np.errstate(all="ignore"):
        r8, rdq, ra = fp8_path.pack_weight(qtype, blocks, n, k)
    assert np.float32(amax).view(np.uint32) == ra.view(np.uint32), (amax, ra)
    assert np.float32(scale).view(np.uint32) == rdq.view(np.uint32), (scale, rdq)
    np.testing.assert_array_equal(host(w8), r8)
    return ra


@pytest.mark.parametrize("qtype,n,k,mode", CASES)
def test_pack_special_scales(rz, qtype, n, k, mode):
    blocks = random_blocks(qtype, n, k, 7100 + n + qtype, mode)
    print(f"\n  pack qtype={qtype} n={n} k={k} mode={mode}", flush=True)
    w8, scale, amax = rz.rz_fp8_pack_weight(qtype, dev(blocks), n, k)
    ra = _check_pack(qtype, blocks, n, k, w8, scale, amax)
    if mode == "raw":
        assert np.isinf(ra)  # the Inf absmax case: q = 0, dq = Inf
    else:
        assert np.isfinite(ra) and ra > 0
    # the scale-only pass of the K-quant GEMM gives the same scales
    q, dq, a2 = rz.rz_kquant_weight_scale(qtype, dev(blocks), n, k)
    assert np.float32(a2).view(np.uint32) == np.float32(amax).view(np.uint32)
    assert np.float32(dq).view(np.uint32) == np.float32(scale).view(np.uint32)
    assert np.float32(q) == fp8_path.scales_from_absmax(ra)[0]


def test_pack_weights_special_scales_mixed_set(rz):
    # every case above in one batched call (one mixed-type launch set)
    blocks = [random_blocks(q, n, k, 7200 + i, mode) for i, (q, n, k, mode) in enumerate(CASES)]
    print(f"\n  pack_weights: {len(CASES)} special-scale weights", flush=True)
    outs = rz.rz_fp8_pack_weights([(q, dev(b), n, k, None) for (q, n, k, _), b in zip(CASES, blocks)])
    for (q, n, k, _), b, (w8, scale, amax) in zip(CASES, blocks, outs):
        _check_pack(q, b, n, k, w8, scale, amax)
