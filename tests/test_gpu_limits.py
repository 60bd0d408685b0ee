"""GPU tests at the boundary's size limits: the largest K the GEMM accepts
on each plan that small M takes, the interior kernel with more than 2^32
outputs or activation bytes, and an activation quantisation and a weight
pack of more than 2^32 elements (element indices past 32 bits).  The inputs
are built so that the oracle checks them on a few distinct values or rows:
all-1.0 codes make every partial sum of the GEMM an integer below 2^24
(exact in fp32, in any order and split), and the large tensors repeat one
row except for one that sets the absmax."""
import numpy as np
import pytest

import workloads as W
from oracle import e4m3, fp8_path

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rz():
    import fp8_prefill_gemm_amd as rz
    rz.lib()  # loud failure if the HIP library is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return rz


def host(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("m,n", [(3, 64), (40, 64), (100, 64), (200, 256)])  # GEMV, skinny, 64x32, 128x128 tiles
def test_gemm_largest_k(rz, m, n):
    k = (1 << 24) - 256  # RZ_MAX_GEMM_K
    mp = rz.rz_pad_m(m)
    print(f"gemm at the largest K: m={m} n={n} k={k} plan={rz.rz_fp8_gemm_plan(m, n, k)}", flush=True)
    a8 = torch.full((mp, k), 0x38, dtype=torch.uint8, device="cuda")  # 1.0
    w8 = torch.full((n, k), 0x38, dtype=torch.uint8, device="cuda")
    sc = torch.tensor([1.0, 1.0, 0.0, 0.0], dtype=torch.float32, device="cuda")
    y = rz.rz_fp8_gemm(a8, w8, m, sc, 1.0)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (m, n)
    assert bool((y == float(k)).all()), f"{int((y != float(k)).sum())} outputs differ from {k}"
    del a8, w8, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m,n,k", [(65536, 65536, 512),    # 2^32 outputs (17 GB): 65536 interior tiles
                                   (300000, 256, 16384)])  # a 4.9 GB activation, 1172 m-tiles
def test_gemm_interior_past_2_32(rz, m, n, k):
    mp = rz.rz_pad_m(m)
    assert rz.rz_fp8_gemm_plan(m, n, k)[:2] == (256, 256)
    print(f"interior gemm m={m} n={n} k={k}", flush=True)
    a8 = torch.full((mp, k), 0x38, dtype=torch.uint8, device="cuda")
    w8 = torch.full((n, k), 0x38, dtype=torch.uint8, device="cuda")
    sc = torch.tensor([1.0, 1.0, 0.0, 0.0], dtype=torch.float32, device="cuda")
    y = rz.rz_fp8_gemm(a8, w8, m, sc, 0.5)
    torch.cuda.synchronize()
    assert bool((y == float(k) * 0.5).all())
    del a8, w8, y
    torch.cuda.empty_cache()


def test_quant_act_past_2_32_elements(rz):
    k = 3584
    m = (1 << 32) // k + 16  # 4.29e9 + elements
    print(f"quant_act m={m} k={k} ({m * k} elements)", flush=True)
    x = torch.full((m, k), 0.7431640625, dtype=torch.float32, device="cuda")
    x[m - 1, k - 1] = -3.25  # the absmax, at the last element
    x[m // 2, 17] = float("nan")  # ignored by the absmax, encoded as 0x7E
    a8, sc = rz.rz_fp8_quant_act(x)
    torch.cuda.synchronize()
    vals = np.array([0.7431640625, -3.25, np.nan], np.float32)
    q, dq = fp8_path.scales_from_absmax(fp8_path.absmax(vals))
    c = e4m3.encode_scaled(vals, q)
    s = host(sc)
    assert s[0] == np.float32(3.25) and s[1].view(np.uint32) == np.float32(dq).view(np.uint32)
    flat = a8.view(-1)
    assert int(flat[m * k - 1]) == int(c[1])
    assert int(flat[(m // 2) * k + 17]) == int(c[2])
    flat[m * k - 1] = int(c[0])
    flat[(m // 2) * k + 17] = int(c[0])
    assert bool((flat[: m * k] == int(c[0])).all())
    assert bool((flat[m * k:] == 0).all())  # pad rows
    del x, a8, flat
    torch.cuda.empty_cache()


@pytest.mark.parametrize("qtype", [W.Q4_K, W.Q6_K])
def test_pack_past_2_32_weights(rz, qtype):
    k = 3584
    n = (1 << 32) // k + 8
    bb = 144 if qtype == W.Q4_K else 210
    kb = k // 256
    two = W.weight_blocks(qtype, 9700 + qtype, 2, k)  # row 0 everywhere, row 1 last
    if qtype == W.Q4_K:
        two.reshape(2, kb, bb)[1, :, 0:2] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)  # larger d
    else:
        two.reshape(2, kb, bb)[1, :, 208:210] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    r8, rdq, ra = fp8_path.pack_weight(qtype, two, 2, k)
    print(f"pack qtype={qtype} n={n} k={k} ({n * k} weights)", flush=True)
    row = torch.from_numpy(two.reshape(2, kb * bb)).cuda()
    blocks = row[0].repeat(n, 1)
    blocks[n - 1] = row[1]
    w8, scale, amax = rz.rz_fp8_pack_weight(qtype, blocks.view(-1), n, k)
    torch.cuda.synchronize()
    assert np.float32(amax).view(np.uint32) == np.float32(ra).view(np.uint32)
    assert np.float32(scale).view(np.uint32) == np.float32(rdq).view(np.uint32)
    r0 = torch.from_numpy(r8[0]).cuda()
    assert bool((w8[: n - 1] == r0).all())
    assert bool((w8[n - 1] == torch.from_numpy(r8[1]).cuda()).all())
    del blocks, w8
    torch.cuda.empty_cache()
