"""rz_fp8_quant_act_noalloc against rz_fp8_quant_act (GPU).

The no-allocation variant uses the library's per-GPU scratch array instead
of a workspace.  Two calls in a row, the second on a smaller input whose
absmax is far below the first's (so keys left in the scratch by the first
call would show in its scale), must give exactly the bytes and scales of
the workspace entry point and of the oracle.
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


def _quant_both(rz, x_h):
    m, k = x_h.shape
    x = torch.from_numpy(np.ascontiguousarray(x_h)).cuda()
    a_ref, sc_ref = rz.rz_fp8_quant_act(x)
    a8 = torch.full((rz.rz_pad_m(m), k), 0xA5, dtype=torch.uint8, device="cuda")  # stale pad rows
    sc = torch.full((4,), -1.0, dtype=torch.float32, device="cuda")
    rz.rz_fp8_quant_act_noalloc(x, a8, sc)
    torch.cuda.synchronize()
    return a8.cpu().numpy(), sc.cpu().numpy(), a_ref.cpu().numpy(), sc_ref.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice(rz):
    big = W.act_normal(9101, 1000, 3584) * np.float32(50.0)   # absmax about 250
    small = W.act_student_t(9102, 37, 512)
    small = (small / np.abs(small).max()).astype(np.float32)  # absmax 1
    for x_h in (big, small):
        m, k = x_h.shape
        print(f"\n  noalloc quant m={m} k={k}", flush=True)
        a8, sc, a_ref, sc_ref = _quant_both(rz, x_h)
        r8, ra, rdq = fp8_path.quant_act(x_h)
        assert sc[0] == sc_ref[0] == ra and sc[1] == sc_ref[1] == rdq
        np.testing.assert_array_equal(a8, a_ref)
        np.testing.assert_array_equal(a8, r8)


def test_noalloc_empty_and_rejects(rz):
    sc = torch.full((4,), -1.0, dtype=torch.float32, device="cuda")
    lib = rz.lib()
    import ctypes
    assert lib.rz_fp8_quant_act_noalloc(None, 0, 512, None, ctypes.c_void_p(sc.data_ptr()), None) == 0
    torch.cuda.synchronize()
    s = sc.cpu().numpy()
    assert s[0] == 0.0 and s[1] == np.float32(1.0 / 448.0)
    # k not a multiple of 256 is rejected before any launch
    x = torch.zeros((4, 300), dtype=torch.float32, device="cuda")
    a8 = torch.zeros((16, 300), dtype=torch.uint8, device="cuda")
    with pytest.raises(rz.RzError):
        rz.rz_fp8_quant_act_noalloc(x, a8, sc)
