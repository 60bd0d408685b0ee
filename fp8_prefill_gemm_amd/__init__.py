"""Python binding of librz_fp8: the FP8 prefill matmul path on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
``librz_fp8.so`` (built for gfx950 by ``fp8_prefill_gemm_amd.build``); torch
tensors are used for device memory and the current HIP stream.  There is no
fallback: if the library is missing, importing the binding's functions
raises.

The functions carry the names of the C entry points (include/rz_fp8.h) and
take torch tensors instead of raw pointers; outputs that are not passed in
are allocated on the input's device.
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

Q4_K = 12
Q6_K = 14
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210}

_STATUS = {0: "RZ_OK", -1: "RZ_ERR_NULL", -2: "RZ_ERR_QTYPE", -3: "RZ_ERR_SHAPE",
           -4: "RZ_ERR_ALIGN", -5: "RZ_ERR_HIP", -6: "RZ_ERR_VALUE"}


class RzError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None

_vp, _u32, _u64, _i32, _f32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int, ctypes.c_float
_SIGS = {
    "rz_block_bytes": (ctypes.c_size_t, [_i32]),
    "rz_weight_bytes": (ctypes.c_size_t, [_i32, _u32, _u32]),
    "rz_pad_m": (_u32, [_u32]),
    "rz_workspace_bytes": (ctypes.c_size_t, []),
    "rz_fp8_pack_weight": (_i32, [_i32, _vp, _u32, _u32, _vp, _vp, _vp, _vp, _vp]),
    "rz_fp8_pack_weights": (_i32, [_u32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "rz_fp8_quant_act": (_i32, [_vp, _u32, _u32, _vp, _vp, _vp, _vp]),
    "rz_fp8_quant_act_noalloc": (_i32, [_vp, _u32, _u32, _vp, _vp, _vp]),
    "rz_fp8_gemm": (_i32, [_vp, _vp, _u32, _u32, _u32, _vp, _f32, _vp, _vp, ctypes.c_size_t, _vp]),
    "rz_fp8_gemm_workspace_bytes": (ctypes.c_size_t, [_u32, _u32, _u32]),
    "rz_fp8_gemm_group": (_i32, [_vp, _u32, _u32, _vp, _u32, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "rz_q8_1_bytes": (ctypes.c_size_t, [_u32, _u32]),
    "rz_q8_1_quant": (_i32, [_vp, _u32, _u32, _vp, _vp]),
    "rz_q8_q4k_gemm": (_i32, [_vp, _u32, _vp, _u32, _u32, _vp, _vp]),
    "rz_fp16_pack_weight": (_i32, [_i32, _vp, _u32, _u32, _vp, _vp]),
    "rz_fp16_convert_act": (_i32, [_vp, _u32, _u32, _vp, _vp]),
    "rz_fp16_gemm": (_i32, [_vp, _vp, _u32, _u32, _u32, _vp, _vp]),
    "rz_dequant_f32": (_i32, [_i32, _vp, _u32, _u32, _vp, _vp]),
    "rz_absmax_f32": (_i32, [_vp, _u64, _vp, _vp, _vp]),
    "rz_e4m3_encode": (_i32, [_vp, _u64, _f32, _vp, _vp]),
    "rz_fp8_scales": (_i32, [_vp, _u64, _vp, _vp, _vp]),
    "rz_fp8_gemm_plan": (_i32, [_u32, _u32, _u32, _vp]),
    "rz_kquant_gemv": (_i32, [_i32, _vp, _u32, _u32, _vp, _u32, _vp, _vp]),
    "rz_route_kquant_gemv": (_i32, [_u32]),
    "rz_kquant_weight_scale": (_i32, [_i32, _vp, _u32, _u32, _vp, _vp, _vp, _vp, _vp]),
    "rz_kquant_fp8_gemm": (_i32, [_vp, _u32, _vp, _i32, _vp, _u32, _u32, _f32, _f32, _vp, _vp]),
    "rz_status_string": (ctypes.c_char_p, [_i32]),
    "rz_last_error_string": (ctypes.c_char_p, []),
    "rz_version": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGS)


def lib_path() -> str:
    return _build.LIB_PATH


def lib() -> ctypes.CDLL:
    """Load librz_fp8.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it with `python -m fp8_prefill_gemm_amd.build` "
                "(hipcc, gfx950); there is no fallback implementation")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise RzError(status, lib().rz_last_error_string().decode(errors="replace"))


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _torch_stream(stream, device):
    """The torch stream a call runs on: `stream`, or the device's current one."""
    torch = _torch()
    return torch.cuda.current_stream(device) if stream is None else stream


def _stream(stream, device):
    return ctypes.c_void_p(_torch_stream(stream, device).cuda_stream)


def _empty(shape, dtype, device, stream=None):
    """A new device tensor allocated on the call's stream.

    The caching allocator ties a block to the stream it was allocated on:
    once the tensor is freed, the block is reused only by work ordered after
    what that stream has queued, so a temporary freed when a call returns
    (a workspace, an output the caller drops) is never handed to a new
    allocation while the call's kernels still use it."""
    torch = _torch()
    with torch.cuda.stream(_torch_stream(stream, device)):
        return torch.empty(shape, dtype=dtype, device=device)


def _require_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("rz_fp8 works on device (cuda/hip) tensors only")


def workspace(device, stream=None) -> "torch.Tensor":
    """A fresh device workspace of rz_workspace_bytes() bytes, allocated on
    `stream` (default: the device's current stream)."""
    torch = _torch()
    return _empty(lib().rz_workspace_bytes(), torch.uint8, device, stream)


_ws_cache = {}


def _call_workspace(device, stream=None):
    """The workspace the calls below use when given none: one
    rz_workspace_bytes() buffer per (device, stream), made on that stream.
    Calls on one stream are ordered, so they can share it; calls on
    different streams get their own."""
    torch = _torch()
    dev = torch.device(device)
    st = _torch_stream(stream, dev)
    key = (dev.index or 0, st.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None:
        buf = workspace(dev, st)
        _ws_cache[key] = buf
    return buf


def rz_pad_m(m: int) -> int:
    return int(lib().rz_pad_m(m))


def rz_weight_bytes(qtype: int, n: int, k: int) -> int:
    return int(lib().rz_weight_bytes(qtype, n, k))


def rz_workspace_bytes() -> int:
    return int(lib().rz_workspace_bytes())


def rz_fp8_gemm_plan(m: int, n: int, k: int) -> tuple[int, int, int, int]:
    out = (ctypes.c_int32 * 4)()
    _check(lib().rz_fp8_gemm_plan(m, n, k, ctypes.cast(out, ctypes.c_void_p)))
    return tuple(out)


# ------------------------------------------------------------- entry points

def rz_fp8_pack_weight(qtype: int, blocks, n: int, k: int, w_fp8=None, ws=None, stream=None):
    """-> (w_fp8 uint8 [n][k], w_scale float, w_absmax float).  Returns once the
    scale is on the host; w_fp8 is complete for later work on the stream."""
    torch = _torch()
    _require_cuda(blocks, w_fp8, ws)
    dev = blocks.device
    if w_fp8 is None:
        w_fp8 = _empty((n, k), torch.uint8, dev, stream)
    if ws is None:
        ws = _call_workspace(dev, stream)
    scale = ctypes.c_float()
    amax = ctypes.c_float()
    _check(lib().rz_fp8_pack_weight(qtype, _ptr(blocks), n, k, _ptr(w_fp8), ctypes.addressof(scale),
                                    ctypes.addressof(amax), _ptr(ws), _stream(stream, dev)))
    return w_fp8, scale.value, amax.value


def rz_fp8_pack_weights(weights, ws=None, stream=None):
    """weights: sequence of (qtype, blocks, n, k, w_fp8 or None) -> list of
    (w_fp8, w_scale, w_absmax), packed in one call with one host wait."""
    torch = _torch()
    weights = list(weights)
    cnt = len(weights)
    if cnt == 0:
        return []
    dev = weights[0][1].device
    outs = []
    for q, b, n, k, w8 in weights:
        _require_cuda(b, w8)
        outs.append(_empty((n, k), torch.uint8, b.device, stream) if w8 is None else w8)
    if ws is None:
        ws = _call_workspace(dev, stream)
    _require_cuda(ws)
    qt = (ctypes.c_int * cnt)(*[w[0] for w in weights])
    bp = (ctypes.c_void_p * cnt)(*[_ptr(w[1]) for w in weights])
    nn = (ctypes.c_uint32 * cnt)(*[w[2] for w in weights])
    kk = (ctypes.c_uint32 * cnt)(*[w[3] for w in weights])
    op = (ctypes.c_void_p * cnt)(*[_ptr(o) for o in outs])
    sc = (ctypes.c_float * cnt)()
    am = (ctypes.c_float * cnt)()
    _check(lib().rz_fp8_pack_weights(cnt, ctypes.addressof(qt), ctypes.addressof(bp), ctypes.addressof(nn),
                                     ctypes.addressof(kk), ctypes.addressof(op), ctypes.addressof(sc),
                                     ctypes.addressof(am), _ptr(ws), _stream(stream, dev)))
    return [(outs[i], sc[i], am[i]) for i in range(cnt)]


def rz_fp8_quant_act(x, a_fp8=None, act_scale=None, ws=None, stream=None):
    """x fp32 [m][k] -> (a_fp8 uint8 [pad_m(m)][k], act_scale float32[2] = {absmax, dq})."""
    torch = _torch()
    _require_cuda(x, a_fp8, act_scale, ws)
    m, k = x.shape
    dev = x.device
    if a_fp8 is None:
        a_fp8 = _empty((rz_pad_m(m), k), torch.uint8, dev, stream)
    if act_scale is None:
        act_scale = _empty(4, torch.float32, dev, stream)
    if ws is None:
        ws = _call_workspace(dev, stream)
    _check(lib().rz_fp8_quant_act(_ptr(x), m, k, _ptr(a_fp8), _ptr(act_scale), _ptr(ws),
                                  _stream(stream, dev)))
    return a_fp8, act_scale


def rz_fp8_quant_act_noalloc(x, a_fp8, act_scale, stream=None):
    """rz_fp8_quant_act into caller-provided outputs, with the library's
    per-GPU scratch array instead of a workspace: the call allocates
    nothing (calls that overlap on one GPU race on that array)."""
    _require_cuda(x, a_fp8, act_scale)
    m, k = x.shape
    _check(lib().rz_fp8_quant_act_noalloc(_ptr(x), m, k, _ptr(a_fp8), _ptr(act_scale),
                                          _stream(stream, x.device)))
    return a_fp8, act_scale


_gemm_ws = {}


def gemm_workspace(device, nbytes: int, stream=None):
    """A zero-filled GEMM workspace of at least `nbytes`, cached per (device,
    stream).

    The GEMM returns its workspace to the zero state, so one buffer serves
    every call issued in order on one stream; calls on different streams
    must not share one (their split-K counters and partial sums would race),
    so each stream gets its own.  The buffer is allocated and zero-filled on
    that stream, so the fill is ordered before the stream's GEMMs."""
    torch = _torch()
    dev = torch.device(device)
    st = _torch_stream(stream, dev)
    key = (dev.index or 0, st.cuda_stream)
    buf = _gemm_ws.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(st):
            buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _gemm_ws[key] = buf
    return buf


def rz_fp8_gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib().rz_fp8_gemm_workspace_bytes(m, n, k))


def rz_fp8_gemm(a_fp8, w_fp8, m: int, act_scale, w_scale: float, y=None, stream=None, ws="auto"):
    """-> y fp32 [m][n] = dec(a)[:m] @ dec(w)^T * act_scale[1] * w_scale.

    ws: "auto" (a cached zero-filled workspace sized for the shape), None (no
    workspace: no K split), or a zero-filled uint8 device tensor."""
    torch = _torch()
    _require_cuda(a_fp8, w_fp8, act_scale, y)
    n, k = w_fp8.shape
    dev = w_fp8.device
    if y is None:
        y = _empty((m, n), torch.float32, dev, stream)
    if isinstance(ws, str):
        need = rz_fp8_gemm_workspace_bytes(m, n, k)
        ws = gemm_workspace(dev, need, stream) if need else None
    _require_cuda(ws)
    _check(lib().rz_fp8_gemm(_ptr(a_fp8), _ptr(w_fp8), m, n, k, _ptr(act_scale), float(w_scale),
                             _ptr(y), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream, dev)))
    return y


KGEMV_MAX_M = 8


def rz_kquant_gemv(qtype: int, blocks, n: int, k: int, x, y=None, stream=None):
    """-> y fp32 [m][n] = x @ dequant(blocks)^T, straight from the K-quant
    blocks (x fp32 [m][k], 1 <= m <= KGEMV_MAX_M)."""
    torch = _torch()
    _require_cuda(blocks, x, y)
    m = x.shape[0]
    if y is None:
        y = _empty((m, n), torch.float32, blocks.device, stream)
    _check(lib().rz_kquant_gemv(qtype, _ptr(blocks), n, k, _ptr(x), m, _ptr(y), _stream(stream, blocks.device)))
    return y


def rz_route_kquant_gemv(m: int) -> bool:
    """True when a batch of m rows should take rz_kquant_gemv rather than the
    FP8 path (activation quantisation + FP8 GEMM)."""
    return bool(lib().rz_route_kquant_gemv(m))


def rz_kquant_weight_scale(qtype: int, blocks, n: int, k: int, ws=None, stream=None):
    """-> (w_q, w_dq, w_absmax) of a K-quant weight, without its FP8 codes."""
    _require_cuda(blocks, ws)
    dev = blocks.device
    if ws is None:
        ws = _call_workspace(dev, stream)
    q, dq, amax = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    _check(lib().rz_kquant_weight_scale(qtype, _ptr(blocks), n, k, ctypes.addressof(q), ctypes.addressof(dq),
                                        ctypes.addressof(amax), _ptr(ws), _stream(stream, dev)))
    return q.value, dq.value, amax.value


def rz_kquant_fp8_gemm(a_fp8, m: int, act_scale, qtype: int, blocks, n: int, k: int, w_q: float, w_dq: float,
                       y=None, stream=None):
    """-> y fp32 [m][n] = dec(a)[:m] @ dec(E4M3(RN(w * w_q)))^T * act_scale[1] * w_dq,
    the weight codes made from the K-quant blocks inside the GEMM."""
    torch = _torch()
    _require_cuda(a_fp8, act_scale, blocks, y)
    dev = blocks.device
    if y is None:
        y = _empty((m, n), torch.float32, dev, stream)
    _check(lib().rz_kquant_fp8_gemm(_ptr(a_fp8), m, _ptr(act_scale), qtype, _ptr(blocks), n, k, float(w_q),
                                    float(w_dq), _ptr(y), _stream(stream, dev)))
    return y


def rz_fp8_gemm_group(a_fp8, m: int, act_scale, weights, ys=None, stream=None, ws="auto"):
    """weights: sequence of (w_fp8 uint8 [n][k], w_scale) sharing the FP8
    activation a_fp8 -> list of y fp32 [m][n], in one launch when the shapes
    allow it (see include/rz_fp8.h)."""
    torch = _torch()
    weights = list(weights)
    cnt = len(weights)
    _require_cuda(a_fp8, act_scale, *[w for w, _ in weights])
    k = a_fp8.shape[1]
    dev = a_fp8.device
    if ys is None:
        ys = [_empty((m, w.shape[0]), torch.float32, dev, stream) for w, _ in weights]
    _require_cuda(*ys)
    if isinstance(ws, str):
        need = max([rz_fp8_gemm_workspace_bytes(m, w.shape[0], k) for w, _ in weights] + [0])
        ws = gemm_workspace(dev, need, stream) if need else None
    _require_cuda(ws)
    wp = (ctypes.c_void_p * max(cnt, 1))(*[_ptr(w) for w, _ in weights])
    nn = (ctypes.c_uint32 * max(cnt, 1))(*[w.shape[0] for w, _ in weights])
    sc = (ctypes.c_float * max(cnt, 1))(*[float(s) for _, s in weights])
    yp = (ctypes.c_void_p * max(cnt, 1))(*[_ptr(y) for y in ys])
    _check(lib().rz_fp8_gemm_group(_ptr(a_fp8), m, k, _ptr(act_scale), cnt, ctypes.addressof(wp),
                                   ctypes.addressof(nn), ctypes.addressof(sc), ctypes.addressof(yp), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream, dev)))
    return ys


def rz_q8_1_quant(x, q8=None, stream=None):
    """x fp32 [m][k] -> Q8_1 blocks, uint8 [m][k/32][36]."""
    torch = _torch()
    _require_cuda(x, q8)
    m, k = x.shape
    if q8 is None:
        q8 = _empty((m, k // 32, 36), torch.uint8, x.device, stream)
    _check(lib().rz_q8_1_quant(_ptr(x), m, k, _ptr(q8), _stream(stream, x.device)))
    return q8


def rz_q8_q4k_gemm(q8, m: int, blocks, n: int, k: int, y=None, stream=None):
    """-> y fp32 [m][n] = dequant(Q8_1 activation) @ dequant(Q4_K weight)^T."""
    torch = _torch()
    _require_cuda(q8, blocks, y)
    if y is None:
        y = _empty((m, n), torch.float32, blocks.device, stream)
    _check(lib().rz_q8_q4k_gemm(_ptr(q8), m, _ptr(blocks), n, k, _ptr(y), _stream(stream, blocks.device)))
    return y


def rz_fp16_pack_weight(qtype: int, blocks, n: int, k: int, w_f16=None, stream=None):
    """-> fp16 [n][k]: the dequantised weight rounded to fp16 (the FP16
    comparator's weight cache)."""
    torch = _torch()
    _require_cuda(blocks, w_f16)
    if w_f16 is None:
        w_f16 = _empty((n, k), torch.float16, blocks.device, stream)
    _check(lib().rz_fp16_pack_weight(qtype, _ptr(blocks), n, k, _ptr(w_f16), _stream(stream, blocks.device)))
    return w_f16


def rz_fp16_convert_act(x, a_f16=None, stream=None):
    """x fp32 [m][k] -> fp16 [pad_m(m)][k] (pad rows zero)."""
    torch = _torch()
    _require_cuda(x, a_f16)
    m, k = x.shape
    if a_f16 is None:
        a_f16 = _empty((rz_pad_m(m), k), torch.float16, x.device, stream)
    _check(lib().rz_fp16_convert_act(_ptr(x), m, k, _ptr(a_f16), _stream(stream, x.device)))
    return a_f16


def rz_fp16_gemm(a_f16, w_f16, m: int, y=None, stream=None):
    """-> y fp32 [m][n] = a_f16[:m] @ w_f16^T (fp32 accumulation, no scales)."""
    torch = _torch()
    _require_cuda(a_f16, w_f16, y)
    n, k = w_f16.shape
    if y is None:
        y = _empty((m, n), torch.float32, w_f16.device, stream)
    _check(lib().rz_fp16_gemm(_ptr(a_f16), _ptr(w_f16), m, n, k, _ptr(y), _stream(stream, w_f16.device)))
    return y


def rz_dequant_f32(qtype: int, blocks, n: int, k: int, out=None, stream=None):
    torch = _torch()
    _require_cuda(blocks, out)
    if out is None:
        out = _empty((n, k), torch.float32, blocks.device, stream)
    _check(lib().rz_dequant_f32(qtype, _ptr(blocks), n, k, _ptr(out), _stream(stream, blocks.device)))
    return out


def rz_absmax_f32(x, out=None, ws=None, stream=None):
    torch = _torch()
    _require_cuda(x, out, ws)
    if out is None:
        out = _empty(4, torch.float32, x.device, stream)
    if ws is None:
        ws = workspace(x.device, stream)
    _check(lib().rz_absmax_f32(_ptr(x), x.numel(), _ptr(out), _ptr(ws), _stream(stream, x.device)))
    return out


def rz_e4m3_encode(x, scale: float, out=None, stream=None):
    torch = _torch()
    _require_cuda(x, out)
    if out is None:
        out = _empty(x.shape, torch.uint8, x.device, stream)
    _check(lib().rz_e4m3_encode(_ptr(x), x.numel(), float(scale), _ptr(out), _stream(stream, x.device)))
    return out


def rz_fp8_scales(absmax, q=None, dq=None, stream=None):
    torch = _torch()
    _require_cuda(absmax, q, dq)
    if q is None:
        q = _empty(absmax.shape, absmax.dtype, absmax.device, stream)
    if dq is None:
        dq = _empty(absmax.shape, absmax.dtype, absmax.device, stream)
    _check(lib().rz_fp8_scales(_ptr(absmax), absmax.numel(), _ptr(q), _ptr(dq),
                               _stream(stream, absmax.device)))
    return q, dq
