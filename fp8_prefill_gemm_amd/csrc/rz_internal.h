// Host-side launchers shared between the kernel translation units and the
// C ABI layer (the GEMM's are in rz_gemm.h).  Every launcher assumes its arguments were validated by the
// caller (api.hip) and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rz_gemm.h"

namespace rz {

// Workspace layout (bytes): [0, 8192) partial absmax keys (uint32, at most
// kMaxPartials), [8192, 8208) the weight path's {a, q, dq, 0}.
constexpr int kMaxPartials = 2048;
constexpr size_t kWsScaleOffset = 8192;
constexpr size_t kWsBytes = 8448;

// ---- kquant.hip
hipError_t launch_dequant_f32(int qtype, const uint8_t* blocks, uint64_t nblocks, float* out,
                              hipStream_t st);
// Two kernels: partial absmax keys, then (reduce + encode).  Writes
// {a, q, dq, 0} as floats at ws + kWsScaleOffset and, when host_scale is not
// null, {a, q, dq} to that coherent host memory followed by `ticket` (as a
// uint32, release order) in its fourth word, before the codes.
hipError_t launch_pack(int qtype, const uint8_t* blocks, uint64_t nblocks, uint8_t* w_fp8,
                       uint8_t* ws, float* host_scale, uint32_t ticket, hipStream_t st);

// ---- actquant.hip
hipError_t launch_quant_act(const float* x, uint64_t count_real, uint64_t count_total,
                            uint8_t* a_fp8, float* act_scale, uint8_t* ws, hipStream_t st);
hipError_t launch_absmax(const float* x, uint64_t count, float* out, uint8_t* ws, hipStream_t st);
hipError_t launch_encode(const float* x, uint64_t count, float scale, uint8_t* out,
                         hipStream_t st);
hipError_t launch_scales(const float* a, uint64_t count, float* q, float* dq, hipStream_t st);

// ---- kgemv.hip
// y[m][n] = x[m][k] * dequant(blocks)^T for 1 <= m <= RZ_KGEMV_MAX_M.
hipError_t launch_kquant_gemv(int qtype, const uint8_t* blocks, uint32_t n, uint32_t k, const float* x,
                              uint32_t m, float* y, hipStream_t st);

}  // namespace rz
