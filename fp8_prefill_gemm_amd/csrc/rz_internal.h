// Host-side launchers shared between the kernel translation units and the
// C ABI layer (the GEMM's are in rz_gemm.h).  Every launcher assumes its arguments were validated by the
// caller (api.hip) and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rz_gemm.h"

namespace rz {

// Workspace layout (bytes): [0, 32768) partial absmax keys (uint32; one
// reduction uses at most kMaxPartials of them, a pack set up to kWsPartials
// in total), [32768, 33024) the weight path's {a, q, dq, 0}, one record per
// weight of a pack set (room for 16), [33024, 33056) the activation
// quantisation's record (kQuantTail: {a, q, dq, 0}).  Nothing in it needs
// to start at zero: every call writes what it reads.
constexpr int kMaxPartials = 2048;
constexpr int kWsPartials = 8192;
constexpr size_t kWsScaleOffset = 4 * (size_t)kWsPartials;
constexpr size_t kWsQuantOffset = kWsScaleOffset + 256;
constexpr size_t kQuantTail = 32;  // float {a, q, dq, 0}, padded
constexpr size_t kWsBytes = kWsQuantOffset + 256;

// A set of weights packed by one pass-1 and one pass-2 launch (kquant.hip):
// weight i owns pass-1 workgroups [g1[i], g1[i+1]) (and their partial keys,
// at most kMaxPartials) and pass-2 workgroups [g2[i], g2[i+1]);
// g1[count] <= kWsPartials.
constexpr int kMaxPackSet = 8;
struct PackSet {
    int count;
    int qtype[kMaxPackSet];
    const uint8_t* blocks[kMaxPackSet];
    uint64_t nb[kMaxPackSet];
    uint8_t* w_fp8[kMaxPackSet];
    float* host[kMaxPackSet];
    uint32_t ticket[kMaxPackSet];
    int g1[kMaxPackSet + 1];
    int g2[kMaxPackSet + 1];
};

// ---- kquant.hip
hipError_t launch_dequant_f32(int qtype, const uint8_t* blocks, uint64_t nblocks, float* out,
                              hipStream_t st);
// Three kernels: partial absmax keys, one workgroup per weight that
// reduces them and publishes the scales, then the encode.  Writes
// {a, q, dq, 0} as floats at ws + kWsScaleOffset and, when host_scale is
// not null, {a, q, dq} to that coherent host memory followed by `ticket`
// (as a uint32, release order) in its fourth word, before the codes.
hipError_t launch_pack(int qtype, const uint8_t* blocks, uint64_t nblocks, uint8_t* w_fp8,
                       uint8_t* ws, float* host_scale, uint32_t ticket, hipStream_t st);
// w_fp8 may be null: then only the scales are computed and published (the
// pass over the blocks for the absmax, no codes written).
// Pass-1 workgroups (= partial keys) of one weight.
int pack_absmax_groups(int qtype, uint64_t nb);
// The two passes for `count` (<= kMaxPackSet) weights whose pass-1 groups
// add up to at most kWsPartials; weight i's scales go to ws +
// kWsScaleOffset + 16 i and, when host_scale[i] is not null, to that host
// memory followed by ticket[i].
hipError_t launch_pack_set(int count, const int* qtype, const uint8_t* const* blocks, const uint64_t* nb,
                           uint8_t* const* w_fp8, uint8_t* ws, float* const* host_scale, const uint32_t* ticket,
                           hipStream_t st);

// FP16 comparator: the K-quant weight dequantised and rounded to fp16
// [nb*256] (row-major [N][K]).
hipError_t launch_fp16_pack(int qtype, const uint8_t* blocks, uint64_t nb, uint16_t* out, hipStream_t st);

// ---- kqgemm.hip
// Y[m][n] = dec(A) * dec(E4M3(RN(w * w_q)))^T * (act_scale[1] * w_dq), the
// weight codes made from the K-quant blocks inside the GEMM.
hipError_t launch_kquant_fp8_gemm(const uint8_t* a_fp8, uint32_t m, const float* act_scale, int qtype,
                                  const uint8_t* blocks, uint32_t n, uint32_t k, float w_q, float w_dq, float* y,
                                  hipStream_t st);

// ---- actquant.hip
// Three kernels: partial absmax keys, one workgroup that reduces them and
// publishes {a, dq} to act_scale and {a, q, dq, 0} to tail, then the
// encode.  partial: kMaxPartials uint32; tail: kQuantTail bytes.
hipError_t launch_quant_act(const float* x, uint64_t count_real, uint64_t count_total,
                            uint8_t* a_fp8, float* act_scale, uint32_t* partial, uint8_t* tail, hipStream_t st);
// Partial keys launch_quant_act writes for count_real elements (<= kMaxPartials).
int quant_act_partials(uint64_t count_real);
// Device address of the quantisation scratch array (kQuantScratchBytes) of
// the current device, looked up once per device: the partial keys, then the
// scale record.
constexpr size_t kQuantScratchBytes = 4 * (size_t)kMaxPartials + kQuantTail;
hipError_t quant_scratch_ptr(uint8_t** ptr);
// fp16 copy of x (count_real values, then zeros up to count_total).
hipError_t launch_fp16_convert(const float* x, uint64_t count_real, uint64_t count_total, uint16_t* out,
                               hipStream_t st);
hipError_t launch_absmax(const float* x, uint64_t count, float* out, uint8_t* ws, hipStream_t st);
hipError_t launch_encode(const float* x, uint64_t count, float scale, uint8_t* out,
                         hipStream_t st);
hipError_t launch_scales(const float* a, uint64_t count, float* q, float* dq, hipStream_t st);

// ---- q8gemm.hip
// Q8_1 blocks (36 bytes per 32 values) of `count` fp32 values (a multiple of 32).
hipError_t launch_q8_1_quant(const float* x, uint64_t count, uint8_t* out, hipStream_t st);
// y[m][n] = dequant(q8)[m][k] * dequant(Q4_K blocks)[n][k]^T.
hipError_t launch_q8_q4k_gemm(const uint8_t* q8, uint32_t m, const uint8_t* blocks, uint32_t n, uint32_t k,
                              float* y, hipStream_t st);

// ---- kgemv.hip
// y[m][n] = x[m][k] * dequant(blocks)^T for 1 <= m <= RZ_KGEMV_MAX_M.
hipError_t launch_kquant_gemv(int qtype, const uint8_t* blocks, uint32_t n, uint32_t k, const float* x,
                              uint32_t m, float* y, hipStream_t st);

}  // namespace rz
