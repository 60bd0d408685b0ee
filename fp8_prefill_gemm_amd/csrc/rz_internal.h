// Host-side launchers shared between the kernel translation units and the
// C ABI layer.  Every launcher assumes its arguments were validated by the
// caller (api.hip) and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// null, to that device-accessible host memory too.
hipError_t launch_pack(int qtype, const uint8_t* blocks, uint64_t nblocks, uint8_t* w_fp8,
                       uint8_t* ws, float* host_scale, hipStream_t st);

// ---- actquant.hip
hipError_t launch_quant_act(const float* x, uint64_t count_real, uint64_t count_total,
                            uint8_t* a_fp8, float* act_scale, uint8_t* ws, hipStream_t st);
hipError_t launch_absmax(const float* x, uint64_t count, float* out, uint8_t* ws, hipStream_t st);
hipError_t launch_encode(const float* x, uint64_t count, float scale, uint8_t* out,
                         hipStream_t st);
hipError_t launch_scales(const float* a, uint64_t count, float* q, float* dq, hipStream_t st);

// ---- gemm.hip, gemm_edge.hip
enum GemmKind { kGemmTiles = 0, kGemmMedium = 1, kGemmSmall = 2, kGemmLargeEdge = 3, kGemmSkinny = 4, kGemmGemv = 5 };
struct GemmPlan {
    int bn, bm, threads, workgroups, kind;
    // interior-tile plan: CUs, whole-tile rounds, tiles left over (run as
    // half tiles), workgroups for those half tiles
    int G, R, rem, half_workgroups;
    // edge-capable plans: K chunks per tile (1: no split)
    int s;
    size_t ws_bytes;  // workspace the plan needs (0: none)
};
GemmPlan plan_gemm(uint32_t m, uint32_t n, uint32_t k, int cus, bool split_allowed);
hipError_t launch_gemm(const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n,
                       uint32_t k, const float* act_scale, float w_scale, float* y, void* ws,
                       size_t ws_bytes, int cus, hipStream_t st);
// The kernels of every plan kind but kGemmTiles (gemm_edge.hip); ws holds
// the split-K counters and partial sums when p.s > 1.
hipError_t launch_gemm_edge(const GemmPlan& p, const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n,
                            uint32_t k, const float* act_scale, float w_scale, float* y, void* ws, hipStream_t st);
// Split-K workspace: arrival counters of the split tiles (one uint32 each),
// padded to 256 bytes; the partial sums follow.
inline size_t split_counter_bytes(int tiles) { return ((size_t)tiles * sizeof(unsigned) + 255) / 256 * 256; }

}  // namespace rz
