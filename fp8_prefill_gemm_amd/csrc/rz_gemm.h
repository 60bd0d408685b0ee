// Host-side GEMM plan and launchers (gemm.hip, gemm_edge.hip), shared with
// the C ABI layer.  Every launcher assumes its arguments were validated by
// the caller (api.hip) and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rz {

enum GemmKind { kGemmTiles = 0, kGemmMedium = 1, kGemmSmall = 2, kGemmLargeEdge = 3, kGemmSkinny = 4, kGemmGemv = 5 };
struct GemmPlan {
    int bn, bm, threads, workgroups, kind;
    // interior-tile plan: CUs (the persistent grid, one workgroup each)
    int G;
    // edge-capable plans: tiles, K chunks per tile (1: no split)
    int rem, s;
    size_t ws_bytes;  // workspace the plan needs (0: none)
};
GemmPlan plan_gemm(uint32_t m, uint32_t n, uint32_t k, int cus, bool split_allowed);
// Weights and outputs of the GEMMs one interior launch computes on a shared
// activation: group g owns columns [n_end[g-1], n_end[g]) of the launch
// (n_end[-1] = 0), with its own weight rows, fp32 output [M][width] and
// weight scale.  With several groups every n_end is a multiple of 256.
constexpr int kMaxGemmGroups = 4;
struct GemmGroups {
    int count;
    int n_end[kMaxGemmGroups];
    const uint8_t* w[kMaxGemmGroups];
    float* y[kMaxGemmGroups];
    float w_scale[kMaxGemmGroups];
};
// The interior-tile kernel (p.kind == kGemmTiles, p planned for the total
// width n = G.n_end[G.count - 1]).
// f16: the operands are fp16 (k is then the row length in bytes) and there
// are no scales (act_scale unused, every w_scale 1).
hipError_t launch_interior(const GemmPlan& p, const uint8_t* a_fp8, const GemmGroups& G, uint32_t m, uint32_t n,
                           uint32_t k, const float* act_scale, hipStream_t st, bool f16);
hipError_t launch_gemm(const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n,
                       uint32_t k, const float* act_scale, float w_scale, float* y, void* ws,
                       size_t ws_bytes, int cus, hipStream_t st);
// The kernels of every plan kind but kGemmTiles (gemm_edge.hip); ws holds
// the split-K counters and partial sums when p.s > 1.
hipError_t launch_gemm_edge(const GemmPlan& p, const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n,
                            uint32_t k, const float* act_scale, float w_scale, float* y, void* ws, hipStream_t st);
// y[m][n] = a[m][k] * w[n][k]^T over fp16 operands (a: pad16(m) rows), fp32
// accumulation and output, no scales; k in elements.  Never splits K.
hipError_t launch_fp16_gemm(const uint16_t* a_f16, const uint16_t* w_f16, uint32_t m, uint32_t n, uint32_t k,
                            float* y, int cus, hipStream_t st);
// The edge-capable plans of launch_gemm_edge on fp16 operands (kb = row
// bytes; kinds kGemmLargeEdge, kGemmMedium, kGemmSmall; no split).
hipError_t launch_gemm_edge_fp16(const GemmPlan& p, const uint8_t* a, const uint8_t* w, uint32_t m, uint32_t n,
                                 uint32_t kb, float* y, hipStream_t st);
// Split-K workspace: one arrival counter (uint32) per tile in a region of
// fixed size at its start, the partial sums after it.  The region does not
// depend on the shape, so a workspace shared by calls of different shapes
// never finds one call's partial sums where the next keeps its counters
// (every call leaves its counters at zero; the partial sums are written
// before they are read).  Only plans with at most kSplitMaxTiles tiles split.
constexpr int kSplitMaxTiles = 256;
constexpr size_t kSplitCounterBytes = kSplitMaxTiles * sizeof(unsigned);

}  // namespace rz
