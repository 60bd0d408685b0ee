// Shared device definitions of the FP8 GEMM kernels (gemm.hip: interior
// 256x256 tiles; gemm_edge.hip: edge, small-tile and skinny kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rz {
namespace gemm {
typedef int v8i __attribute__((ext_vector_type(8)));
// Native 16-byte vector for staging: plain loads/stores (HIP's uint4 is a
// class whose copies become memcpy and keep the staging arrays in memory).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;
constexpr int kXcds = 8;

// 16-byte chunk swizzle of a 128-byte LDS row.  It depends only on row bits
// 0..4, so rows r and r + 32i share it (the per-thread LDS addresses of a
// stage then differ by immediates), and any 8 consecutive rows starting at
// a multiple of 8 (or 16 starting at a multiple of 16) hit distinct banks.
__device__ __forceinline__ int swz(int row) { return ((row ^ (row >> 3)) & 3) ^ (row & 4); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, uint32_t bytes) {
    // gfx9-family raw buffer: stride 0, range `bytes`, default data format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
}

// Origin of tile t of BN x BM tiles in the grouped order of a tiles_m x
// tiles_n region (groups of gm m-tiles, m fastest inside a group).
template <int BN, int BM>
__device__ __forceinline__ void grouped_origin_bb(int t, int tiles_m, int tiles_n, int gm_full, int& n0, int& m0) {
    const int per_group = gm_full * tiles_n;
    const int gidx = t / per_group;
    const int first_m = gidx * gm_full;
    const int gm = (tiles_m - first_m) < gm_full ? (tiles_m - first_m) : gm_full;
    const int tin = t - gidx * per_group;
    n0 = (tin / gm) * BN;
    m0 = (first_m + tin % gm) * BM;
}

}  // namespace gemm
}  // namespace rz
