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
typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// One 32x32 output block times one 32-byte K fragment per lane (src0: the
// rows of the result, src1: its columns; lane l holds row / column l % 32).
//   FP8 (E4M3 codes): one v_mfma_f32_32x32x64_f8f6f4, 64 K values;
//   F16: the fragment is 16 halves, so two v_mfma_f32_32x32x16_f16, on
//        bytes 0..15 and 16..31 of every lane's fragment.  Inside each MFMA
//        lanes 0-31 and 32-63 carry different K values; both operands come
//        from the same LDS chunks in the same lane order, so every K value
//        still meets its partner exactly once.
template <bool F16>
__device__ __forceinline__ v16f mma32(const v8i& src0, const v8i& src1, v16f acc) {
    if constexpr (F16) {
        const v8h a0 = __builtin_bit_cast(v8h, __builtin_shufflevector(src0, src0, 0, 1, 2, 3));
        const v8h a1 = __builtin_bit_cast(v8h, __builtin_shufflevector(src0, src0, 4, 5, 6, 7));
        const v8h b0 = __builtin_bit_cast(v8h, __builtin_shufflevector(src1, src1, 0, 1, 2, 3));
        const v8h b1 = __builtin_bit_cast(v8h, __builtin_shufflevector(src1, src1, 4, 5, 6, 7));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(src0, src1, acc, 0, 0, 0, 0, 0, 0);
    }
}

// Cache-policy operand of the raw buffer load/store builtins on gfx950: its
// bits 0 and 4 are the instruction's SC0 and SC1 scope bits.  Device scope
// (SC1): a store writes through the XCD's L2 and completes once it is
// visible to every XCD.  System scope (SC0 and SC1): a load misses in the
// L1 and the L2 and reads memory.  Bit 1 is NT, the streaming hint: the
// line is not kept in the caches for reuse.
constexpr int kScopeDevice = 16;
constexpr int kScopeSystem = 17;
constexpr int kNonTemporal = 2;

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

// Global -> registers: L x 16 bytes per thread of a [rows][128-byte] K-slice
// starting at column kb; rows at or past `limit` read as zero.
template <int L, int NT>
__device__ __forceinline__ void load_rows(u32x4 (&r)[L], const uint8_t* __restrict__ src, int row0,
                                          int limit, int K, int kb, int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int idx = tid + i * NT;
        const int gr = row0 + (idx >> 3);
        u32x4 v = (u32x4){0u, 0u, 0u, 0u};
        if (gr < limit) v = *reinterpret_cast<const u32x4*>(src + (size_t)gr * K + kb + ((idx & 7) << 4));
        r[i] = v;
    }
}

// Registers -> one LDS stage (128-byte rows, XOR-swizzled 16-byte chunks).
template <int L, int NT>
__device__ __forceinline__ void store_rows(uint8_t* dst, const u32x4 (&r)[L], int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int idx = tid + i * NT;
        const int row = idx >> 3;
        *reinterpret_cast<u32x4*>(dst + row * kBK + (((idx & 7) ^ swz(row)) << 4)) = r[i];
    }
}

// One 32-byte MFMA operand: row `row`, chunks c0 and c0+1 of a stage.
__device__ __forceinline__ v8i frag(const uint8_t* base, int row, int c0) {
    const uint8_t* r = base + row * kBK;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(r + ((c0 ^ swz(row)) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(r + (((c0 + 1) ^ swz(row)) << 4));
    return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// acc * scale -> Y for a TN x TM wave tile whose rows start at m0 and
// columns at n0.  With the activation as the MFMA A operand, acc[i][j][e]
// is row m0 + 32j + 8*(e/4) + 4*(lane/32) + e%4, column n0 + 32i + lane%32:
// a store instruction covers two 128-byte row segments.  Elements outside
// [0, M) x [0, N) are skipped.
template <int TN, int TM, int WTN, int WTM>
__device__ __forceinline__ void store_tile(const v16f (&acc)[TN][TM], float* __restrict__ Y, int M, int N, int m0,
                                           int n0, int lane, float s) {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int n = n0 + i * 32 + (lane & 31);
        if (n >= N) continue;
#pragma unroll
        for (int j = 0; j < TM; ++j) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + j * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (m < M) Y[(size_t)m * N + n] = acc[i][j][e] * s;
            }
        }
    }
}

}  // namespace gemm
}  // namespace rz
