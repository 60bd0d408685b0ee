// FP8 x FP8 GEMM with fp32 accumulation and the fused dual-scale epilogue.
//
// Source: realizar 0.8.4 source page cublas_prefill/gemm.rs,
// cublas_prefill_fp8_gemm: Y[M][N] = X[M][K] * W[N][K]^T where both operands
// are E4M3 codes, K-contiguous (leading dimension k for both), the products
// are summed without scaling and the output is multiplied by
// (act_absmax/448) * (w_absmax/448).  The pages run the GEMM in a closed
// library with an fp16 output and apply the activation scale in a second
// pass over the output (F16_TO_F32_ACT_SCALED_PTX on the mod.rs page); here
// the accumulator stays fp32 and both scales are applied in the epilogue,
// before the single fp32 store.
//
// gfx950 design.  The contraction runs on the CDNA4 f8f6f4 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, E4M3 x E4M3 -> fp32, unscaled form).  Both
// operands are K-contiguous, which is the native MFMA operand layout: lane l
// of a 32x32x64 MFMA supplies row l%32 and 32 consecutive K bytes at offset
// 32*(l/32), so no transpose is needed.  The weight is the MFMA "A" side
// (output rows = n) and the activation the "B" side (columns = m), so each
// lane ends with runs of 4 consecutive n of one output row m: 16-byte stores
// into the row-major fp32 output.
//
// A workgroup owns a BN x BM output tile and walks K in steps of 128 bytes
// with two LDS stages: the next step's global loads are issued before the
// current step's MFMAs and written to the other stage afterwards (one
// barrier per step).  LDS rows are 128 bytes; the 16-byte chunk c of row r
// is stored at c ^ ((r ^ r>>3) & 7) so that the MFMA operand reads (8 or 16
// consecutive rows, same chunk) and the stage writes hit distinct banks.
//
// Workgroup -> tile mapping is XCD-aware: the dispatcher sends workgroup w
// to XCD w % 8, so w is first remapped to a contiguous range of tiles per
// XCD; inside it tiles go m-fastest within groups of `group_m` m-tiles, so
// the workgroups that run together on one XCD share weight rows and
// activation rows through that XCD's L2.
#include "rz_device.h"
#include "rz_internal.h"

namespace rz {
namespace {

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

// Global -> registers for one operand of a stage: thread `tid` moves the
// 16-byte chunk (tid & 7) of rows (tid >> 3) + (NT/8)*i, i < L.  Buffer loads
// keep the addressing in one per-lane 32-bit offset (`voff` = (tid >> 3) * K
// + 16 * (tid & 7)) plus a uniform scalar offset (the stage's K offset plus
// i rows-steps), so no per-load 64-bit address stays live in VGPRs.  `rsrc`
// covers the tile's rows from its first row; the caller keeps every offset
// below 2^32 (K < 2^24).
template <int L, int NT>
__device__ __forceinline__ void load_buf(u32x4 (&r)[L], __amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                         uint32_t kb, uint32_t step) {
#pragma unroll
    for (int i = 0; i < L; ++i)
        r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, kb + i * step, 0));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, uint32_t bytes) {
    // gfx9-family raw buffer: stride 0, range `bytes`, default data format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
}

// Edge tiles: rows at or past `limit` are clamped to the last valid row
// (their products only reach outputs that are never stored).
template <int L, int NT>
__device__ __forceinline__ void load_clamped(u32x4 (&r)[L], const uint8_t* __restrict__ src, int row0,
                                             int limit, int K, int kb, int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
        int gr = row0 + (tid >> 3) + (NT / 8) * i;
        gr = gr < limit ? gr : limit - 1;
        r[i] = *reinterpret_cast<const u32x4*>(src + (size_t)gr * K + kb + 16 * (tid & 7));
    }
}

// All MFMAs of one 128-byte K-step for one wave: for each 64-byte half, the
// wave's TN weight fragments stay in registers while its TM activation
// fragments are read one at a time.
template <int BN, int WTN, int WTM, int TN, int TM>
__device__ __forceinline__ void mma_stage(v16f (&acc)[TN][TM], const uint8_t* stage, int wn, int wm,
                                          int lane) {
    const uint8_t* sw = stage;
    const uint8_t* sa = stage + BN * kBK;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int c0 = kk * 4 + (lane >> 5) * 2;
        v8i af[TN];
#pragma unroll
        for (int i = 0; i < TN; ++i) af[i] = frag(sw, wn * WTN + i * 32 + (lane & 31), c0);
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const v8i bf = frag(sa, wm * WTM + j * 32 + (lane & 31), c0);
#pragma unroll
            for (int i = 0; i < TN; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf, acc[i][j], 0, 0,
                                                                            0, 0, 0, 0);
        }
    }
}

// Per-lane LDS offsets of the persistent kernel, computed once.  The swizzle
// only depends on row bits 0..4, so every row the lane touches (its own row
// plus multiples of 32) shares it and all addresses differ by immediates.
struct PipeOffsets {
    uint32_t st;         // stage store: row tid>>3, chunk tid&7
    uint32_t fa[2][2];   // weight fragment, [kk][lo/hi chunk]
    uint32_t fb[2][2];   // activation fragment (includes the 256*128 operand base)
};

__device__ __forceinline__ PipeOffsets pipe_offsets(int tid, int wn, int wm, int lane) {
    PipeOffsets o;
    const int r = tid >> 3;
    o.st = (uint32_t)(r * kBK + (((tid & 7) ^ swz(r)) << 4));
    const int lr = lane & 31, sl = swz(lr);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int chunk = ((kk * 4 + (lane >> 5) * 2 + h) ^ sl) << 4;
            o.fa[kk][h] = (uint32_t)((wn * 128 + lr) * kBK + chunk);
            o.fb[kk][h] = (uint32_t)(256 * kBK + (wm * 128 + lr) * kBK + chunk);
        }
    return o;
}

__device__ __forceinline__ v8i frag_at(const uint8_t* base, uint32_t lo, uint32_t hi) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(base + lo);
    const u32x4 b = *reinterpret_cast<const u32x4*>(base + hi);
    return __builtin_bit_cast(v8i, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One 128-byte K-step of the persistent kernel for one wave (256x256 tile,
// 2x2 waves of 128x128: 4x4 MFMA tiles of 32x32, two 64-byte K halves).
//   cur  LDS slot holding this step's operands (weight rows, then activation
//        rows, 128 bytes each);
//   nxt  the other slot, which receives the next step's operands;
//   x    16 staged 16-byte chunks per thread holding the next step's data
//        (chunks 0..7 weight rows tid/8 + 32c, 8..15 activation rows); each
//        is written to `nxt` and then refilled from global memory with the
//        K-step three ahead of this one (byte offset kb; rsrc wrs / ars).
// The step is eight MFMA groups (one activation fragment against the four
// weight fragments of one K half).  A sched_barrier closes every group, so
// the program order is exactly: fragment reads for the next group, 4 MFMAs,
// 2 chunk writes, 2 chunk loads.  A chunk load therefore has two full steps
// to land before the same group of the step after next writes it to LDS.
// The caller places a workgroup barrier after each step.
__device__ __forceinline__ void kstep(v16f (&acc)[4][4], const uint8_t* cur, uint8_t* nxt, u32x4 (&x)[16],
                                      __amdgpu_buffer_rsrc_t wrs, __amdgpu_buffer_rsrc_t ars, uint32_t voff,
                                      uint32_t kb, uint32_t step, const PipeOffsets& o) {
    constexpr int kRow32 = 32 * kBK;  // 32 rows
    v8i a[2][4];
    v8i b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[0][i] = frag_at(cur + i * kRow32, o.fa[0][0], o.fa[0][1]);
    b[0] = frag_at(cur, o.fb[0][0], o.fb[0][1]);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const int kk = g >> 2, j = g & 3;
        if (g < 7) {
            const int gn = g + 1;
            b[gn & 1] = frag_at(cur + (gn & 3) * kRow32, o.fb[gn >> 2][0], o.fb[gn >> 2][1]);
        }
        if (g == 1 || g == 2) {  // second K half's weight fragments, two per group
#pragma unroll
            for (int i = 2 * (g - 1); i < 2 * g; ++i) a[1][i] = frag_at(cur + i * kRow32, o.fa[1][0], o.fa[1][1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[kk][i], b[g & 1], acc[i][j], 0, 0, 0,
                                                                        0, 0, 0);
#pragma unroll
        for (int c = 2 * g; c < 2 * g + 2; ++c) {
            *reinterpret_cast<u32x4*>(nxt + (c >> 3) * 256 * kBK + (c & 7) * kRow32 + o.st) = x[c];
            x[c] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(c < 8 ? wrs : ars, voff, kb + (c & 7) * step, 0));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// Interior 256x256 tiles.
//
// When padded M and N are multiples of 256 the output splits into T whole
// tiles.  G = one workgroup per CU; the first R*G tiles (R = floor(T/G) full
// rounds, chosen as whole n-columns of tiles) run one tile per workgroup.
// The rem = T - R*G tiles left over would leave most CUs idle for a whole
// tile time, so each of them is split along K into s chunks (s*rem <= G;
// s <= 2: each extra chunk adds a 256 KB partial sum to write and read back,
// which costs more than the finer balance gains) that run in parallel, as
// workgroups after the whole tiles in the same
// launch; the chunks store partial sums in a workspace, and the last chunk
// of a tile to finish adds the s partial sums in chunk order (so the result
// does not depend on the arrival order) and writes the output.  No
// workgroup waits for another.
//
// The K loop (tile_mainloop): two LDS slots, the global loads three K-steps
// ahead of the MFMAs in two register sets.
// ---------------------------------------------------------------------------

// Origin of tile t in the grouped order of a tiles_m x tiles_n region
// (groups of gm m-tiles, m fastest inside a group).
__device__ __forceinline__ void grouped_origin(int t, int tiles_m, int tiles_n, int gm_full, int& n0,
                                               int& m0) {
    const int per_group = gm_full * tiles_n;
    const int gidx = t / per_group;
    const int first_m = gidx * gm_full;
    const int gm = (tiles_m - first_m) < gm_full ? (tiles_m - first_m) : gm_full;
    const int tin = t - gidx * per_group;
    n0 = (tin / gm) * 256;
    m0 = (first_m + tin % gm) * 256;
}

// acc (or acc*scale) over the K-steps [k0, k0+KS) of the tile whose weight
// rows start at `wrs` and activation rows at `ars` (KS even, >= 4).
//
// K-step t computes from LDS slot t%2 while register set (t%2 ? xq : xp)
// moves the data of step t+1 into the other slot and is refilled with step
// t+3; so each load has two steps of MFMA work to land.
__device__ __forceinline__ void tile_mainloop(v16f (&acc)[4][4], uint8_t (&smem)[2][512 * kBK],
                                              __amdgpu_buffer_rsrc_t wrs, __amdgpu_buffer_rsrc_t ars,
                                              uint32_t voff, uint32_t step, int k0, int KS,
                                              const PipeOffsets& po) {
    const __amdgpu_buffer_rsrc_t zr = tile_rsrc(nullptr, 0u);  // range 0: loads return 0, no traffic
    const uint32_t kb0 = (uint32_t)k0 * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};
    u32x4 xp[16], xq[16];
    // K-step 0 -> slot 0 (through xq), K-step 1 -> xp, K-step 2 -> xq
#pragma unroll
    for (int c = 0; c < 16; ++c)
        xq[c] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(c < 8 ? wrs : ars, voff, kb0 + (c & 7) * step, 0));
#pragma unroll
    for (int c = 0; c < 16; ++c)
        xp[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c < 8 ? wrs : ars, voff,
                                                                                kb0 + kBK + (c & 7) * step, 0));
#pragma unroll
    for (int c = 0; c < 16; ++c)
        *reinterpret_cast<u32x4*>(smem[0] + (c >> 3) * 256 * kBK + (c & 7) * 32 * kBK + po.st) = xq[c];
#pragma unroll
    for (int c = 0; c < 16; ++c)
        xq[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              c < 8 ? wrs : ars, voff, kb0 + 2 * kBK + (c & 7) * step, 0));
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    for (int kt = 0; kt < KS; kt += 2) {
        const bool in3 = kt + 3 < KS, in4 = kt + 4 < KS;
        kstep(acc, smem[0], smem[1], xp, in3 ? wrs : zr, in3 ? ars : zr, voff, kb0 + (uint32_t)(kt + 3) * kBK, step,
              po);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        kstep(acc, smem[1], smem[0], xq, in4 ? wrs : zr, in4 ? ars : zr, voff, kb0 + (uint32_t)(kt + 4) * kBK, step,
              po);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    }
}

// acc * mul -> a 256x256 fp32 tile at byte offset 4*(row*stride + nb + col)
// of `rs` (float4 runs of the output column).  For the output, `rs` covers
// the tile's valid rows only, so the stores of rows m >= M fall outside the
// buffer range and are dropped by the hardware (no branches).
__device__ __forceinline__ void store_acc(const v16f (&acc)[4][4], __amdgpu_buffer_rsrc_t rs, uint32_t stride,
                                          uint32_t nb, int wn, int wm, int lane, float mul) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t row = (uint32_t)(wm * 128 + j * 32 + (lane & 31));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t col = nb + (uint32_t)(wn * 128 + i * 32 + 8 * q + 4 * (lane >> 5));
                const float4 v = make_float4(acc[i][j][4 * q] * mul, acc[i][j][4 * q + 1] * mul,
                                             acc[i][j][4 * q + 2] * mul, acc[i][j][4 * q + 3] * mul);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (row * stride + col) * 4u, 0,
                                                       0);
            }
        }
    }
}

// Rows [m0, min(m0+256, M)) of Y; the planner keeps 256*N*4 below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_out_rsrc(float* Y, int M, int N, int m0) {
    const int rows = (M - m0) < 256 ? (M - m0) : 256;
    return __builtin_amdgcn_make_buffer_rsrc(Y + (size_t)m0 * N, (short)0, rows * N * 4, 0x00020000);
}

// Work of the interior-tile kernel.  The grid is nwhole whole-tile
// workgroups followed by the K chunks of the split tiles.
//   Whole tiles: the first nd n-columns of tiles (all m), in the grouped
//   order (groups of group_m m-tiles).  The dispatcher sends workgroup w to
//   XCD w % 8, so XCD x is given the contiguous range [x*T/8, (x+1)*T/8) of
//   that order: the workgroups that run together on one XCD share weight
//   and activation rows through its L2.
//   Split tiles: n-columns [nd, tiles_n), rem tiles in a grouped order with
//   groups of tail_gm m-tiles.  XCD x owns the tiles [x*per_xcd,
//   (x+1)*per_xcd) and its workgroups take them chunk by chunk, so the s
//   chunks of a tile run on one XCD, whose L2 is coherent for its CUs.
//   Chunk c covers the 256-byte K pairs [c*pairs/s, (c+1)*pairs/s).
struct InteriorPlan {
    int tiles_m, nd, nwhole, group_m;
    int rem, tail_gm, per_xcd, s, pairs;
};

// Split-tile epilogue, after the chunk has stored its partial sum (a
// 256x256 fp32 tile, row stride 256) in its slot: wait until the stores
// have reached the XCD's L2 and count in.  The last chunk to arrive resets
// the counter, adds the s partial sums in chunk order, scales, and writes
// the output: float4 f of the tile (row f/64, columns 4*(f%64)..+3), 64
// per thread, NB at a time (NB*S loads in flight per thread).
template <int S, int NB>
__device__ __forceinline__ void split_finish(const float* __restrict__ parts, unsigned* arr, unsigned& arrival,
                                             __amdgpu_buffer_rsrc_t yrs, int N, int n0, int tid, float scale) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) arrival = __hip_atomic_fetch_add(arr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrival != (unsigned)(S - 1)) return;
    if (tid == 0) __hip_atomic_store(arr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next call
    const __amdgpu_buffer_rsrc_t prs =
        tile_rsrc(reinterpret_cast<const uint8_t*>(parts), (uint32_t)S * 256u * 256u * 4u);
    for (int f0 = 0; f0 < 64; f0 += NB) {
        u32x4 v[S][NB];
#pragma unroll
        for (int c = 0; c < S; ++c)
#pragma unroll
            for (int u = 0; u < NB; ++u)  // sc0: not from this CU's L1
                v[c][u] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               prs, ((uint32_t)c * 65536u + (uint32_t)((f0 + u) * 256 + tid) * 4u) * 4u, 0, 1));
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const uint32_t f = (uint32_t)((f0 + u) * 256 + tid);
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float sum = __uint_as_float(v[0][u][e]);
#pragma unroll
                for (int c = 1; c < S; ++c) sum += __uint_as_float(v[c][u][e]);
                r[e] = sum * scale;
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, make_float4(r[0], r[1], r[2], r[3])), yrs,
                                                   ((f >> 6) * (uint32_t)N + (uint32_t)n0 + 4u * (f & 63u)) * 4u, 0, 0);
        }
    }
}

__global__ __launch_bounds__(256) void fp8_gemm_interior_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Wt, float* __restrict__ Y, int M, int N, int K,
    const float* __restrict__ act_scale, float w_scale, InteriorPlan P, float* __restrict__ part,
    unsigned* __restrict__ cnt) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2][512 * kBK];
    __shared__ unsigned arrival;

    const int bid = blockIdx.x;
    int n0, m0, k0 = 0, KS = K / kBK, tl = -1, chunk = 0;
    if (bid < P.nwhole) {
        const int T = P.nwhole;
        const int tall = T / kXcds, rem = T % kXcds;
        const int x = bid % kXcds, loc = bid / kXcds;
        grouped_origin(x * tall + (x < rem ? x : rem) + loc, P.tiles_m, P.nd, P.group_m, n0, m0);
    } else {
        const int g = bid - P.nwhole;  // nwhole is a multiple of 8: same XCD
        const int x = g % kXcds, j = g / kXcds;
        const int base = x * P.per_xcd;
        int count = P.rem - base;
        count = count < P.per_xcd ? count : P.per_xcd;
        if (count <= 0 || j >= count * P.s) return;
        tl = base + j / P.s;
        chunk = j % P.s;
        grouped_origin(tl, P.tiles_m, (N >> 8) - P.nd, P.tail_gm, n0, m0);
        n0 += P.nd * 256;
        const int p0 = chunk * P.pairs / P.s, p1 = (chunk + 1) * P.pairs / P.s;
        k0 = 2 * p0;
        KS = 2 * (p1 - p0);
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wn = wid & 1, wm = wid >> 1;
    const uint32_t voff = (uint32_t)(tid >> 3) * (uint32_t)K + 16u * (uint32_t)(tid & 7);
    const PipeOffsets po = pipe_offsets(tid, wn, wm, lane);

    v16f acc[4][4];
    tile_mainloop(acc, smem, tile_rsrc(Wt + (size_t)n0 * K, 256u * (uint32_t)K),
                  tile_rsrc(A + (size_t)m0 * K, 256u * (uint32_t)K), voff, 32u * (uint32_t)K, k0, KS, po);
    const __amdgpu_buffer_rsrc_t yrs = tile_out_rsrc(Y, M, N, m0);
    const float scale = act_scale[1] * w_scale;
    // One store for both kinds of work: a whole tile writes acc*scale to Y;
    // a K chunk writes acc (times 1, exact) to its partial slot.
    float* parts = tl < 0 ? nullptr : part + (size_t)tl * P.s * (256 * 256);
    const __amdgpu_buffer_rsrc_t srs =
        tl < 0 ? yrs : tile_rsrc(reinterpret_cast<const uint8_t*>(parts + (size_t)chunk * (256 * 256)), 256u * 256u * 4u);
    store_acc(acc, srs, tl < 0 ? (uint32_t)N : 256u, tl < 0 ? (uint32_t)n0 : 0u, wn, wm, lane, tl < 0 ? scale : 1.0f);
    if (tl < 0) return;
    unsigned* arr = cnt + tl;  // arrival counters [0, rem); partial slots follow
    switch (P.s) {
        case 2: split_finish<2, 16>(parts, arr, arrival, yrs, N, n0, tid, scale); break;
        case 3: split_finish<3, 16>(parts, arr, arrival, yrs, N, n0, tid, scale); break;
        default: split_finish<4, 8>(parts, arr, arrival, yrs, N, n0, tid, scale); break;
    }
}

template <int BN, int BM, int WN, int WM>
__global__ __launch_bounds__(64 * WN * WM) void fp8_gemm_deep_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Wt, float* __restrict__ Y, int M,
    int Mp, int N, int K, const float* __restrict__ act_scale, float w_scale, int tiles_m,
    int tiles_n, int group_m) {
    constexpr int NT = 64 * WN * WM;
    constexpr int WTN = BN / WN, WTM = BM / WM;
    constexpr int TN = WTN / 32, TM = WTM / 32;
    constexpr int LW = BN * 8 / NT, LA = BM * 8 / NT;
    static_assert(TN >= 1 && TM >= 1, "wave tile must hold at least one 32x32 MFMA tile");
    static_assert((BN * 8) % NT == 0 && (BM * 8) % NT == 0, "stage load must split evenly");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BN + BM) * kBK];

    const int T = tiles_m * tiles_n;
    const int w = blockIdx.x;
    const int tall = T / kXcds, rem = T % kXcds;
    const int x = w % kXcds, loc = w / kXcds;
    const int t = x * tall + (x < rem ? x : rem) + loc;
    const int per_group = group_m * tiles_n;
    const int gidx = t / per_group;
    const int first_m = gidx * group_m;
    const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int tin = t - gidx * per_group;
    const int n0 = (tin / gm) * BN;
    const int m0 = (first_m + tin % gm) * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wn = wid % WN, wm = wid / WN;

    v16f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = (v16f){};

    // Two-deep global prefetch: the loads for K-step s+2 are issued at step s
    // into the register set that step s-1 already wrote to LDS, so each load
    // has two steps of MFMA work to land.  Two LDS stages.  K/128 is even (K is
    // a multiple of 256), so the loop is unrolled by two and the register sets
    // are static.
    const int KT = K / kBK;
    const bool edge = (n0 + BN > N) || (m0 + BM > Mp);
    const __amdgpu_buffer_rsrc_t wrs = tile_rsrc(Wt + (size_t)n0 * K, (uint32_t)BN * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t ars = tile_rsrc(A + (size_t)m0 * K, (uint32_t)BM * (uint32_t)K);
    const uint32_t voff = (uint32_t)(tid >> 3) * (uint32_t)K + 16u * (uint32_t)(tid & 7);
    const uint32_t step = (uint32_t)(NT / 8) * (uint32_t)K;
    u32x4 rw0[LW], ra0[LA], rw1[LW], ra1[LA];
#define RZ_STAGE_LOAD(RW, RA, KB)                                        \
    do {                                                                 \
        if (edge) {                                                      \
            load_clamped<LW, NT>(RW, Wt, n0, N, K, (KB), tid);           \
            load_clamped<LA, NT>(RA, A, m0, Mp, K, (KB), tid);           \
        } else {                                                         \
            load_buf<LW, NT>(RW, wrs, voff, (KB), step);                 \
            load_buf<LA, NT>(RA, ars, voff, (KB), step);                 \
        }                                                                \
    } while (0)
    RZ_STAGE_LOAD(rw0, ra0, 0);
    RZ_STAGE_LOAD(rw1, ra1, kBK);
    store_rows<LW, NT>(smem[0], rw0, tid);
    store_rows<LA, NT>(smem[0] + BN * kBK, ra0, tid);
    __syncthreads();
    for (int kt = 0; kt < KT; kt += 2) {
        if (kt + 2 < KT) RZ_STAGE_LOAD(rw0, ra0, (kt + 2) * kBK);
        mma_stage<BN, WTN, WTM, TN, TM>(acc, smem[0], wn, wm, lane);
        store_rows<LW, NT>(smem[1], rw1, tid);
        store_rows<LA, NT>(smem[1] + BN * kBK, ra1, tid);
        __syncthreads();
        if (kt + 3 < KT) RZ_STAGE_LOAD(rw1, ra1, (kt + 3) * kBK);
        mma_stage<BN, WTN, WTM, TN, TM>(acc, smem[1], wn, wm, lane);
        if (kt + 2 < KT) {
            store_rows<LW, NT>(smem[0], rw0, tid);
            store_rows<LA, NT>(smem[0] + BN * kBK, ra0, tid);
        }
        __syncthreads();
    }
#undef RZ_STAGE_LOAD

    const float s = act_scale[1] * w_scale;
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int m = m0 + wm * WTM + j * 32 + (lane & 31);
            if (m >= M) continue;
            float* yrow = Y + (size_t)m * N;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WTN + i * 32 + 8 * g + 4 * (lane >> 5);
                const float4 v = make_float4(acc[i][j][4 * g] * s, acc[i][j][4 * g + 1] * s,
                                             acc[i][j][4 * g + 2] * s, acc[i][j][4 * g + 3] * s);
                if (vec && n + 3 < N) {
                    *reinterpret_cast<float4*>(yrow + n) = v;
                } else {
                    if (n < N) yrow[n] = v.x;
                    if (n + 1 < N) yrow[n + 1] = v.y;
                    if (n + 2 < N) yrow[n + 2] = v.z;
                    if (n + 3 < N) yrow[n + 3] = v.w;
                }
            }
        }
    }
}

template <int BN, int BM, int WN, int WM>
__global__ __launch_bounds__(64 * WN * WM) void fp8_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Wt, float* __restrict__ Y, int M,
    int Mp, int N, int K, const float* __restrict__ act_scale, float w_scale, int tiles_m,
    int tiles_n, int group_m) {
    constexpr int NT = 64 * WN * WM;
    constexpr int WTN = BN / WN, WTM = BM / WM;
    constexpr int TN = WTN / 32, TM = WTM / 32;
    constexpr int LW = BN * 8 / NT, LA = BM * 8 / NT;
    static_assert(TN >= 1 && TM >= 1, "wave tile must hold at least one 32x32 MFMA tile");
    static_assert((BN * 8) % NT == 0 && (BM * 8) % NT == 0, "stage load must split evenly");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BN + BM) * kBK];

    // ---- tile mapping
    const int T = tiles_m * tiles_n;
    const int w = blockIdx.x;
    const int tall = T / kXcds, rem = T % kXcds;
    const int x = w % kXcds, loc = w / kXcds;
    const int t = x * tall + (x < rem ? x : rem) + loc;
    const int per_group = group_m * tiles_n;
    const int gidx = t / per_group;
    const int first_m = gidx * group_m;
    const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int tin = t - gidx * per_group;
    const int n0 = (tin / gm) * BN;
    const int m0 = (first_m + tin % gm) * BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wn = wid % WN, wm = wid / WN;

    v16f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = (v16f){};

    u32x4 rw[LW], ra[LA];
    const int KT = K / kBK;

    // prologue: stage 0
    load_rows<LW, NT>(rw, Wt, n0, N, K, 0, tid);
    load_rows<LA, NT>(ra, A, m0, Mp, K, 0, tid);
    store_rows<LW, NT>(smem[0], rw, tid);
    store_rows<LA, NT>(smem[0] + BN * kBK, ra, tid);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        if (more) {
            load_rows<LW, NT>(rw, Wt, n0, N, K, (kt + 1) * kBK, tid);
            load_rows<LA, NT>(ra, A, m0, Mp, K, (kt + 1) * kBK, tid);
        }
        const uint8_t* sw = smem[kt & 1];
        const uint8_t* sa = smem[kt & 1] + BN * kBK;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int c0 = kk * 4 + (lane >> 5) * 2;
            v8i af[TN], bf[TM];
#pragma unroll
            for (int i = 0; i < TN; ++i) af[i] = frag(sw, wn * WTN + i * 32 + (lane & 31), c0);
#pragma unroll
            for (int j = 0; j < TM; ++j) bf[j] = frag(sa, wm * WTM + j * 32 + (lane & 31), c0);
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[i], bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        }
        if (more) {
            store_rows<LW, NT>(smem[(kt + 1) & 1], rw, tid);
            store_rows<LA, NT>(smem[(kt + 1) & 1] + BN * kBK, ra, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: y = acc * (s_act * s_w), fp32 row-major
    const float s = act_scale[1] * w_scale;
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int m = m0 + wm * WTM + j * 32 + (lane & 31);
            if (m >= M) continue;
            float* yrow = Y + (size_t)m * N;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WTN + i * 32 + 8 * g + 4 * (lane >> 5);
                const float4 v = make_float4(acc[i][j][4 * g] * s, acc[i][j][4 * g + 1] * s,
                                             acc[i][j][4 * g + 2] * s, acc[i][j][4 * g + 3] * s);
                if (vec && n + 3 < N) {
                    *reinterpret_cast<float4*>(yrow + n) = v;
                } else {
                    if (n < N) yrow[n] = v.x;
                    if (n + 1 < N) yrow[n + 1] = v.y;
                    if (n + 2 < N) yrow[n + 2] = v.z;
                    if (n + 3 < N) yrow[n + 3] = v.w;
                }
            }
        }
    }
}

enum Kind { kTiles = 0, kMedium = 1, kSmall = 2, kLargeEdge = 3 };

struct KindInfo {
    int bn, bm, threads;
};
constexpr KindInfo kKinds[4] = {{256, 256, 256}, {128, 128, 256}, {64, 32, 128}, {256, 256, 256}};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Arrival counters of the split tiles (one uint32 each), padded to 256 bytes;
// the partial sums follow.
size_t split_counter_bytes(int rem) { return ((size_t)rem * sizeof(unsigned) + 255) / 256 * 256; }

}  // namespace

// Kernel choice per shape:
//  * interior 256x256 tiles (tile kernel, plus the split kernel for the
//    last partial round) when N and padded M are multiples of 256,
//    K >= 512, N <= 2^21 and there are at least 64 tiles;
//  * 256x256 edge-capable kernel when tiles cross N or padded M but there are
//    still >= 256 of them;
//  * 128x128 tiles when that gives >= 256 tiles;
//  * 64x32 tiles otherwise (small M, few tiles).
GemmPlan plan_gemm(uint32_t m, uint32_t n, uint32_t k, int cus, bool split_allowed) {
    const int mp = (int)((m + 15u) & ~15u);
    GemmPlan p = {};
    const int t256 = ceil_div(mp, 256) * ceil_div((int)n, 256);
    if (mp % 256 == 0 && n % 256u == 0 && k >= 512u && n <= (1u << 21) && t256 >= 64 && cus % kXcds == 0) {
        p.kind = kTiles;
        p.G = cus;
        const int tiles_m = mp / 256;
        p.R = t256 / cus;
        // the whole-tile rounds must be whole n-columns of tiles
        if ((p.R * cus) % tiles_m != 0) p.R = 0;
        p.rem = t256 - p.R * cus;
        p.s = 1;
        const int pairs = (int)(k / 256u);
        const int per_xcd = ceil_div(p.rem, kXcds);
        if (p.rem > 0 && p.rem <= cus && split_allowed) {
            int s = (cus / kXcds) / per_xcd;
            s = s < 1 ? 1 : (s > 2 ? 2 : s);
            p.s = s > pairs / 2 ? pairs / 2 : s;  // chunks of >= 2 pairs (>= 4 K-steps)
        }
        if (p.s > 1) {
            p.workgroups = p.R * cus;
            p.split_workgroups = kXcds * per_xcd * p.s;
            p.ws_bytes = split_counter_bytes(p.rem) + (size_t)p.rem * p.s * 256 * 256 * sizeof(float);
        } else {  // every tile whole
            p.R = t256 / cus;
            p.rem = 0;
            p.workgroups = t256;
        }
    } else if (t256 >= 256) {
        p.kind = kLargeEdge;
    } else if (mp >= 128 && ceil_div(mp, 128) * ceil_div((int)n, 128) >= 256) {
        p.kind = kMedium;
    } else {
        p.kind = kSmall;
    }
    p.bn = kKinds[p.kind].bn;
    p.bm = kKinds[p.kind].bm;
    p.threads = kKinds[p.kind].threads;
    if (p.kind != kTiles) p.workgroups = ceil_div(mp, p.bm) * ceil_div((int)n, p.bn);
    return p;
}

hipError_t launch_gemm(const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n,
                       uint32_t k, const float* act_scale, float w_scale, float* y, void* ws,
                       size_t ws_bytes, int cus, hipStream_t st) {
    GemmPlan p = plan_gemm(m, n, k, cus, true);
    if (p.kind == kTiles && p.ws_bytes > 0 && (ws == nullptr || ws_bytes < p.ws_bytes))
        p = plan_gemm(m, n, k, cus, false);  // no room for partial sums: whole tiles only
    const int mp = (int)((m + 15u) & ~15u);
    const int tiles_m = ceil_div(mp, p.bm), tiles_n = ceil_div((int)n, p.bn);
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    switch (p.kind) {
        case kTiles: {
            InteriorPlan ip;
            ip.tiles_m = tiles_m;
            ip.nwhole = p.workgroups;  // whole tiles: the first n-columns (all of them without a split)
            ip.nd = p.workgroups / tiles_m;
            ip.group_m = group_m;
            ip.rem = p.s > 1 ? p.rem : 0;
            ip.per_xcd = ceil_div(ip.rem, kXcds);
            // groups of ~sqrt(tiles per XCD) m-tiles: each XCD's block of split tiles is near square
            int tgm = 1;
            while (tgm * 2 <= tiles_m && tgm * tgm * 4 <= ip.per_xcd) tgm *= 2;
            ip.tail_gm = tgm;
            ip.s = p.s;
            ip.pairs = (int)(k / 256u);
            unsigned* cnt = p.s > 1 ? static_cast<unsigned*>(ws) : nullptr;
            float* part = p.s > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + split_counter_bytes(p.rem))
                                  : nullptr;
            const int grid = p.workgroups + (p.s > 1 ? p.split_workgroups : 0);
            fp8_gemm_interior_kernel<<<grid, 256, 0, st>>>(a_fp8, w_fp8, y, (int)m, (int)n, (int)k, act_scale, w_scale,
                                                           ip, part, cnt);
            (void)tiles_n;
            break;
        }
        case kLargeEdge:
            fp8_gemm_deep_kernel<256, 256, 2, 2><<<p.workgroups, p.threads, 0, st>>>(
                a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n, group_m);
            break;
        case kMedium:
            fp8_gemm_deep_kernel<128, 128, 2, 2><<<p.workgroups, p.threads, 0, st>>>(
                a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n, group_m);
            break;
        default:
            fp8_gemm_kernel<64, 32, 2, 1><<<p.workgroups, p.threads, 0, st>>>(
                a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n, group_m);
            break;
    }
    return hipGetLastError();
}

}  // namespace rz
