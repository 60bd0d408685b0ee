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
// 32*(l/32), so no transpose is needed.  In the interior kernel the
// activation is the MFMA "A" side (result rows = m) and the weight the "B"
// side (result columns = n): lane l then holds output column n = l%32 of
// its block, so a store instruction writes two full 128-byte output row
// segments (lanes 0-31 one row, 32-63 another).  With the roles the other
// way round each lane holds 4 consecutive n and an instruction covers 32
// rows x 32 bytes, which measured 2-7 % slower per launch on the large
// shapes (same results: the products and their order are the same).
//
// This file: the 256x256 interior-tile kernel (the large prefill GEMMs),
// the plan that picks a kernel per shape, and the launcher.  Kernels for
// tiles that cross N or padded M, small M and few tiles are in
// gemm_edge.hip.
//
// Workgroup -> tile mapping is XCD-aware: the dispatcher sends workgroup w
// to XCD w % 8, so w is first remapped to a contiguous range of tiles per
// XCD; inside it tiles go m-fastest within groups of `group_m` m-tiles, so
// the workgroups that run together on one XCD share weight rows and
// activation rows through that XCD's L2.
#include "gemm_common.h"
#include "rz_gemm.h"

namespace rz {
namespace {
using namespace gemm;

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

// Per-lane LDS offsets of the K loop, computed once.  The swizzle
// only depends on row bits 0..4, so every row the lane touches (its own row
// plus multiples of 32) shares it and all addresses differ by immediates.
struct PipeOffsets {
    uint32_t st;         // stage store: row tid>>3, chunk tid&7
    uint32_t fa[2][2];   // weight fragment, [kk][lo/hi chunk]
    uint32_t fb[2][2];   // activation fragment (includes the 256*128 operand base)
};

template <int TM>
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
            o.fb[kk][h] = (uint32_t)(256 * kBK + (wm * 32 * TM + lr) * kBK + chunk);
        }
    return o;
}

__device__ __forceinline__ v8i frag_at(const uint8_t* base, uint32_t lo, uint32_t hi) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(base + lo);
    const u32x4 b = *reinterpret_cast<const u32x4*>(base + hi);
    return __builtin_bit_cast(v8i, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One 128-byte K-step for one wave of a 256 x (64*TM) tile: 2x2 waves of
// 128 x 32*TM, i.e. 4 x TM MFMA tiles of 32x32, two 64-byte K halves
// (TM = 4: whole 256x256 tile; TM = 2: half tile of 128 activation rows;
// TM = 1: quarter tile of 64).
//   cur  LDS slot holding this step's operands (256 weight rows, then the
//        activation rows, 128 bytes each);
//   nxt  the other slot, which receives the next step's operands;
//   x    8 + 2*TM staged 16-byte chunks per thread holding the next step's
//        data (chunks 0..7 weight rows tid/8 + 32c, then activation rows);
//        each is written to `nxt` and then refilled from global memory with
//        the K-step three ahead of this one (byte offset kb; rsrc wrs / ars).
// The step is 2*TM MFMA groups (one activation fragment against the four
// weight fragments of one K half).  A sched_barrier closes every group, so
// the program order is exactly: fragment reads for the next group, 4 MFMAs
// with the group's chunk writes and loads between them (2 of each for
// TM = 4, 3 for TM = 2).  A chunk load therefore has two full steps to land
// before the same group of the step after next writes it to LDS.  (A
// quarter tile has two groups of 4 MFMAs, each with 5 chunk writes and
// loads; its first group also reads all of the second K half's weight
// fragments.)  The caller places a workgroup barrier after each step.
template <int TM, bool F16>
__device__ __forceinline__ void kstep(v16f (&acc)[4][TM], const uint8_t* cur, uint8_t* nxt,
                                      u32x4 (&x)[8 + 2 * TM], __amdgpu_buffer_rsrc_t wrs,
                                      __amdgpu_buffer_rsrc_t ars, uint32_t voff, uint32_t kb, uint32_t step,
                                      const PipeOffsets& o) {
    static_assert(TM == 4 || TM == 2 || TM == 1, "whole, half or quarter tile");
    constexpr int kRow32 = 32 * kBK;  // 32 rows
    constexpr int kGroups = 2 * TM;
    constexpr int kPer = (8 + 2 * TM) / kGroups;  // chunks per group
    constexpr int kA1 = TM == 4 ? 1 : 0;          // groups kA1, kA1+1 read the second K half's weights
    constexpr int kMf = F16 ? 2 : 1;              // MFMA instructions per mma32
    v8i a[2][4];
    v8i b[2];
    // b first: LDS reads complete in order, so MFMA i of group 0 waits only
    // for b[0] and a[0][0..i]
    b[0] = frag_at(cur, o.fb[0][0], o.fb[0][1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[0][i] = frag_at(cur + i * kRow32, o.fa[0][0], o.fa[0][1]);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        const int kk = g / TM, j = g % TM;
        if (g < kGroups - 1) {
            const int gn = g + 1;
            b[gn & 1] = frag_at(cur + (gn % TM) * kRow32, o.fb[gn / TM][0], o.fb[gn / TM][1]);
        }
        if constexpr (TM == 1) {  // one group per K half: all four now
            if (g == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) a[1][i] = frag_at(cur + i * kRow32, o.fa[1][0], o.fa[1][1]);
            }
        } else if (g == kA1 || g == kA1 + 1) {  // two weight fragments per group
#pragma unroll
            for (int i = 2 * (g - kA1); i < 2 * (g - kA1) + 2; ++i)
                a[1][i] = frag_at(cur + i * kRow32, o.fa[1][0], o.fa[1][1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[i][j] = mma32<F16>(b[g & 1], a[kk][i], acc[i][j]);
#pragma unroll
        for (int c = kPer * g; c < kPer * g + kPer; ++c) {
            *reinterpret_cast<u32x4*>(nxt + (c >> 3) * 256 * kBK + (c & 7) * kRow32 + o.st) = x[c];
            x[c] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(c < 8 ? wrs : ars, voff, kb + (c & 7) * step, 0));
        }
        // order inside the group: the fragment reads (group 0 also holds the
        // 10 reads before the loop), then each chunk write and each load in
        // the shadow of an MFMA
        if constexpr (TM == 4) {
            if (g == 0)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 12, 0);
            else if (g == 1 || g == 2)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
            else if (g < 7)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMf, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMf, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMf, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMf, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
        } else if constexpr (TM == 1) {
            if (g == 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 20, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMf, 0);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
            }
#pragma unroll
            for (int mm = 0; mm < 3; ++mm) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMf, 0);
                if (mm < 2) {
                    __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
        } else {
            if (g == 0)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 16, 0);
            else if (g == 1)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
            else if (g == 2)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMf, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMf, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// Interior 256x256 tiles: a persistent kernel.
//
// The output splits into T = tiles_m * tiles_n tiles of 256 x 256
// (tiles_m = ceil(padded M / 256), tiles_n = ceil(N / 256); see the kernel
// for the last tile when padded M or N is not a multiple of 256).  The
// 128 KB of LDS leave room for one workgroup per CU, so the grid is one
// workgroup per CU, W per XCD, and each workgroup runs a list of tiles.
// A tile runs the whole K range and stores its own output: no partial sums,
// no workspace, no workgroup waits for another.
//
// The K loop (tile_mainloop): two LDS slots, the global loads three K-steps
// ahead of the MFMAs in two register sets.
// ---------------------------------------------------------------------------


// acc over the K-steps [0, KS) of the 256 x 64*TM tile whose weight rows
// start at `wrs` and activation rows at `ars` (KS even, >= 4).
//
// K-step t computes from LDS slot t%2 while register set (t%2 ? xq : xp)
// moves the data of step t+1 into the other slot and is refilled with step
// t+3; so each load has two steps of MFMA work to land.
template <int TM, bool F16>
__device__ __forceinline__ void tile_mainloop(v16f (&acc)[4][TM], uint8_t (&smem)[2][512 * kBK],
                                              __amdgpu_buffer_rsrc_t wrs, __amdgpu_buffer_rsrc_t ars,
                                              uint32_t voff, uint32_t step, int KS, const PipeOffsets& po) {
    constexpr int kC = 8 + 2 * TM;  // staged chunks per thread
    const __amdgpu_buffer_rsrc_t zr = tile_rsrc(nullptr, 0u);  // range 0: loads return 0, no traffic
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = (v16f){};
    u32x4 xp[kC], xq[kC];
    // K-step 0 -> slot 0 (through xq), K-step 1 -> xp, K-step 2 -> xq
#pragma unroll
    for (int c = 0; c < kC; ++c)
        xq[c] = __builtin_bit_cast(u32x4,
                                   __builtin_amdgcn_raw_buffer_load_b128(c < 8 ? wrs : ars, voff, (c & 7) * step, 0));
#pragma unroll
    for (int c = 0; c < kC; ++c)
        xp[c] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(c < 8 ? wrs : ars, voff, kBK + (c & 7) * step, 0));
#pragma unroll
    for (int c = 0; c < kC; ++c)
        *reinterpret_cast<u32x4*>(smem[0] + (c >> 3) * 256 * kBK + (c & 7) * 32 * kBK + po.st) = xq[c];
#pragma unroll
    for (int c = 0; c < kC; ++c)
        xq[c] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(c < 8 ? wrs : ars, voff, 2 * kBK + (c & 7) * step, 0));
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    for (int kt = 0; kt < KS; kt += 2) {
        const bool in3 = kt + 3 < KS, in4 = kt + 4 < KS;
        kstep<TM, F16>(acc, smem[0], smem[1], xp, in3 ? wrs : zr, in3 ? ars : zr, voff, (uint32_t)(kt + 3) * kBK,
                       step, po);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        kstep<TM, F16>(acc, smem[1], smem[0], xq, in4 ? wrs : zr, in4 ? ars : zr, voff, (uint32_t)(kt + 4) * kBK,
                       step, po);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    }
}

// acc * scale -> the 256 x 64*TM output tile at (n0, m0).  acc[i][j][e]
// is activation row wm*32*TM + 32j + 8*(e/4) + 4*(lane/32) + e%4 and
// output column n0 + wn*128 + 32i + lane%32 (32x32 MFMA result layout with
// the activation as the A operand), so each dword store covers 128
// consecutive bytes of two output rows.  `rs` covers the valid rows from m0
// only, so the stores of rows m >= M fall outside the buffer range and are
// dropped by the hardware (no branches).  The stores are non-temporal: the
// output (155 MB per FFN GEMM at M=2048) is written once and would
// otherwise fill the MALL with dirty lines that the next kernels' reads
// must first evict (in the FFN step: the down input's quantisation 80 ->
// 72 us, the down GEMM 142 -> 132 us, this launch unchanged).
template <int TM>
__device__ __forceinline__ void store_acc(const v16f (&acc)[4][TM], __amdgpu_buffer_rsrc_t rs, uint32_t N,
                                          uint32_t n0, int wn, int wm, int lane, float scale) {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
        const uint32_t row0 = (uint32_t)(wm * 32 * TM + j * 32 + 4 * (lane >> 5));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t col = n0 + (uint32_t)(wn * 128 + i * 32 + (lane & 31));
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t row = row0 + (uint32_t)(8 * (e >> 2) + (e & 3));
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[i][j][e] * scale), rs,
                                                      (row * N + col) * 4u, 0, kNonTemporal);
            }
        }
    }
}

// Rows [m0, min(m0+256, M)) of Y; the planner keeps 256*N*4 below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_out_rsrc(float* Y, int M, int N, int m0) {
    const int rows = (M - m0) < 256 ? (M - m0) : 256;
    return __builtin_amdgcn_make_buffer_rsrc(Y + (size_t)m0 * N, (short)0, rows * N * 4, 0x00020000);
}

// Work of the interior-tile kernel.  The dispatcher sends workgroup w to
// XCD w % 8; workgroup j = w / 8 of XCD x (j < W) works on a contiguous
// run of the T tiles in the grouped order (groups of group_m m-tiles, m
// fastest inside a group), Tx of them, so the workgroups that run together
// on one XCD share weight and activation rows through its L2:
//   R = Tx / W whole rounds: tile r*W + j of the run in round r;
//   the L = Tx - R*W tiles left over run as half tiles of 128 activation
//   rows when a whole round comes before them or their 2L halves fit one
//   round (else as whole tiles, one each for workgroups j < L).  When the
//   2L halves are more than W but at most 1.5 W, every workgroup takes one
//   half and the halves beyond the first W run as quarter tiles of 64
//   activation rows instead, at most one per workgroup, so that no
//   workgroup runs two halves (a half tile costs ~0.6 of a whole one).
// Half and quarter tiles go out in half_rank order (the odd workgroups
// first), and an odd workgroup runs its quarter tile, or else its first
// half tile, before its whole tiles, an even one after them: the two halves
// of an XCD then reach the end of their whole tiles a quarter or half a tile
// apart.  The two halves hold different activation rows but the same weight
// rows; a quarter tile apart (~7 K-steps, under 3 MB of the XCD's loads)
// the later half finds the weight rows still in the 4 MB L2, half a tile
// apart it reads them again (gate+up at M=2048 in the FFN step: 242 against
// 245 us).  Measured on the 256x256 tiles, the 256 KB
// output store of a tile takes ~7k cycles when 16 CUs of an XCD store
// together and ~16k when all 32 do, whether or not the other XCDs store at
// the same time (the XCD's write path is the limit, not HBM).
// When the padded M (mp, a multiple of 16) is not a multiple of the tile
// height, the last m-tile (half) starts at mp - 256 (mp - 128) instead, and
// when N is not a multiple of 256 the last n-tile starts at N - 256: such a
// tile overlaps the one before it, so every row it loads exists and every
// column it stores is < N, and the outputs both compute get the same
// operands in the same order, so both store the same values there.  Every
// output element is so computed over the whole K in one order, whichever
// workgroup runs it: the results do not depend on the CU count or on which
// GEMMs share a launch.
struct InteriorPlan {
    int tiles_m, tiles_n, group_m, T, W;
};

// XCD-local rank of workgroup j in the hand-out order of half tiles: the
// odd workgroups first, then the even ones.
__device__ __forceinline__ int half_rank(int j, int W) { return (j & 1) ? (j >> 1) : (W >> 1) + (j >> 1); }

// The weight and output of the n-tile starting at column n0 of the launch:
// the launch's N columns are the groups' columns one after the other (every
// group boundary a multiple of 256 when there are several groups, so a tile
// never straddles two).  n0 becomes the column inside the group, N its width.
__device__ __forceinline__ int group_of(const GemmGroups& G, int& n0, int& N) {
    int g = 0;
    while (g + 1 < G.count && n0 >= G.n_end[g]) ++g;
    const int begin = g ? G.n_end[g - 1] : 0;
    n0 -= begin;
    N = G.n_end[g] - begin;
    return g;
}

// F16: fp16 operands (K is then the row length in bytes, twice the
// element count), no scales (act_scale is not read, w_scale is 1).
template <bool F16>
__global__ __launch_bounds__(256) void fp8_gemm_interior_kernel(const uint8_t* __restrict__ A, GemmGroups G,
                                                                int M, int N, int K,
                                                                const float* __restrict__ act_scale,
                                                                InteriorPlan P) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2][512 * kBK];

    const int bid = blockIdx.x;
    const uint32_t step = 32u * (uint32_t)K;
    const float act_dq = F16 ? 1.0f : act_scale[1];
    const int mp = (M + 15) & ~15;  // >= 256 here
    const int x = bid % kXcds, j = bid / kXcds;
    const int tall = P.T / kXcds, trem = P.T % kXcds;
    const int first = x * tall + (x < trem ? x : trem);
    const int Tx = tall + (x < trem ? 1 : 0);
    const int R = Tx / P.W, L = Tx - R * P.W;
    const bool halves = R > 0 || 2 * L <= P.W;
    int H = halves ? 2 * L : 0;  // half tiles of this XCD
    int Q = 0;                   // quarter tiles: halves H.. of the left-over tiles, split
    if (H > P.W && 2 * (H - P.W) <= P.W) {
        Q = 2 * (H - P.W);
        H = P.W;
    }
    const int hr = half_rank(j, P.W);
    // items in order: [quarter hr if j is odd, else half hr if j is odd]
    // [whole rounds] [the left-over whole tile j] [halves hr (unless run
    // early), hr + W, hr + 2W, ...] [quarter hr (unless run early)]
    const bool early_q = (j & 1) && hr < Q;
    const bool early = (j & 1) && hr < H && !early_q;
    int idx = (early || early_q) ? -1 : 0;  // -1: the early quarter or half; 0..R-1: rounds; R: left-over whole tile
    int hnext = early ? hr + P.W : hr;
    bool quarter_left = hr < Q && !early_q;
    for (;;) {
        int part = 4;    // activation rows / 64: 4 whole, 2 half, 1 quarter
        int lt, mo = 0;  // tile of the XCD's run, activation row offset in it
        if (idx < 0 && early_q) {
            part = 1;
            const int h = H + hr / 2;  // the half tile this quarter belongs to
            lt = R * P.W + h / 2;
            mo = 128 * (h & 1) + 64 * (hr & 1);
            idx = 0;
        } else if (idx < 0) {
            part = 2;
            lt = R * P.W + hr / 2;
            mo = 128 * (hr & 1);
            idx = 0;
        } else if (idx < R) {
            lt = idx * P.W + j;
            ++idx;
        } else if (idx == R && !halves && j < L) {
            lt = R * P.W + j;
            ++idx;
        } else if (hnext < H) {
            part = 2;
            lt = R * P.W + hnext / 2;
            mo = 128 * (hnext & 1);
            hnext += P.W;
        } else if (quarter_left) {
            part = 1;
            const int h = H + hr / 2;  // the half tile this quarter belongs to
            lt = R * P.W + h / 2;
            mo = 128 * (h & 1) + 64 * (hr & 1);
            quarter_left = false;
        } else {
            break;
        }
        // the per-lane values are rebuilt from an opaque copy of the thread
        // id for every tile, so that the compiler keeps none of them (nor
        // the addresses made from them) live across the tile loop
        int tid = (int)threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wid = tid >> 6;
        const int wn = wid & 1, wm = wid >> 1;
        const uint32_t voff = (uint32_t)(tid >> 3) * (uint32_t)K + 16u * (uint32_t)(tid & 7);
        int n0, m0;
        grouped_origin_bb<256, 256>(first + lt, P.tiles_m, P.tiles_n, P.group_m, n0, m0);
        n0 = n0 < N - 256 ? n0 : N - 256;
        int Ng;
        const int g = group_of(G, n0, Ng);
        if (part == 4) {
            m0 = m0 < mp - 256 ? m0 : mp - 256;
            const PipeOffsets po = pipe_offsets<4>(tid, wn, wm, lane);
            v16f acc[4][4];
            tile_mainloop<4, F16>(acc, smem, tile_rsrc(G.w[g] + (size_t)n0 * K, 256u * (uint32_t)K),
                                  tile_rsrc(A + (size_t)m0 * K, 256u * (uint32_t)K), voff, step, K / kBK, po);
            store_acc<4>(acc, tile_out_rsrc(G.y[g], M, Ng, m0), (uint32_t)Ng, (uint32_t)n0, wn, wm, lane,
                         act_dq * G.w_scale[g]);
        } else if (part == 2) {
            m0 += mo;
            m0 = m0 < mp - 128 ? m0 : mp - 128;
            const PipeOffsets po = pipe_offsets<2>(tid, wn, wm, lane);
            v16f acc[4][2];
            tile_mainloop<2, F16>(acc, smem, tile_rsrc(G.w[g] + (size_t)n0 * K, 256u * (uint32_t)K),
                                  tile_rsrc(A + (size_t)m0 * K, 128u * (uint32_t)K), voff, step, K / kBK, po);
            store_acc<2>(acc, tile_out_rsrc(G.y[g], M, Ng, m0), (uint32_t)Ng, (uint32_t)n0, wn, wm, lane,
                         act_dq * G.w_scale[g]);
        } else {
            m0 += mo;
            m0 = m0 < mp - 64 ? m0 : mp - 64;
            const PipeOffsets po = pipe_offsets<1>(tid, wn, wm, lane);
            v16f acc[4][1];
            tile_mainloop<1, F16>(acc, smem, tile_rsrc(G.w[g] + (size_t)n0 * K, 256u * (uint32_t)K),
                                  tile_rsrc(A + (size_t)m0 * K, 64u * (uint32_t)K), voff, step, K / kBK, po);
            store_acc<1>(acc, tile_out_rsrc(G.y[g], M, Ng, m0), (uint32_t)Ng, (uint32_t)n0, wn, wm, lane,
                         act_dq * G.w_scale[g]);
        }
    }
}

struct KindInfo {
    int bn, bm, threads;
};
// indexed by GemmKind
constexpr KindInfo kKinds[6] = {{256, 256, 256}, {128, 128, 256}, {64, 32, 128}, {256, 256, 256}, {16, 0, 256}, {4, 0, 256}};

int ceil_div(int a, int b) { return (a + b - 1) / b; }


// K chunks per tile for the edge-capable kinds.  The 128x128 kernel (two
// workgroups per CU) splits until the chunks fill one workgroup per CU, in
// chunks of >= 2 K pairs; the 64x32 kernel, which is memory-bound, until
// there are about two workgroups per CU, in chunks of >= 1 pair.  The
// 256x256 edge kernel only runs with >= 256 tiles and never splits.
int edge_split(int kind, int mp, uint32_t n, uint32_t k) {
    const int pairs = (int)(k / 256u);
    int s = 1;
    if (kind == kGemmMedium) {
        const int T = ceil_div(mp, 128) * ceil_div((int)n, 128);
        s = 256 / T < pairs / 2 ? 256 / T : pairs / 2;
    } else if (kind == kGemmSmall) {
        const int T = ceil_div(mp, 32) * ceil_div((int)n, 64);
        s = 512 / T < pairs ? 512 / T : pairs;
    }
    return s < 1 ? 1 : s;
}

}  // namespace

// Kernel choice per shape:
//  * the GEMV kernel (one weight row per wave, vector ALU) when M <= 3
//    (measured: faster than the skinny kernel up to M = 2, equal at 3; the
//    pages also route M < 4 to their GEMV path);
//  * the skinny kernel (16 weight rows per workgroup, K split over its
//    waves) when padded M <= 64;
//  * the persistent interior kernel (256x256 tiles in rounds, the tiles
//    left over as half tiles; one workgroup per CU) when N and padded M
//    are >= 256, K >= 512, N < 2^21, there are at least 64 tiles and the
//    CUs split evenly over the 8 XCDs, at least 2 on each;
//  * 256x256 edge-capable kernel when padded M < 256 but there are still
//    >= 256 tiles;
//  * 128x128 tiles when M_pad >= 128 and tiles times K chunks give >= 128
//    workgroups;
//  * 64x32 tiles otherwise (small M, few tiles).
// The last two split K (edge_split) when a workspace is given.
GemmPlan plan_gemm(uint32_t m, uint32_t n, uint32_t k, int cus, bool split_allowed) {
    const int mp = (int)((m + 15u) & ~15u);
    GemmPlan p = {};
    p.s = 1;
    const int t256 = ceil_div(mp, 256) * ceil_div((int)n, 256);
    if (mp >= 256 && n >= 256u && k >= 512u && n < (1u << 21) && t256 >= 64 && cus % kXcds == 0 &&
        cus / kXcds >= 2) {
        p.kind = kGemmTiles;
        p.G = cus;
        p.workgroups = cus;  // persistent: one workgroup per CU
    } else if (m <= 3) {
        p.kind = kGemmGemv;
    } else if (mp <= 64) {
        p.kind = kGemmSkinny;
    } else if (t256 >= 256) {
        p.kind = kGemmLargeEdge;
    } else if (mp >= 128 && ceil_div(mp, 128) * ceil_div((int)n, 128) * edge_split(kGemmMedium, mp, n, k) >= 128) {
        p.kind = kGemmMedium;
    } else {
        p.kind = kGemmSmall;
    }
    p.bn = kKinds[p.kind].bn;
    p.bm = (p.kind == kGemmSkinny || p.kind == kGemmGemv) ? mp : kKinds[p.kind].bm;
    p.threads = kKinds[p.kind].threads;
    if (p.kind == kGemmGemv) {
        p.workgroups = ceil_div((int)n, 4);  // one weight row per wave
    } else if (p.kind == kGemmSkinny) {
        p.workgroups = ceil_div((int)n, 16);
    } else if (p.kind != kGemmTiles) {
        const int T = ceil_div(mp, p.bm) * ceil_div((int)n, p.bn);
        p.workgroups = T;
        p.s = split_allowed && T <= kSplitMaxTiles ? edge_split(p.kind, mp, n, k) : 1;
        if (p.s > 1) {  // XCD x runs the chunks of its own tiles (tile_of_workgroup)
            p.rem = T;
            p.workgroups = kXcds * ceil_div(T, kXcds) * p.s;
            p.ws_bytes = kSplitCounterBytes + (size_t)T * p.s * p.bn * p.bm * sizeof(float);
        }
    }
    return p;
}

hipError_t launch_gemm(const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n,
                       uint32_t k, const float* act_scale, float w_scale, float* y, void* ws,
                       size_t ws_bytes, int cus, hipStream_t st) {
    GemmPlan p = plan_gemm(m, n, k, cus, true);
    if (p.ws_bytes > 0 && (ws == nullptr || ws_bytes < p.ws_bytes))
        p = plan_gemm(m, n, k, cus, false);  // no room for partial sums: whole tiles only
    if (p.kind != kGemmTiles) return launch_gemm_edge(p, a_fp8, w_fp8, m, n, k, act_scale, w_scale, y, ws, st);
    GemmGroups G = {};
    G.count = 1;
    G.n_end[0] = (int)n;
    G.w[0] = w_fp8;
    G.y[0] = y;
    G.w_scale[0] = w_scale;
    return launch_interior(p, a_fp8, G, m, n, k, act_scale, st, false);
}

hipError_t launch_fp16_gemm(const uint16_t* a_f16, const uint16_t* w_f16, uint32_t m, uint32_t n, uint32_t k,
                            float* y, int cus, hipStream_t st) {
    const uint32_t kb = 2u * k;  // row length in bytes: the kernels walk K in 128-byte steps
    GemmPlan p = plan_gemm(m, n, kb, cus, false);
    const uint8_t* a = reinterpret_cast<const uint8_t*>(a_f16);
    const uint8_t* w = reinterpret_cast<const uint8_t*>(w_f16);
    if (p.kind != kGemmTiles) {
        // no GEMV or skinny kernel for fp16 operands: small M takes the 64x32 tiles
        if (p.kind == kGemmGemv || p.kind == kGemmSkinny) {
            p.kind = kGemmSmall;
            p.bn = kKinds[kGemmSmall].bn;
            p.bm = kKinds[kGemmSmall].bm;
            p.threads = kKinds[kGemmSmall].threads;
            const int mp = (int)((m + 15u) & ~15u);
            p.workgroups = ceil_div(mp, p.bm) * ceil_div((int)n, p.bn);
            p.s = 1;
        }
        return launch_gemm_edge_fp16(p, a, w, m, n, kb, y, st);
    }
    GemmGroups G = {};
    G.count = 1;
    G.n_end[0] = (int)n;
    G.w[0] = w;
    G.y[0] = y;
    G.w_scale[0] = 1.0f;
    return launch_interior(p, a, G, m, n, kb, nullptr, st, true);
}

hipError_t launch_interior(const GemmPlan& p, const uint8_t* a_fp8, const GemmGroups& G, uint32_t m, uint32_t n,
                           uint32_t k, const float* act_scale, hipStream_t st, bool f16) {
    const int mp = (int)((m + 15u) & ~15u);
    InteriorPlan ip;
    ip.tiles_m = ceil_div(mp, 256);
    ip.tiles_n = ceil_div((int)n, 256);
    ip.group_m = ip.tiles_m < 8 ? ip.tiles_m : 8;
    ip.T = ip.tiles_m * ip.tiles_n;
    ip.W = p.G / kXcds;
    // When an XCD's tiles fit one round, the group height is the one that
    // gives each XCD's run the fewest distinct m- and n-tiles (ties: the
    // taller group), so that less of the activation and weight streams
    // through each XCD's L2: the down GEMM at M=2048 (14 tiles per XCD)
    // takes 4 m-tiles x 4 n-tiles instead of 8 x 2 (FFN step, alternating
    // runs on one box: 128.6 against 131.9 us).  With several rounds the
    // groups stay 8 high.
    const int tx = ceil_div(ip.T, kXcds);
    if (tx <= ip.W) {
        int best = ip.group_m, cost = best + ceil_div(tx, best);
        for (int a = 4; a >= 1; a >>= 1) {
            if (a >= ip.group_m) continue;
            const int c = a + ceil_div(tx, a);
            if (c < cost) { cost = c; best = a; }
        }
        ip.group_m = best;
    }
    if (f16)
        fp8_gemm_interior_kernel<true><<<p.workgroups, 256, 0, st>>>(a_fp8, G, (int)m, (int)n, (int)k, act_scale, ip);
    else
        fp8_gemm_interior_kernel<false><<<p.workgroups, 256, 0, st>>>(a_fp8, G, (int)m, (int)n, (int)k, act_scale, ip);
    return hipGetLastError();
}

}  // namespace rz
