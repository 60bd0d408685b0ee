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

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;

// One 128-byte K-step of the pipelined kernel for one wave (256x256 tile,
// 2x2 waves of 128x128, so TN = TM = 4).  The step is one basic block:
//   * all 8 weight fragments of the step (both 64-byte halves) and the first
//     activation fragment are read up front; every later activation fragment
//     is read one MFMA group ahead into the other half of a double buffer;
//   * the 16 stage stores of the next K-step (staged one step earlier, into
//     the other LDS slot) and the 16 buffer loads of the K-step after that
//     are spread between the 32 MFMAs;
// so the matrix pipe always has queued work while LDS and memory traffic
// proceed.  The caller puts a barrier after each step.
// Per-lane LDS offsets of the pipelined kernel, computed once.  The swizzle
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

// One 128-byte K-step of the pipelined kernel for one wave (256x256 tile,
// 2x2 waves of 128x128, so TN = TM = 4).  The step is one basic block:
//   * all 8 weight fragments of the step (both 64-byte halves) and the first
//     activation fragment are read up front; every later activation fragment
//     is read one MFMA group ahead into the other half of a double buffer;
//   * the 16 stage stores of the next K-step (staged one step earlier, into
//     the other LDS slot) and the 16 buffer loads of the K-step after that
//     are spread between the 32 MFMAs;
// so the matrix pipe always has queued work while LDS and memory traffic
// proceed.  The caller puts a barrier after each step.
template <int LG>
__device__ __forceinline__ void pipe_step(v16f (&acc)[4][4], const uint8_t* cur, uint8_t* nxt,
                                          const u32x4 (&st)[LG], u32x4 (&ld)[LG],
                                          __amdgpu_buffer_rsrc_t wrs, __amdgpu_buffer_rsrc_t ars,
                                          uint32_t voff, uint32_t kb_next, uint32_t step,
                                          const PipeOffsets& o) {
    constexpr int kRow32 = 32 * kBK;  // 32 rows
    v8i a[2][4];
    v8i b[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[kk][i] = frag_at(cur + i * kRow32, o.fa[kk][0], o.fa[kk][1]);
    b[0] = frag_at(cur, o.fb[0][0], o.fb[0][1]);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const int kk = g >> 2, j = g & 3;
        if (g < 7) {
            const int kn = (g + 1) >> 2, jn = (g + 1) & 3;
            b[(g + 1) & 1] = frag_at(cur + jn * kRow32, o.fb[kn][0], o.fb[kn][1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[kk][i], b[g & 1], acc[i][j], 0,
                                                                        0, 0, 0, 0, 0);
        // two stage stores and two prefetch loads per MFMA group; chunk c < 8
        // is weight row block c, c >= 8 activation row block c-8
#pragma unroll
        for (int c = 2 * g; c < 2 * g + 2; ++c)
            *reinterpret_cast<u32x4*>(nxt + (c / (LG / 2)) * 256 * kBK + (c % (LG / 2)) * kRow32 + o.st) = st[c];
#pragma unroll
        for (int c = 2 * g; c < 2 * g + 2; ++c) {
            const __amdgpu_buffer_rsrc_t rs = c < LG / 2 ? wrs : ars;
            ld[c] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, kb_next + (c % (LG / 2)) * step, 0));
        }
    }
    // interleave: per group, 2 fragment reads, 4 MFMAs with the 2 stores
    // and 2 loads between them (the 10 up-front reads go first)
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 10, 0);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        if (g < 7) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
}

// 256x256 tile, 4 waves, fully software-pipelined K loop (interior tiles
// only: every row of the tile exists in both operands).  Register sets:
// set 0 / set 1 alternate between "being stored to LDS this step" and
// "being loaded for two steps ahead".  Loads past the last K-step re-read
// K-step 0 (their data is stored to the idle slot and never read).
__global__ __launch_bounds__(256) void fp8_gemm_pipe_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Wt, float* __restrict__ Y, int M,
    int Mp, int N, int K, const float* __restrict__ act_scale, float w_scale, int tiles_m,
    int tiles_n, int group_m) {
    constexpr int BN = 256, BM = 256, NT = 256, LG = 16;  // 8 weight + 8 activation chunks
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
    const int wn = wid & 1, wm = wid >> 1;

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

    const __amdgpu_buffer_rsrc_t wrs = tile_rsrc(Wt + (size_t)n0 * K, (uint32_t)BN * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t ars = tile_rsrc(A + (size_t)m0 * K, (uint32_t)BM * (uint32_t)K);
    const uint32_t voff = (uint32_t)(tid >> 3) * (uint32_t)K + 16u * (uint32_t)(tid & 7);
    const uint32_t step = (uint32_t)(NT / 8) * (uint32_t)K;
    const int KT = K / kBK;  // even

    u32x4 s0[LG], s1[LG];
    // prologue: K-step 0 -> slot 0 (through set 0), K-step 1 -> set 1
#pragma unroll
    for (int c = 0; c < LG; ++c)
        s0[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              c < LG / 2 ? wrs : ars, voff, (c % (LG / 2)) * step, 0));
#pragma unroll
    for (int c = 0; c < LG; ++c)
        s1[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              c < LG / 2 ? wrs : ars, voff, kBK + (c % (LG / 2)) * step, 0));
    const PipeOffsets po = pipe_offsets(tid, wn, wm, lane);
#pragma unroll
    for (int c = 0; c < LG; ++c)
        *reinterpret_cast<u32x4*>(smem[0] + (c / (LG / 2)) * BN * kBK + (c % (LG / 2)) * 32 * kBK + po.st) = s0[c];
    __syncthreads();
    for (int kt = 0; kt < KT; kt += 2) {
        // step kt: slot 0 computes, set 1 (K-step kt+1) -> slot 1, set 0 <- K-step kt+2
        const uint32_t kb2 = (kt + 2 < KT) ? (uint32_t)(kt + 2) * kBK : 0u;
        pipe_step<LG>(acc, smem[0], smem[1], s1, s0, wrs, ars, voff, kb2, step, po);
        __syncthreads();
        // step kt+1: slot 1 computes, set 0 (K-step kt+2) -> slot 0, set 1 <- K-step kt+3
        const uint32_t kb3 = (kt + 3 < KT) ? (uint32_t)(kt + 3) * kBK : 0u;
        pipe_step<LG>(acc, smem[1], smem[0], s0, s1, wrs, ars, voff, kb3, step, po);
        __syncthreads();
    }

    const float s = act_scale[1] * w_scale;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + wm * 128 + j * 32 + (lane & 31);
            if (m >= M) continue;
            float* yrow = Y + (size_t)m * N;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * 128 + i * 32 + 8 * g + 4 * (lane >> 5);
                *reinterpret_cast<float4*>(yrow + n) =
                    make_float4(acc[i][j][4 * g] * s, acc[i][j][4 * g + 1] * s, acc[i][j][4 * g + 2] * s,
                                acc[i][j][4 * g + 3] * s);
            }
        }
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

enum Kind { kLarge = 0, kMedium = 1, kSmall = 2 };

struct KindInfo {
    int bn, bm, threads;
};
constexpr KindInfo kKinds[3] = {{256, 256, 256}, {128, 128, 256}, {64, 32, 128}};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace

GemmPlan plan_gemm(uint32_t m, uint32_t n, uint32_t k) {
    (void)k;
    const int mp = (int)((m + 15u) & ~15u);
    int kind = kSmall;
    for (int c = kLarge; c <= kMedium; ++c) {
        const int tiles = ceil_div(mp, kKinds[c].bm) * ceil_div((int)n, kKinds[c].bn);
        if (mp >= kKinds[c].bm && tiles >= 256) {
            kind = c;
            break;
        }
    }
    GemmPlan p;
    p.kind = kind;
    p.bn = kKinds[kind].bn;
    p.bm = kKinds[kind].bm;
    p.threads = kKinds[kind].threads;
    p.workgroups = ceil_div(mp, p.bm) * ceil_div((int)n, p.bn);
    return p;
}

hipError_t launch_gemm(const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n,
                       uint32_t k, const float* act_scale, float w_scale, float* y,
                       hipStream_t st) {
    const GemmPlan p = plan_gemm(m, n, k);
    const int mp = (int)((m + 15u) & ~15u);
    const int tiles_m = ceil_div(mp, p.bm), tiles_n = ceil_div((int)n, p.bn);
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    switch (p.kind) {
        case kLarge:
            if ((n % 256u) == 0 && (mp % 256) == 0)  // every tile interior: pipelined kernel
                fp8_gemm_pipe_kernel<<<p.workgroups, p.threads, 0, st>>>(
                    a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n,
                    group_m);
            else
                fp8_gemm_deep_kernel<256, 256, 2, 2><<<p.workgroups, p.threads, 0, st>>>(
                    a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n,
                    group_m);
            break;
        case kMedium:
            fp8_gemm_deep_kernel<128, 128, 2, 2><<<p.workgroups, p.threads, 0, st>>>(
                a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n,
                group_m);
            break;
        default:
            fp8_gemm_kernel<64, 32, 2, 1><<<p.workgroups, p.threads, 0, st>>>(
                a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n,
                group_m);
            break;
    }
    return hipGetLastError();
}

}  // namespace rz
