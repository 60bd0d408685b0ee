// FP8 GEMM kernels for the shapes the interior 256x256 kernel does not
// take (same operation as gemm.hip: Y = dec(A) * dec(W)^T scaled by
// act_scale[1] * w_scale, fp32 out; realizar 0.8.4 source page
// cublas_prefill/gemm.rs, cublas_prefill_fp8_gemm):
//   * fp8_gemm_deep_kernel: BN x BM tiles that may cross N or padded M,
//     with a two-deep register prefetch, optionally split along K;
//   * fp8_gemm_kernel: 64x32 tiles with a one-deep prefetch, optionally
//     split along K;
//   * fp8_gemm_skinny_kernel: padded M <= 64, bound by the weight read;
//   * fp8_gemv_kernel: M <= 3, on the vector ALU.
//
// The tiled kernels walk K in steps of 128 bytes with two LDS stages: the
// next step's global loads are issued before the current step's MFMAs and
// written to the other stage afterwards.  LDS rows are 128 bytes; the
// 16-byte chunk c of row r is stored at c ^ swz(r) so that the MFMA operand
// reads (8 or 16 consecutive rows, same chunk) and the stage writes hit
// distinct banks.
#include "gemm_common.h"
#include "rz_gemm.h"

namespace rz {
namespace {
using namespace gemm;

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
template <int BN, int WTN, int WTM, int TN, int TM, bool F16>
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
            for (int i = 0; i < TN; ++i) acc[i][j] = mma32<F16>(bf, af[i], acc[i][j]);
        }
    }
}

// ---------------------------------------------------------------------------
// Edge and small-tile kernels: tiles that may cross N or M_pad, and split-K.
//
// With s = 1 workgroup w computes tile t (XCD-aware, see tile_of_workgroup)
// over all of K.  Shapes with too few tiles to keep the CUs busy (small M,
// narrow N) split K into s chunks of whole 256-byte pairs: XCD x owns a
// contiguous range of tiles and its workgroups take them chunk by chunk, so
// the s chunks of a tile run on one XCD.  Each chunk stores its raw partial
// sum in the tile's slot of the workspace (thread-major float4 blocks: block
// b of thread t at float4 index b*NT + t), counts itself in, and the last to
// arrive adds the s partials in chunk order (so the sum does not depend on
// the arrival order) and writes the output.  No workgroup waits for another.
//
// The hand-over needs no cache-wide maintenance: the partials are stored at
// device scope (the store writes through the XCD's L2), each wave waits
// until its stores are complete at that scope before the arrival count is
// taken, and the last arriver reads the partials at system scope (the loads
// miss in its L1 and L2).  So a chunk that ran on another XCD is seen as
// well as one that ran on the reader's own, whatever the dispatcher's
// placement.  (A release/acquire pair on the counter instead costs an L2
// write-back in every workgroup and an L2 invalidate in the last: measured
// 2.4x slower at M=512, N=512, K=3584.)
// ---------------------------------------------------------------------------
struct SplitK {
    int s;          // K chunks per tile (1: no split)
    int pairs;      // K / 256
    float* part;    // s partial slots per tile
    unsigned* cnt;  // arrival counter per tile
};

// Tile and K chunk of workgroup w among T tiles; false if w has no work.
__device__ __forceinline__ bool tile_of_workgroup(int w, int T, const SplitK& S, int& t, int& chunk) {
    const int tall = T / kXcds, rem = T % kXcds;
    const int x = w % kXcds, j = w / kXcds;
    const int first = x * tall + (x < rem ? x : rem);
    if (S.s <= 1) {
        t = first + j;
        chunk = 0;
        return true;
    }
    const int count = tall + (x < rem ? 1 : 0);
    const int tl = j / S.s;
    chunk = j % S.s;
    t = first + tl;
    return tl < count;
}

// Split-K epilogue for a TN x TM wave tile of NT threads: store this chunk's
// partial, count in; the last chunk returns true with acc = the sum of the s
// partials in chunk order (read 4 chunks per batch).
template <int TN, int TM, int NT>
__device__ __forceinline__ bool split_reduce(v16f (&acc)[TN][TM], const SplitK& S, int t, int chunk,
                                             unsigned& arrival, int tid) {
    constexpr int NB = TN * TM * 4;  // float4 blocks per thread
    constexpr uint32_t kSlot = NB * NT * 16u;  // bytes per slot
    float* slots = S.part + (size_t)t * S.s * (kSlot / 4);
    float4* mine = reinterpret_cast<float4*>(slots + (size_t)chunk * (kSlot / 4));
    const __amdgpu_buffer_rsrc_t mrs = tile_rsrc(reinterpret_cast<const uint8_t*>(mine), kSlot);
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(acc[i][j][4 * g + e]);
                __builtin_amdgcn_raw_buffer_store_b128(v, mrs, (uint32_t)(((i * TM + j) * 4 + g) * NT + tid) * 16u, 0,
                                                       kScopeDevice);
            }
    // every wave waits until its device-scope stores are complete; the
    // barrier orders them before thread 0's count, and the second barrier
    // orders every wave's partial loads after the count is known
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) arrival = __hip_atomic_fetch_add(S.cnt + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrival != (unsigned)(S.s - 1)) return false;
    if (tid == 0) __hip_atomic_store(S.cnt + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
    const __amdgpu_buffer_rsrc_t prs =
        tile_rsrc(reinterpret_cast<const uint8_t*>(slots), (uint32_t)S.s * kSlot);
    const __amdgpu_buffer_rsrc_t zr = tile_rsrc(nullptr, 0u);
    for (int c0 = 0; c0 < S.s; c0 += 4) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)  // chunks past s read as zero (range-0 resource) and are skipped
                v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     c0 + u < S.s ? prs : zr,
                                                     (uint32_t)(c0 + u) * kSlot + (uint32_t)(b * NT + tid) * 16u, 0, kScopeSystem));
            const int i = b / (TM * 4), j = (b / 4) % TM, g = b % 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float sum = c0 == 0 ? __uint_as_float(v[0][e]) : acc[i][j][4 * g + e] + __uint_as_float(v[0][e]);
#pragma unroll
                for (int u = 1; u < 4; ++u)
                    if (c0 + u < S.s) sum += __uint_as_float(v[u][e]);
                acc[i][j][4 * g + e] = sum;
            }
        }
    }
    return true;
}

// F16: fp16 operands (K = row bytes), no scales (act_scale not read).
template <int BN, int BM, int WN, int WM, bool kSplit, bool F16 = false>
__global__ __launch_bounds__(64 * WN * WM) void fp8_gemm_deep_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Wt, float* __restrict__ Y, int M,
    int Mp, int N, int K, const float* __restrict__ act_scale, float w_scale, int tiles_m,
    int tiles_n, int group_m, SplitK S) {
    constexpr int NT = 64 * WN * WM;
    constexpr int WTN = BN / WN, WTM = BM / WM;
    constexpr int TN = WTN / 32, TM = WTM / 32;
    constexpr int LW = BN * 8 / NT, LA = BM * 8 / NT;
    static_assert(TN >= 1 && TM >= 1, "wave tile must hold at least one 32x32 MFMA tile");
    static_assert((BN * 8) % NT == 0 && (BM * 8) % NT == 0, "stage load must split evenly");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BN + BM) * kBK];
    __shared__ unsigned arrival;

    int t, chunk;
    if (!tile_of_workgroup(blockIdx.x, tiles_m * tiles_n, S, t, chunk)) return;
    int n0, m0;
    grouped_origin_bb<BN, BM>(t, tiles_m, tiles_n, group_m, n0, m0);
    const int p0 = chunk * S.pairs / S.s, p1 = (chunk + 1) * S.pairs / S.s;
    const int k0 = 2 * p0, KT = 2 * (p1 - p0);  // K-steps of 128 bytes: [k0, k0 + KT)

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
    RZ_STAGE_LOAD(rw0, ra0, k0 * kBK);
    RZ_STAGE_LOAD(rw1, ra1, (k0 + 1) * kBK);
    store_rows<LW, NT>(smem[0], rw0, tid);
    store_rows<LA, NT>(smem[0] + BN * kBK, ra0, tid);
    __syncthreads();
    for (int kt = 0; kt < KT; kt += 2) {
        if (kt + 2 < KT) RZ_STAGE_LOAD(rw0, ra0, (k0 + kt + 2) * kBK);
        mma_stage<BN, WTN, WTM, TN, TM, F16>(acc, smem[0], wn, wm, lane);
        store_rows<LW, NT>(smem[1], rw1, tid);
        store_rows<LA, NT>(smem[1] + BN * kBK, ra1, tid);
        __syncthreads();
        if (kt + 3 < KT) RZ_STAGE_LOAD(rw1, ra1, (k0 + kt + 3) * kBK);
        mma_stage<BN, WTN, WTM, TN, TM, F16>(acc, smem[1], wn, wm, lane);
        if (kt + 2 < KT) {
            store_rows<LW, NT>(smem[0], rw0, tid);
            store_rows<LA, NT>(smem[0] + BN * kBK, ra0, tid);
        }
        __syncthreads();
    }
#undef RZ_STAGE_LOAD

    if constexpr (kSplit)  // (the 256x256 instance never splits: its registers are full)
        if (S.s > 1 && !split_reduce<TN, TM, NT>(acc, S, t, chunk, arrival, tid)) return;
    store_tile<TN, TM, WTN, WTM>(acc, Y, M, N, m0 + wm * WTM, n0 + wn * WTN, lane,
                                 F16 ? 1.0f : act_scale[1] * w_scale);
}

template <int BN, int BM, int WN, int WM, bool F16 = false>
__global__ __launch_bounds__(64 * WN * WM) void fp8_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Wt, float* __restrict__ Y, int M,
    int Mp, int N, int K, const float* __restrict__ act_scale, float w_scale, int tiles_m,
    int tiles_n, int group_m, SplitK S) {
    constexpr int NT = 64 * WN * WM;
    constexpr int WTN = BN / WN, WTM = BM / WM;
    constexpr int TN = WTN / 32, TM = WTM / 32;
    constexpr int LW = BN * 8 / NT, LA = BM * 8 / NT;
    static_assert(TN >= 1 && TM >= 1, "wave tile must hold at least one 32x32 MFMA tile");
    static_assert((BN * 8) % NT == 0 && (BM * 8) % NT == 0, "stage load must split evenly");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BN + BM) * kBK];
    __shared__ unsigned arrival;

    // ---- tile mapping
    int t, chunk;
    if (!tile_of_workgroup(blockIdx.x, tiles_m * tiles_n, S, t, chunk)) return;
    int n0, m0;
    grouped_origin_bb<BN, BM>(t, tiles_m, tiles_n, group_m, n0, m0);
    const int p0 = chunk * S.pairs / S.s, p1 = (chunk + 1) * S.pairs / S.s;
    const int k0 = 2 * p0;  // first K-step of 128 bytes

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
    const int KT = 2 * (p1 - p0);

    // prologue: stage 0
    load_rows<LW, NT>(rw, Wt, n0, N, K, k0 * kBK, tid);
    load_rows<LA, NT>(ra, A, m0, Mp, K, k0 * kBK, tid);
    store_rows<LW, NT>(smem[0], rw, tid);
    store_rows<LA, NT>(smem[0] + BN * kBK, ra, tid);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        if (more) {
            load_rows<LW, NT>(rw, Wt, n0, N, K, (k0 + kt + 1) * kBK, tid);
            load_rows<LA, NT>(ra, A, m0, Mp, K, (k0 + kt + 1) * kBK, tid);
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
                for (int j = 0; j < TM; ++j) acc[i][j] = mma32<F16>(bf[j], af[i], acc[i][j]);
        }
        if (more) {
            store_rows<LW, NT>(smem[(kt + 1) & 1], rw, tid);
            store_rows<LA, NT>(smem[(kt + 1) & 1] + BN * kBK, ra, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: y = acc * (s_act * s_w), fp32 row-major
    if (S.s > 1 && !split_reduce<TN, TM, NT>(acc, S, t, chunk, arrival, tid)) return;
    store_tile<TN, TM, WTN, WTM>(acc, Y, M, N, m0 + wm * WTM, n0 + wn * WTN, lane,
                                 F16 ? 1.0f : act_scale[1] * w_scale);
}

// ---------------------------------------------------------------------------
// Skinny kernel: padded M <= 64 (one to four 16-row activation blocks).
//
// Here the product is bound by reading the weight once (N*K bytes; the
// activation bytes stay in L2), so the kernel keeps many weight loads in
// flight and needs no operand reuse across waves.  A workgroup of four
// waves owns 16 weight rows; wave w takes a quarter of the 128-byte K-steps.
// Loads are coalesced (8 lanes per 128-byte row segment: one load covers 8
// rows); MFMA operands need lane l to hold row l%16, so each wave passes its
// data through its own LDS region (row-major 128-byte rows, 16-byte chunks
// XOR-swizzled by row) and reads the 16x16x128 operands back.  The region
// is private to the wave, so the K loop has no workgroup barrier.  Steps go
// C at a time: while chunk c is staged and read from LDS, the loads of
// chunks c+1 and c+2 are in flight in two register sets.  The 128 K bytes of a step are dealt to the lane
// groups g = l/16 as chunks g and 4+g, the same for both operands (the sum
// over K does not depend on which lane carries which bytes).  Activation
// rows at or past M lie outside their block's buffer range and read as zero
// without memory traffic.  The four partial 16 x 16*MB tiles are added in
// wave order through LDS and stored.
// ---------------------------------------------------------------------------
typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kSkinnyWaves = 4;

template <int MB>
struct SkinnyCfg {
    static constexpr int C = MB == 1 ? 4 : 2;       // K-steps per chunk
    static constexpr int R = 16 * (1 + MB);         // LDS rows per step: weight, then activation blocks
    static constexpr int L = 2 * C * (1 + MB);      // 16-byte loads per lane per chunk
};

// Loads of chunk [s, s+C) (steps past s1 read as zero): for step c, load
// 2*(1+MB)*c + 2*o + h covers rows 8h..8h+7 of operand o (0: weight, 1+b:
// activation block b).
template <int MB>
__device__ __forceinline__ void skinny_load(u32x4 (&r)[SkinnyCfg<MB>::L], __amdgpu_buffer_rsrc_t wrs,
                                            const __amdgpu_buffer_rsrc_t (&ars)[MB], uint32_t voff, uint32_t K8,
                                            int s, int s1) {
    constexpr int C = SkinnyCfg<MB>::C;
    const __amdgpu_buffer_rsrc_t zr = tile_rsrc(nullptr, 0u);
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const bool in = s + c < s1;
        const uint32_t kb = (uint32_t)(s + c) * kBK;
#pragma unroll
        for (int o = 0; o < 1 + MB; ++o)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                r[2 * (1 + MB) * c + 2 * o + h] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(in ? (o == 0 ? wrs : ars[o > 0 ? o - 1 : 0]) : zr,
                                                                 voff + h * K8, kb, 0));
    }
}

template <int MB>
__device__ __forceinline__ void skinny_stage(uint8_t* lds, const u32x4 (&r)[SkinnyCfg<MB>::L], int lane) {
    constexpr int C = SkinnyCfg<MB>::C, R = SkinnyCfg<MB>::R;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int o = 0; o < 1 + MB; ++o)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 16 * o + 8 * h + (lane >> 3);
                *reinterpret_cast<u32x4*>(lds + (c * R + row) * kBK + (((lane & 7) ^ swz(row)) << 4)) =
                    r[2 * (1 + MB) * c + 2 * o + h];
            }
}

template <int MB>
__device__ __forceinline__ void skinny_mma(v4f (&acc)[MB], const uint8_t* lds, int lane) {
    constexpr int C = SkinnyCfg<MB>::C, R = SkinnyCfg<MB>::R;
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        v8i op[1 + MB];
#pragma unroll
        for (int o = 0; o < 1 + MB; ++o) {
            const int row = 16 * o + r;
            const uint8_t* base = lds + (c * R + row) * kBK;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(base + ((g ^ swz(row)) << 4));
            const u32x4 hi = *reinterpret_cast<const u32x4*>(base + (((4 + g) ^ swz(row)) << 4));
            op[o] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int b = 0; b < MB; ++b)
            acc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(op[0], op[1 + b], acc[b], 0, 0, 0, 0, 0, 0);
    }
}

template <int MB>
__global__ __launch_bounds__(64 * kSkinnyWaves) void fp8_gemm_skinny_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ Wt, float* __restrict__ Y, int M, int N, int K,
    const float* __restrict__ act_scale, float w_scale) {
    constexpr int C = SkinnyCfg<MB>::C, R = SkinnyCfg<MB>::R, L = SkinnyCfg<MB>::L;
    __shared__ __attribute__((aligned(16))) uint8_t stage[kSkinnyWaves][C * R * kBK];
    __shared__ v4f red[kSkinnyWaves][MB][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 16;
    const int KS = K / kBK;
    const int s0 = wave * KS / kSkinnyWaves, s1 = (wave + 1) * KS / kSkinnyWaves;
    // weight rows [n0, min(n0+16, N)) and activation rows [16b, min(16b+16,
    // M)) of block b: lanes of rows past the end get offsets outside the
    // resource (the range check covers the per-lane offset) and read zero
    const int rows_w = N - n0 < 16 ? N - n0 : 16;
    const __amdgpu_buffer_rsrc_t wrs = tile_rsrc(Wt + (size_t)n0 * K, (uint32_t)rows_w * (uint32_t)K);
    __amdgpu_buffer_rsrc_t ars[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        const int rows_a = M - 16 * b < 16 ? (M - 16 * b > 0 ? M - 16 * b : 0) : 16;
        ars[b] = tile_rsrc(A + (size_t)16 * b * K, (uint32_t)rows_a * (uint32_t)K);
    }
    const uint32_t voff = (uint32_t)(lane >> 3) * (uint32_t)K + 16u * (uint32_t)(lane & 7);
    const uint32_t K8 = 8u * (uint32_t)K;
    uint8_t* lds = stage[wave];
    v4f acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = (v4f){0.f, 0.f, 0.f, 0.f};
    // two register sets: chunks c+1 and c+2 are in flight while chunk c is
    // staged and multiplied
    u32x4 ra[L], rb[L];
    if (s0 < s1) skinny_load<MB>(ra, wrs, ars, voff, K8, s0, s1);
    if (s0 + C < s1) skinny_load<MB>(rb, wrs, ars, voff, K8, s0 + C, s1);
    for (int s = s0; s < s1; s += 2 * C) {
        skinny_stage<MB>(lds, ra, lane);
        if (s + 2 * C < s1) skinny_load<MB>(ra, wrs, ars, voff, K8, s + 2 * C, s1);
        skinny_mma<MB>(acc, lds, lane);
        if (s + C < s1) {
            skinny_stage<MB>(lds, rb, lane);
            if (s + 3 * C < s1) skinny_load<MB>(rb, wrs, ars, voff, K8, s + 3 * C, s1);
            skinny_mma<MB>(acc, lds, lane);
        }
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) red[wave][b][lane] = acc[b];
    __syncthreads();
    if (tid >= 64 * MB) return;
    // output block b, lane l: column m = 16b + l%16, rows n = n0 + 4*(l/16) + 0..3
    const int b = tid >> 6;
    v4f sum = red[0][b][lane];
#pragma unroll
    for (int w = 1; w < kSkinnyWaves; ++w) sum += red[w][b][lane];
    const int m = 16 * b + (lane & 15);
    const int n = n0 + 4 * (lane >> 4);
    if (m >= M) return;
    const float sc = act_scale[1] * w_scale;
    float* yrow = Y + (size_t)m * N;
    const float4 v = make_float4(sum[0] * sc, sum[1] * sc, sum[2] * sc, sum[3] * sc);
    if ((N & 3) == 0 && n + 3 < N) {
        *reinterpret_cast<float4*>(yrow + n) = v;
    } else {
        if (n < N) yrow[n] = v.x;
        if (n + 1 < N) yrow[n + 1] = v.y;
        if (n + 2 < N) yrow[n + 2] = v.z;
        if (n + 3 < N) yrow[n + 3] = v.w;
    }
}

// ---------------------------------------------------------------------------
// GEMV kernel: at most 3 real activation rows.  The MFMA tiles would be
// mostly padding rows here, so the products run on the vector ALU: one
// wave per weight row, lane l taking K bytes 1024c + 16l (c = 0, 1, ...) of
// the row and of each activation row, with coalesced 16-byte loads (a wave
// reads 1 KB of a row per load).  The bytes are decoded with
// v_cvt_pk_f32_fp8 (OCP E4M3FN, as the encoder writes them); the product of
// two decoded values is exact in fp32, and each lane accumulates its
// products in K order with fused multiply-adds.  The 64 lane sums are added
// by a butterfly over the wave and lane 0 stores y[m][n] for m < M.
// ---------------------------------------------------------------------------
typedef float v2f __attribute__((ext_vector_type(2)));
constexpr int kGemvPass = 4;  // 1 KB chunks of K loaded per pass

template <int MR>
__device__ __forceinline__ void gemv_fma16(float (&acc)[MR], const u32x4& w, const u32x4 (&a)[MR]) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const v2f w0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], false);
        const v2f w1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], true);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const v2f a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a[m][d], false);
            const v2f a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a[m][d], true);
            acc[m] = __builtin_fmaf(w0.x, a0.x, acc[m]);
            acc[m] = __builtin_fmaf(w0.y, a0.y, acc[m]);
            acc[m] = __builtin_fmaf(w1.x, a1.x, acc[m]);
            acc[m] = __builtin_fmaf(w1.y, a1.y, acc[m]);
        }
    }
}

template <int MR>
__global__ __launch_bounds__(256) void fp8_gemv_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ Wt,
                                                       float* __restrict__ Y, int N, int K,
                                                       const float* __restrict__ act_scale, float w_scale) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);  // one weight row per wave
    if (n >= N) return;                                // whole waves
    const __amdgpu_buffer_rsrc_t wrs = tile_rsrc(Wt + (size_t)n * K, (uint32_t)K);
    __amdgpu_buffer_rsrc_t ars[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) ars[m] = tile_rsrc(A + (size_t)m * K, (uint32_t)K);
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
    // offsets at or past K fall outside the resources and read zero
    for (int kb = 0; kb < K; kb += 1024 * kGemvPass) {
        u32x4 w[kGemvPass], a[kGemvPass][MR];
#pragma unroll
        for (int c = 0; c < kGemvPass; ++c) {
            const uint32_t off = (uint32_t)(kb + 1024 * c + 16 * lane);
            w[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0));
#pragma unroll
            for (int m = 0; m < MR; ++m)
                a[c][m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars[m], off, 0, 0));
        }
#pragma unroll
        for (int c = 0; c < kGemvPass; ++c) gemv_fma16<MR>(acc, w[c], a[c]);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int sh = 32; sh >= 1; sh >>= 1) acc[m] += __shfl_xor(acc[m], sh, 64);
    if (lane == 0) {
        const float sc = act_scale[1] * w_scale;
#pragma unroll
        for (int m = 0; m < MR; ++m) Y[(size_t)m * N + n] = acc[m] * sc;
    }
}

}  // namespace

hipError_t launch_gemm_edge(const GemmPlan& p, const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n,
                            uint32_t k, const float* act_scale, float w_scale, float* y, void* ws, hipStream_t st) {
    const int mp = (int)((m + 15u) & ~15u);
    const int tiles_m = (mp + p.bm - 1) / p.bm, tiles_n = ((int)n + p.bn - 1) / p.bn;
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    SplitK S = {1, (int)(k / 256u), nullptr, nullptr};
    if (p.s > 1) {
        S.s = p.s;
        S.cnt = static_cast<unsigned*>(ws);
        S.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kSplitCounterBytes);
    }
    switch (p.kind) {
        case kGemmLargeEdge:
            fp8_gemm_deep_kernel<256, 256, 2, 2, false><<<p.workgroups, p.threads, 0, st>>>(
                a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n, group_m, S);
            break;
        case kGemmMedium:
            fp8_gemm_deep_kernel<128, 128, 2, 2, true><<<p.workgroups, p.threads, 0, st>>>(
                a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n, group_m, S);
            break;
        case kGemmGemv:
            switch (m) {
                case 1: fp8_gemv_kernel<1><<<p.workgroups, p.threads, 0, st>>>(a_fp8, w_fp8, y, (int)n, (int)k, act_scale, w_scale); break;
                case 2: fp8_gemv_kernel<2><<<p.workgroups, p.threads, 0, st>>>(a_fp8, w_fp8, y, (int)n, (int)k, act_scale, w_scale); break;
                default: fp8_gemv_kernel<3><<<p.workgroups, p.threads, 0, st>>>(a_fp8, w_fp8, y, (int)n, (int)k, act_scale, w_scale); break;
            }
            break;
        case kGemmSkinny:
            switch (mp / 16) {
                case 1: fp8_gemm_skinny_kernel<1><<<p.workgroups, p.threads, 0, st>>>(
                            a_fp8, w_fp8, y, (int)m, (int)n, (int)k, act_scale, w_scale); break;
                case 2: fp8_gemm_skinny_kernel<2><<<p.workgroups, p.threads, 0, st>>>(
                            a_fp8, w_fp8, y, (int)m, (int)n, (int)k, act_scale, w_scale); break;
                case 3: fp8_gemm_skinny_kernel<3><<<p.workgroups, p.threads, 0, st>>>(
                            a_fp8, w_fp8, y, (int)m, (int)n, (int)k, act_scale, w_scale); break;
                default: fp8_gemm_skinny_kernel<4><<<p.workgroups, p.threads, 0, st>>>(
                            a_fp8, w_fp8, y, (int)m, (int)n, (int)k, act_scale, w_scale); break;
            }
            break;
        default:
            fp8_gemm_kernel<64, 32, 2, 1><<<p.workgroups, p.threads, 0, st>>>(
                a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n, group_m, S);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_edge_fp16(const GemmPlan& p, const uint8_t* a, const uint8_t* w, uint32_t m, uint32_t n,
                                 uint32_t kb, float* y, hipStream_t st) {
    const int mp = (int)((m + 15u) & ~15u);
    const int tiles_m = (mp + p.bm - 1) / p.bm, tiles_n = ((int)n + p.bn - 1) / p.bn;
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    const SplitK S = {1, (int)(kb / 256u), nullptr, nullptr};
    switch (p.kind) {
        case kGemmLargeEdge:
            fp8_gemm_deep_kernel<256, 256, 2, 2, false, true><<<p.workgroups, p.threads, 0, st>>>(
                a, w, y, (int)m, mp, (int)n, (int)kb, nullptr, 1.0f, tiles_m, tiles_n, group_m, S);
            break;
        case kGemmMedium:
            fp8_gemm_deep_kernel<128, 128, 2, 2, false, true><<<p.workgroups, p.threads, 0, st>>>(
                a, w, y, (int)m, mp, (int)n, (int)kb, nullptr, 1.0f, tiles_m, tiles_n, group_m, S);
            break;
        case kGemmSmall:
            fp8_gemm_kernel<64, 32, 2, 1, true><<<p.workgroups, p.threads, 0, st>>>(
                a, w, y, (int)m, mp, (int)n, (int)kb, nullptr, 1.0f, tiles_m, tiles_n, group_m, S);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rz
