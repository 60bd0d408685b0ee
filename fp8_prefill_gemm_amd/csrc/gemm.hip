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
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Global -> registers: L x 16 bytes per thread of a [rows][128-byte] K-slice
// starting at column kb; rows at or past `limit` read as zero.
template <int L, int NT>
__device__ __forceinline__ void load_rows(uint4 (&r)[L], const uint8_t* __restrict__ src, int row0,
                                          int limit, int K, int kb, int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int idx = tid + i * NT;
        const int gr = row0 + (idx >> 3);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (gr < limit) v = *reinterpret_cast<const uint4*>(src + (size_t)gr * K + kb + ((idx & 7) << 4));
        r[i] = v;
    }
}

// Registers -> one LDS stage (128-byte rows, XOR-swizzled 16-byte chunks).
template <int L, int NT>
__device__ __forceinline__ void store_rows(uint8_t* dst, const uint4 (&r)[L], int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int idx = tid + i * NT;
        const int row = idx >> 3;
        *reinterpret_cast<uint4*>(dst + row * kBK + (((idx & 7) ^ swz(row)) << 4)) = r[i];
    }
}

// One 32-byte MFMA operand: row `row`, chunks c0 and c0+1 of a stage.
__device__ __forceinline__ v8i frag(const uint8_t* base, int row, int c0) {
    const uint8_t* r = base + row * kBK;
    const uint4 lo = *reinterpret_cast<const uint4*>(r + ((c0 ^ swz(row)) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(r + (((c0 + 1) ^ swz(row)) << 4));
    return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
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

    uint4 rw[LW], ra[LA];
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
constexpr KindInfo kKinds[3] = {{256, 256, 512}, {128, 128, 256}, {64, 32, 128}};

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
            fp8_gemm_kernel<256, 256, 2, 4><<<p.workgroups, p.threads, 0, st>>>(
                a_fp8, w_fp8, y, (int)m, mp, (int)n, (int)k, act_scale, w_scale, tiles_m, tiles_n,
                group_m);
            break;
        case kMedium:
            fp8_gemm_kernel<128, 128, 2, 2><<<p.workgroups, p.threads, 0, st>>>(
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
