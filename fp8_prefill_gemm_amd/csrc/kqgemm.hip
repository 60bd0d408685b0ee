// FP8 GEMM straight from the K-quant weight blocks: no FP8 copy of the
// weight is kept.
//
// It computes what the pack plus the FP8 GEMM compute (realizar 0.8.4
// source page cublas_prefill/gemm.rs, get_or_cache_fp8_weight and
// cublas_prefill_fp8_gemm): Y = dec(A) * dec(Wq)^T * (act dq * w dq), with
// Wq = E4M3(RN(w * q)) the per-tensor scaled codes of the dequantised
// weight.  The weight's scale pair {q, dq} comes from its absmax (one pass
// over the blocks, done once per weight); the codes are made inside the
// GEMM: each workgroup decodes the K-quant blocks of its weight rows, one
// half super-block (128 weights) per row and K-step, encodes them with q
// and writes them to the LDS stage the MFMAs read.  The codes are the
// pack's bytes exactly (same exact decode, same encoder), so only the
// accumulation order can differ from the cached path.  This trades the
// 1 byte per weight cache (and its HBM read) for re-decoding every block
// once per 128-row activation tile: the decode is vector-ALU work that
// runs beside the MFMAs of the other workgroup on the CU.
//
// Tiles: 128 weight rows x 128 activation rows, four waves of 64 x 64
// (2 x 2 MFMA 32x32x64 tiles), K-steps of 128 bytes through two LDS stages
// (the fp8 GEMM's row layout: 128-byte rows, 16-byte chunks XOR-swizzled by
// row).  While a stage is multiplied, the raw blocks and activation chunks
// of the next step are in flight in registers; after the MFMAs they are
// decoded and stored to the other stage.
//
// Thread mapping of a K-step (half h = step & 1 of super-block step / 2):
//   Q4_K: thread t takes 16-byte quant slice s = 4h + t%4 (32 weights) of
//         rows t/4 and t/4 + 64, plus each row's 16-byte header;
//   Q6_K: thread t takes unit (h, l0 = 16 (t%2)) (64 weights) of row t/2.
// Weight rows at or past N are clamped to row N-1 (their products only
// reach outputs that are never stored); activation rows at or past the
// padded M read as zero.
#include "gemm_common.h"
#include "rz_device.h"
#include "rz_internal.h"

namespace rz {
namespace {
using namespace gemm;

constexpr int kNT = 256;
constexpr int kBN = 128, kBM = 128;  // weight rows, activation rows per tile
constexpr int kWTN = 64, kWTM = 64;  // wave tile
constexpr int kTN = kWTN / 32, kTM = kWTM / 32;
constexpr int kLA = kBM * 8 / kNT;   // activation 16-byte chunks per thread and step
constexpr int kGroupM = 8;           // m-tiles per group in the tile order
constexpr int kStage = (kBN + kBM) * kBK;

template <int QT>
struct RawW;
template <>
struct RawW<12> {
    uint4 head[2], qs[2];
};
template <>
struct RawW<14> {
    uint4 ql_a, ql_b, qh;
    uint32_t sc4, dbits;
};

// Raw blocks of K-step kt for this thread's rows.
template <int QT>
__device__ __forceinline__ void load_w(RawW<QT>& r, const uint8_t* __restrict__ blocks, int n0, int N, int KB, int kt,
                                       int tid) {
    const int kb = kt >> 1, h = kt & 1;
    if constexpr (QT == 12) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int row = n0 + (tid >> 2) + 64 * i;
            row = row < N ? row : N - 1;
            const uint8_t* blk = blocks + ((size_t)row * KB + kb) * kQ4Bytes;
            r.head[i] = *reinterpret_cast<const uint4*>(blk);
            r.qs[i] = *reinterpret_cast<const uint4*>(blk + 16 + 16 * (4 * h + (tid & 3)));
        }
    } else {
        int row = n0 + (tid >> 1);
        row = row < N ? row : N - 1;
        const uint8_t* blk = blocks + ((size_t)row * KB + kb) * kQ6Bytes;
        q6k_load_unit(blk, h, 16 * (tid & 1), r.ql_a, r.ql_b, r.qh, r.sc4, r.dbits);
    }
}

__device__ __forceinline__ void lds_chunk(uint8_t* stage, int row, int chunk, uint4 v) {
    *reinterpret_cast<uint4*>(stage + row * kBK + ((chunk ^ swz(row)) << 4)) = v;
}

// Decode + encode the raw blocks into the weight rows of an LDS stage.
template <int QT>
__device__ __forceinline__ void store_w(uint8_t* stage, const RawW<QT>& r, int kt, float q, int tid) {
    const int h = kt & 1;
    if constexpr (QT == 12) {
        const int u = tid & 3;
        const int c_lo = 4 * (u >> 1) + (u & 1);  // chunk of the low-nibble run; the high one is 2 further
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            Q4Unit v;
            q4k_decode_unit(r.head[i], r.qs[i], 4 * h + u, v);
            const int row = (tid >> 2) + 64 * i;
            lds_chunk(stage, row, c_lo, e4m3_scaled16(v.lo, q));
            lds_chunk(stage, row, c_lo + 2, e4m3_scaled16(v.hi, q));
        }
    } else {
        Q6Unit v;
        q6k_decode_unit(r.ql_a, r.ql_b, r.qh, r.sc4, r.dbits, v);
        const int row = tid >> 1, c0 = tid & 1;
#pragma unroll
        for (int p = 0; p < 4; ++p) lds_chunk(stage, row, 2 * p + c0, e4m3_scaled16(v.v[p], q));
    }
}

// Tile of workgroup w: XCD x = w % 8 owns a contiguous range of the T tiles.
__device__ __forceinline__ bool tile_of(int w, int T, int& t) {
    const int tall = T / kXcds, rem = T % kXcds;
    const int x = w % kXcds, j = w / kXcds;
    if (j >= tall + (x < rem ? 1 : 0)) return false;
    t = x * tall + (x < rem ? x : rem) + j;
    return true;
}

template <int QT>
__global__ __launch_bounds__(kNT) void kq_fp8_gemm_kernel(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ blocks,
                                                          float* __restrict__ Y, int M, int Mp, int N, int K,
                                                          const float* __restrict__ act_scale, float w_q,
                                                          float w_dq, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2][kStage];

    int t;
    if (!tile_of(blockIdx.x, tiles_m * tiles_n, t)) return;
    int n0, m0;
    grouped_origin_bb<kBN, kBM>(t, tiles_m, tiles_n, kGroupM, n0, m0);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wn = wid & 1, wm = wid >> 1;
    const int KB = K / kQK, KT = K / kBK;

    v16f acc[kTN][kTM];
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j) acc[i][j] = (v16f){};

    RawW<QT> rw;
    u32x4 ra[kLA];
    load_w<QT>(rw, blocks, n0, N, KB, 0, tid);
    load_rows<kLA, kNT>(ra, A, m0, Mp, K, 0, tid);
    store_w<QT>(smem[0], rw, 0, w_q, tid);
    store_rows<kLA, kNT>(smem[0] + kBN * kBK, ra, tid);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        if (more) {
            load_w<QT>(rw, blocks, n0, N, KB, kt + 1, tid);
            load_rows<kLA, kNT>(ra, A, m0, Mp, K, (kt + 1) * kBK, tid);
        }
        const uint8_t* sw = smem[kt & 1];
        const uint8_t* sa = smem[kt & 1] + kBN * kBK;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int c0 = kk * 4 + (lane >> 5) * 2;
            v8i af[kTN], bf[kTM];
#pragma unroll
            for (int i = 0; i < kTN; ++i) af[i] = frag(sw, wn * kWTN + i * 32 + (lane & 31), c0);
#pragma unroll
            for (int j = 0; j < kTM; ++j) bf[j] = frag(sa, wm * kWTM + j * 32 + (lane & 31), c0);
#pragma unroll
            for (int i = 0; i < kTN; ++i)
#pragma unroll
                for (int j = 0; j < kTM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af[i], acc[i][j], 0, 0,
                                                                                0, 0, 0, 0);
        }
        if (more) {
            store_w<QT>(smem[(kt + 1) & 1], rw, kt + 1, w_q, tid);
            store_rows<kLA, kNT>(smem[(kt + 1) & 1] + kBN * kBK, ra, tid);
        }
        __syncthreads();
    }

    store_tile<kTN, kTM, kWTN, kWTM>(acc, Y, M, N, m0 + wm * kWTM, n0 + wn * kWTN, lane, act_scale[1] * w_dq);
}

}  // namespace

hipError_t launch_kquant_fp8_gemm(const uint8_t* a_fp8, uint32_t m, const float* act_scale, int qtype,
                                  const uint8_t* blocks, uint32_t n, uint32_t k, float w_q, float w_dq, float* y,
                                  hipStream_t st) {
    const int mp = (int)((m + 15u) & ~15u);
    const int tiles_m = (mp + kBM - 1) / kBM, tiles_n = ((int)n + kBN - 1) / kBN;
    const int T = tiles_m * tiles_n;
    const int grid = (T + kXcds - 1) / kXcds * kXcds;
    if (qtype == 12)
        kq_fp8_gemm_kernel<12><<<grid, kNT, 0, st>>>(a_fp8, blocks, y, (int)m, mp, (int)n, (int)k, act_scale, w_q,
                                                      w_dq, tiles_m, tiles_n);
    else
        kq_fp8_gemm_kernel<14><<<grid, kNT, 0, st>>>(a_fp8, blocks, y, (int)m, mp, (int)n, (int)k, act_scale, w_q,
                                                      w_dq, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace rz
