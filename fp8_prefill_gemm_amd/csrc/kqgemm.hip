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
// once per activation tile: vector-ALU work (about 7 operations per weight)
// that runs beside the MFMAs of the other waves on the CU.  The decode per
// product falls with the tile's activation rows, so padded M >= 512 takes
// 256-row tiles (eight waves, 96 KB of LDS), smaller M 128-row tiles (four
// waves, 64 KB).
//
// Tiles: 128 weight rows x BM activation rows, waves of 64 x 64 (2 x 2 MFMA
// 32x32x64 tiles), K-steps of 128 bytes through two LDS stages (the fp8
// GEMM's row layout: 128-byte rows, 16-byte chunks XOR-swizzled by row).
// While a stage is multiplied, the raw blocks and activation chunks of the
// step after next are loaded into one of two register sets, and the other
// set (loaded one step earlier) is decoded and stored to the other stage
// after the MFMAs (3 % faster than one set loaded one step ahead).
//
// Thread mapping of a K-step (half h = step & 1 of super-block step / 2),
// rows t/4 + i NT/4 for thread t of NT (each thread 32 weights per row):
//   Q4_K: 16-byte quant slice s = 4h + t%4, plus the row's 16-byte header;
//   Q6_K: runs p = t%2 and t%2 + 2 at l0 = 16 ((t/2)%2) (see load_w).
// Weight rows at or past N are clamped to row N-1 (their products only
// reach outputs that are never stored); activation rows at or past the
// padded M read as zero.
#include <type_traits>

#include "gemm_common.h"
#include "rz_device.h"
#include "rz_internal.h"

namespace rz {
namespace {
using namespace gemm;

constexpr int kBN = 128;             // weight rows per tile
constexpr int kWTN = 64, kWTM = 64;  // wave tile
constexpr int kTN = kWTN / 32, kTM = kWTM / 32;
constexpr int kGroupM = 8;           // m-tiles per group in the tile order

// Raw blocks of one K-step for P = 512 / NT weight rows of this thread.
template <int QT, int P>
struct RawW;
template <int P>
struct RawW<12, P> {
    uint4 head[P], qs[P];
};
template <int P>
struct RawW<14, P> {
    uint4 ql[P], qh[P];
    uint32_t sc2[P], dbits[P];  // sc2: the int8 scales of runs j and j + 2 (bytes 0, 1)
};

// Raw blocks of K-step kt.  Q4_K: thread t takes quant slice s = 4h + t%4
// of rows t/4 + i NT/4.  Q6_K: thread t takes, of rows t/4 + i NT/4, the
// runs p = j and j + 2 (j = t%2) at l0 = 16 ((t/2)%2) of half h: their low
// bits are the low and high nibbles of ql[64h + 32j + l0 ..+16], their high
// bits bit pairs 2j and 2j + 4 of qh[32h + l0 ..+16], their scales
// scales[8h + l0/16 + 2p].
template <int QT, int NT>
__device__ __forceinline__ void load_w(RawW<QT, 512 / NT>& r, const uint8_t* __restrict__ blocks, int n0, int N,
                                       int KB, int kt, int tid) {
    constexpr int P = 512 / NT;
    const int kb = kt >> 1, h = kt & 1;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        int row = n0 + (tid >> 2) + i * (NT / 4);
        row = row < N ? row : N - 1;
        if constexpr (QT == 12) {
            const uint8_t* blk = blocks + ((size_t)row * KB + kb) * kQ4Bytes;
            r.head[i] = *reinterpret_cast<const uint4*>(blk);
            r.qs[i] = *reinterpret_cast<const uint4*>(blk + 16 + 16 * (4 * h + (tid & 3)));
        } else {
            const uint8_t* blk = blocks + ((size_t)row * KB + kb) * kQ6Bytes;
            const int j = tid & 1, l0 = 16 * ((tid >> 1) & 1);
            r.ql[i] = ld16_a2(blk + 64 * h + 32 * j + l0);
            r.qh[i] = ld16_a2(blk + 128 + 32 * h + l0);
            const uint8_t* sc = blk + 192 + 8 * h + (l0 >> 4) + 2 * j;
            r.sc2[i] = (uint32_t)sc[0] | ((uint32_t)sc[4] << 8);
            r.dbits[i] = *reinterpret_cast<const uint16_t*>(blk + 208);
        }
    }
}

__device__ __forceinline__ void lds_chunk(uint8_t* stage, int row, int chunk, uint4 v) {
    *reinterpret_cast<uint4*>(stage + row * kBK + ((chunk ^ swz(row)) << 4)) = v;
}

// Codes of RN(v[i] * q), i < 16, for finite v[i] (and the finite q the
// entry point checks): a product may overflow to +-Inf but is never NaN, so
// the converter only needs the clamp to +-448 and the flush below 2^-6 (the
// same codes e4m3_scaled16 gives for such inputs).
__device__ __forceinline__ uint4 encode16_no_nan(const float v[16], float q) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float y[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float p = v[4 * i + b] * q;
            const float t = __builtin_amdgcn_fmed3f(p, -kFp8Max, kFp8Max);
            y[b] = (fabsf(p) < 0.015625f) ? 0.0f : t;
        }
        int c = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], c, true);
    }
    return (uint4){w[0], w[1], w[2], w[3]};
}

template <bool kFin>
__device__ __forceinline__ uint4 encode16(const float v[16], float q) {
    if constexpr (kFin)
        return encode16_no_nan(v, q);
    else
        return e4m3_scaled16(v, q);
}

// Q6_K runs p = j and j + 2 of a half-unit: 16 values each.  kFin: d is
// finite, so ds * (q - 32), which is exact (at most 23 significant bits),
// is formed as one fused multiply-add ds * q - 32 ds.
template <bool kFin>
__device__ __forceinline__ void q6k_decode_half(uint4 ql, uint4 qh, int j, uint32_t sc2, uint32_t dbits,
                                                float (&v0)[16], float (&v1)[16]) {
    const float d = half_bits_to_float(dbits);
    const float ds0 = d * (float)(int8_t)(sc2 & 0xFFu);
    const float ds1 = d * (float)(int8_t)((sc2 >> 8) & 0xFFu);
    const uint32_t X[4] = {ql.x, ql.y, ql.z, ql.w};
    const uint32_t H[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t q0 = (X[w] & 0x0F0F0F0Fu) | (((H[w] >> (2 * j)) & 0x03030303u) << 4);
        uint32_t q1 = ((X[w] >> 4) & 0x0F0F0F0Fu) | (((H[w] >> (2 * j + 4)) & 0x03030303u) << 4);
        asm("" : "+v"(q0), "+v"(q1));  // byte b converts with v_cvt_f32_ubyte<b>
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float f0 = (float)((q0 >> (8 * b)) & 0xFFu), f1 = (float)((q1 >> (8 * b)) & 0xFFu);
            v0[4 * w + b] = kFin ? __builtin_fmaf(ds0, f0, -32.0f * ds0) : ds0 * (f0 - 32.0f);
            v1[4 * w + b] = kFin ? __builtin_fmaf(ds1, f1, -32.0f * ds1) : ds1 * (f1 - 32.0f);
        }
    }
}

// Decode + encode the raw blocks into the weight rows of an LDS stage.
// Waves whose blocks all have finite f16 scales take the encoder without
// NaN handling (the decoded values are then finite).
template <int QT, int NT>
__device__ __forceinline__ void store_w(uint8_t* stage, const RawW<QT, 512 / NT>& r, int kt, float q, int tid) {
    constexpr int P = 512 / NT;
    const int h = kt & 1;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int row = (tid >> 2) + i * (NT / 4);
        if constexpr (QT == 12) {
            const int u = tid & 3;
            const int c_lo = 4 * (u >> 1) + (u & 1);  // chunk of the low-nibble run; the high one is 2 further
            Q4Unit v;
            q4k_decode_unit(r.head[i], r.qs[i], 4 * h + u, v);
            if (__all(half_finite(r.head[i].x) && half_finite(r.head[i].x >> 16))) {
                lds_chunk(stage, row, c_lo, encode16<true>(v.lo, q));
                lds_chunk(stage, row, c_lo + 2, encode16<true>(v.hi, q));
            } else {
                lds_chunk(stage, row, c_lo, encode16<false>(v.lo, q));
                lds_chunk(stage, row, c_lo + 2, encode16<false>(v.hi, q));
            }
        } else {
            const int j = tid & 1, c0 = (tid >> 1) & 1;
            float v0[16], v1[16];
            // run p at element 32p + l0 of the half: chunk 2p + l0/16
            if (__all(half_finite(r.dbits[i]))) {
                q6k_decode_half<true>(r.ql[i], r.qh[i], j, r.sc2[i], r.dbits[i], v0, v1);
                lds_chunk(stage, row, 2 * j + c0, encode16<true>(v0, q));
                lds_chunk(stage, row, 2 * (j + 2) + c0, encode16<true>(v1, q));
            } else {
                q6k_decode_half<false>(r.ql[i], r.qh[i], j, r.sc2[i], r.dbits[i], v0, v1);
                lds_chunk(stage, row, 2 * j + c0, encode16<false>(v0, q));
                lds_chunk(stage, row, 2 * (j + 2) + c0, encode16<false>(v1, q));
            }
        }
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

// BM activation rows per tile, 2 BM threads: waves 2 (along N) x BM/64.
template <int QT, int BM>
__global__ __launch_bounds__(2 * BM) void kq_fp8_gemm_kernel(const uint8_t* __restrict__ A,
                                                             const uint8_t* __restrict__ blocks,
                                                             float* __restrict__ Y, int M, int Mp, int N, int K,
                                                             const float* __restrict__ act_scale, float w_q,
                                                             float w_dq, int tiles_m, int tiles_n) {
    constexpr int NT = 2 * BM;
    constexpr int kLA = BM * 8 / NT;  // activation 16-byte chunks per thread and step
    constexpr int kStage = (kBN + BM) * kBK;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    int t;
    if (!tile_of(blockIdx.x, tiles_m * tiles_n, t)) return;
    int n0, m0;
    grouped_origin_bb<kBN, BM>(t, tiles_m, tiles_n, kGroupM, n0, m0);

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

    // two register sets: the raw blocks and activation chunks of step kt+2
    // are loaded while step kt is multiplied and step kt+1 (loaded one
    // iteration earlier) is decoded into the other stage
    RawW<QT, 512 / NT> rw[2];
    u32x4 ra[2][kLA];
    load_w<QT, NT>(rw[0], blocks, n0, N, KB, 0, tid);
    load_rows<kLA, NT>(ra[0], A, m0, Mp, K, 0, tid);
    if (KT > 1) {
        load_w<QT, NT>(rw[1], blocks, n0, N, KB, 1, tid);
        load_rows<kLA, NT>(ra[1], A, m0, Mp, K, kBK, tid);
    }
    store_w<QT, NT>(smem, rw[0], 0, w_q, tid);
    store_rows<kLA, NT>(smem + kBN * kBK, ra[0], tid);
    __syncthreads();

    auto step = [&](auto csc, int kt) {
        constexpr int cs = decltype(csc)::value;
        if (kt + 2 < KT) {
            load_w<QT, NT>(rw[cs], blocks, n0, N, KB, kt + 2, tid);
            load_rows<kLA, NT>(ra[cs], A, m0, Mp, K, (kt + 2) * kBK, tid);
        }
        const uint8_t* sw = smem + cs * kStage;
        const uint8_t* sa = sw + kBN * kBK;
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
        if (kt + 1 < KT) {
            uint8_t* nx = smem + (cs ^ 1) * kStage;
            store_w<QT, NT>(nx, rw[cs ^ 1], kt + 1, w_q, tid);
            store_rows<kLA, NT>(nx + kBN * kBK, ra[cs ^ 1], tid);
        }
        __syncthreads();
    };
    for (int kt = 0; kt < KT; kt += 2) {
        step(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < KT) step(std::integral_constant<int, 1>{}, kt + 1);
    }

    store_tile<kTN, kTM, kWTN, kWTM>(acc, Y, M, N, m0 + wm * kWTM, n0 + wn * kWTN, lane, act_scale[1] * w_dq);
}

template <int QT, int BM>
hipError_t launch_bm(const uint8_t* a_fp8, int m, int mp, const float* act_scale, const uint8_t* blocks, int n, int k,
                     float w_q, float w_dq, float* y, hipStream_t st) {
    constexpr int lds = 2 * (kBN + BM) * kBK;
    const int tiles_m = (mp + BM - 1) / BM, tiles_n = (n + kBN - 1) / kBN;
    const int T = tiles_m * tiles_n;
    const int grid = (T + kXcds - 1) / kXcds * kXcds;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kq_fp8_gemm_kernel<QT, BM>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    kq_fp8_gemm_kernel<QT, BM><<<grid, 2 * BM, lds, st>>>(a_fp8, blocks, y, m, mp, n, k, act_scale, w_q, w_dq,
                                                          tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kquant_fp8_gemm(const uint8_t* a_fp8, uint32_t m, const float* act_scale, int qtype,
                                  const uint8_t* blocks, uint32_t n, uint32_t k, float w_q, float w_dq, float* y,
                                  hipStream_t st) {
    const int mp = (int)((m + 15u) & ~15u);
    // 256-row activation tiles halve the decode work per product; below 512
    // rows they would leave too many rows of their tiles empty
    const bool wide = mp >= 512;
    if (qtype == 12)
        return wide ? launch_bm<12, 256>(a_fp8, (int)m, mp, act_scale, blocks, (int)n, (int)k, w_q, w_dq, y, st)
                    : launch_bm<12, 128>(a_fp8, (int)m, mp, act_scale, blocks, (int)n, (int)k, w_q, w_dq, y, st);
    return wide ? launch_bm<14, 256>(a_fp8, (int)m, mp, act_scale, blocks, (int)n, (int)k, w_q, w_dq, y, st)
                : launch_bm<14, 128>(a_fp8, (int)m, mp, act_scale, blocks, (int)n, (int)k, w_q, w_dq, y, st);
}

}  // namespace rz
