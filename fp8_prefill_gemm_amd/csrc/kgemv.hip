// Batched GEMV straight from Q4_K / Q6_K super-blocks, for small batches.
//
// Source: realizar 0.8.4, cublas_prefill/mod.rs page (the note on
// cublas_gemm_threshold: batches below a threshold, 4 by default, go to GEMV
// kernels instead of a GEMM) and q6k_gemv_indexed.rs page (the q4k_gemv_into
// and q6k_gemv_indexed_async dispatchers: fp32 input, K-quant weight read
// directly, fp32 output).  The pages print the dispatchers, not the kernels,
// so the operation is its plain definition:
//
//     y[i][j] = sum_kk x[i][kk] * w[j][kk],   w = the K-quant weight decoded
//                                             to fp32 (correctly rounded)
//
// Design (gfx950, wave64): the weight is read once, at its K-quant size
// (0.5625 B per Q4_K weight, 0.8203 B per Q6_K weight), and never written
// back decoded.  One wave owns RW consecutive weight rows.  Lane l takes a
// fixed piece of every super-block it visits (Q4_K: 16-byte quant slice
// l % 8 of block l / 8, 32 weights; Q6_K: quarter l % 4 of block l / 4, 64
// weights), so the activation values a lane needs are the same for all RW
// rows: each is loaded once per block and used RW times.  Every weight is
// decoded exactly as the dequantisation defines it (one rounding) and
// multiplied into its row's fp32 sums with fused multiply-adds, one sum per
// (row, batch row) per lane, in K order; a butterfly over the wave adds the
// 64 lane sums.  No workspace, no atomics, no LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rz_device.h"
#include "rz_internal.h"

namespace rz {
namespace {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// 16 bytes at a 2-byte-aligned address p: one 16-byte load at p rounded down
// to 4 bytes plus one more word, recombined with byte funnel shifts.  Every
// byte read lies in [p - 2, p + 18): the caller guarantees p + 18 stays
// inside the buffer when p is not 4-byte aligned (the extra word is then
// needed); when p is, the extra word read is the load's own last word.
__device__ __forceinline__ uint4 ld16_a2(const uint8_t* p) {
    const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(p) & 2u);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p - sh);  // keeps the global address space
    uint32_t v[4];
    __builtin_memcpy(v, w, 16);  // dword-aligned 16-byte load
    const uint32_t e = w[sh ? 4 : 3];
    uint4 r;
    r.x = __builtin_amdgcn_alignbyte(v[1], v[0], sh);
    r.y = __builtin_amdgcn_alignbyte(v[2], v[1], sh);
    r.z = __builtin_amdgcn_alignbyte(v[3], v[2], sh);
    r.w = __builtin_amdgcn_alignbyte(e, v[3], sh);
    return r;
}

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ void load_x16(const float* __restrict__ p, float (&o)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * i);
        o[4 * i] = v.x;
        o[4 * i + 1] = v.y;
        o[4 * i + 2] = v.z;
        o[4 * i + 3] = v.w;
    }
}

// Writes the RW x MR wave sums: lane 0 stores y[mi][r0 + i] for rows < n.
template <int RW, int MR>
__device__ __forceinline__ void store_sums(float (&acc)[RW][MR], uint32_t r0, uint32_t n, float* __restrict__ y) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) {
            const float s = wave_sum(acc[i][mi]);
            if (lane == 0 && r0 + i < n) y[(size_t)mi * n + r0 + i] = s;
        }
}

// ---------------------------------------------------------------- Q4_K
//
// Lane l: slice s = l % 8 of block b = l / 8 (+ 8 per step).  The slice's 16
// quant bytes hold the low nibbles of elements 64c + 16h + t and the high
// nibbles of elements 64c + 32 + 16h + t (c = s / 2, h = s % 2, t < 16).
template <int MR, int RW>
__global__ __launch_bounds__(kGemvThreads) void q4k_gemv_kernel(const uint8_t* __restrict__ blocks, uint32_t n,
                                                               uint32_t nb, const float* __restrict__ x,
                                                               uint32_t k, float* __restrict__ y) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t r0 = (blockIdx.x * kGemvWaves + threadIdx.x / kWave) * RW;
    if (r0 >= n) return;  // whole waves leave; no barriers below
    const int s = lane & 7;
    const int xoff = 64 * (s >> 1) + 16 * (s & 1);
    const uint8_t* rowp[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const uint32_t r = (r0 + i < n) ? r0 + i : n - 1;  // rows past n re-read the last row, not stored
        rowp[i] = blocks + (size_t)r * nb * kQ4Bytes + 16 * s;
    }
    float acc[RW][MR];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) acc[i][mi] = 0.0f;

    for (uint32_t b = lane >> 3; b < nb; b += 8) {
        Q4Unit u[RW];
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const uint8_t* blk = rowp[i] + (size_t)b * kQ4Bytes;
            const uint4 head = ld16(blk - 16 * s);
            const uint4 qs = ld16(blk + 16);
            q4k_decode_unit(head, qs, s, u[i]);
        }
        const float* xb = x + (size_t)b * kQK + xoff;
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) {
            float xl[16], xh[16];
            load_x16(xb + (size_t)mi * k, xl);
            load_x16(xb + (size_t)mi * k + 32, xh);
#pragma unroll
            for (int i = 0; i < RW; ++i) {
                float a = acc[i][mi];
#pragma unroll
                for (int t = 0; t < 16; ++t) a = __builtin_fmaf(u[i].lo[t], xl[t], a);
#pragma unroll
                for (int t = 0; t < 16; ++t) a = __builtin_fmaf(u[i].hi[t], xh[t], a);
                acc[i][mi] = a;
            }
        }
    }
    store_sums<RW, MR>(acc, r0, n, y);
}

// ---------------------------------------------------------------- Q6_K
//
// Lane l: quarter q = l % 4 of block b = l / 4 (+ 16 per step), i.e. half
// h = q / 2 and l0 = 16 (q % 2): the runs of 16 elements 128h + 32p + l0 + t
// (p < 4).  A block is 210 bytes, so blocks start 2-byte aligned; its 16-byte
// fields are read with ld16_a2.  The furthest byte read is 2 past the end of
// the 16 scale bytes (offset 208), inside the block.
template <int MR, int RW>
__global__ __launch_bounds__(kGemvThreads) void q6k_gemv_kernel(const uint8_t* __restrict__ blocks, uint32_t n,
                                                               uint32_t nb, const float* __restrict__ x,
                                                               uint32_t k, float* __restrict__ y) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t r0 = (blockIdx.x * kGemvWaves + threadIdx.x / kWave) * RW;
    if (r0 >= n) return;
    const int q = lane & 3;
    const int h = q >> 1, l0 = 16 * (q & 1);
    const int xoff = 128 * h + l0;
    const uint8_t* rowp[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const uint32_t r = (r0 + i < n) ? r0 + i : n - 1;
        rowp[i] = blocks + (size_t)r * nb * kQ6Bytes;
    }
    float acc[RW][MR];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) acc[i][mi] = 0.0f;

    for (uint32_t b = lane >> 2; b < nb; b += 16) {
        Q6Unit u[RW];
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const uint8_t* blk = rowp[i] + (size_t)b * kQ6Bytes;
            const uint4 ql_a = ld16_a2(blk + 64 * h + l0);
            const uint4 ql_b = ld16_a2(blk + 64 * h + 32 + l0);
            const uint4 qh = ld16_a2(blk + 128 + 32 * h + l0);
            const uint4 sc = ld16_a2(blk + 192);
            const uint32_t dbits = *reinterpret_cast<const uint16_t*>(blk + 208);
            const int base = 8 * h + (l0 >> 4);
            const uint32_t sc4 = byte_of(sc, base) | (byte_of(sc, base + 2) << 8) | (byte_of(sc, base + 4) << 16) |
                                 (byte_of(sc, base + 6) << 24);
            if (half_finite(dbits))
                q6k_decode_unit<true>(ql_a, ql_b, qh, sc4, dbits, u[i]);
            else
                q6k_decode_unit<false>(ql_a, ql_b, qh, sc4, dbits, u[i]);
        }
        const float* xb = x + (size_t)b * kQK + xoff;
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float xv[16];
                load_x16(xb + (size_t)mi * k + 32 * p, xv);
#pragma unroll
                for (int i = 0; i < RW; ++i) {
                    float a = acc[i][mi];
#pragma unroll
                    for (int t = 0; t < 16; ++t) a = __builtin_fmaf(u[i].v[p][t], xv[t], a);
                    acc[i][mi] = a;
                }
            }
        }
    }
    store_sums<RW, MR>(acc, r0, n, y);
}

template <int MR, int RW>
hipError_t launch_mr(int qtype, const uint8_t* blocks, uint32_t n, uint32_t nb, const float* x, uint32_t k,
                     float* y, hipStream_t st) {
    const uint32_t waves = (n + RW - 1) / RW;
    const dim3 grid((waves + kGemvWaves - 1) / kGemvWaves), block(kGemvThreads);
    if (qtype == 12)
        q4k_gemv_kernel<MR, RW><<<grid, block, 0, st>>>(blocks, n, nb, x, k, y);
    else
        q6k_gemv_kernel<MR, RW><<<grid, block, 0, st>>>(blocks, n, nb, x, k, y);
    return hipGetLastError();
}

}  // namespace

// Rows per wave: enough rows that each activation value loaded serves
// several weights, few enough that a small n still spreads over the chip.
int kgemv_rows_per_wave(uint32_t m, uint32_t n) {
    (void)m;
    return n >= 4096u ? 2 : 1;
}

hipError_t launch_kquant_gemv(int qtype, const uint8_t* blocks, uint32_t n, uint32_t k, const float* x,
                              uint32_t m, float* y, hipStream_t st) {
    const uint32_t nb = k / kQK;
    const int rw = kgemv_rows_per_wave(m, n);
#define RZ_KGEMV_CASE(MR)                                                                     \
    case MR:                                                                                  \
        return rw == 2 ? launch_mr<MR, 2>(qtype, blocks, n, nb, x, k, y, st)                  \
                       : launch_mr<MR, 1>(qtype, blocks, n, nb, x, k, y, st);
    switch (m) {
        RZ_KGEMV_CASE(1)
        RZ_KGEMV_CASE(2)
        RZ_KGEMV_CASE(3)
        RZ_KGEMV_CASE(4)
        RZ_KGEMV_CASE(5)
        RZ_KGEMV_CASE(6)
        RZ_KGEMV_CASE(7)
        RZ_KGEMV_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef RZ_KGEMV_CASE
}

}  // namespace rz
