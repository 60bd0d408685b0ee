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
// Design (gfx950, wave64).  The weight is read once, at its K-quant size
// (0.5625 B per Q4_K weight, 0.8203 B per Q6_K weight), and never written
// back decoded.  Eight lanes share a super-block, 32 weights each (Q4_K:
// one 16-byte quant slice; Q6_K: one 16-byte ql run with its qh bits), so a
// wave covers eight blocks per step.  A workgroup of WAVES waves owns
// WAVES * RW consecutive rows and walks K in chunks of CB blocks:
//   1. every lane issues the loads of its pieces of the chunk for its RW
//      rows (all of them before any is used);
//   2. the workgroup copies the chunk of the activation (all batch rows)
//      into LDS, permuted so that the 32 values a lane needs are contiguous:
//      one 144-byte slot per (block, lane), so the eight 16-byte reads of a
//      slot by the 64 lanes of a wave hit distinct banks;
//   3. each lane decodes its pieces exactly as the dequantisation defines
//      them (one rounding) and multiplies them into its (row, batch row)
//      fp32 sums with fused multiply-adds, in K order; each activation value
//      read from LDS serves RW rows.
// A butterfly over the wave adds the 64 lane sums.  No workspace, no atomics.
// For a single batch row (and Q6_K at two) a barrier-free variant reads the
// activation straight into registers instead (kgemv_reg_kernel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rz_device.h"
#include "rz_internal.h"

namespace rz {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
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

constexpr int kLanesPerBlock = 8;                          // 32 weights per lane
constexpr int kBlocksPerStep = kWave / kLanesPerBlock;     // blocks a wave covers per step
constexpr int kSlotFloats = 36;                            // 32 values + 4 pad: slots 144 B apart
constexpr int kBlockFloats = kLanesPerBlock * kSlotFloats; // LDS floats per block and batch row
constexpr int kRegThreads = 256;                           // kgemv_reg_kernel group size

// Where element e (0..255) of a super-block lives in the LDS slots: lane
// (slot) u of the block and position in the slot.  Four consecutive elements
// starting at a multiple of 4 stay consecutive.
//   Q4_K: quant byte 32c + l holds element 64c + l (low nibble) and
//         64c + 32 + l (high nibble); lane u = 2c + l/16 takes bytes
//         32c + 16(u%2) .. +15: low nibbles at positions 0..15, high 16..31.
//   Q6_K: in half h, ql byte l / 32 + l (l < 32) and qh byte l give elements
//         l + 32p (p < 4: low nibble of ql[l], low nibble of ql[32+l], high
//         nibble of ql[l], high nibble of ql[32+l], with qh bits 2p..2p+1);
//         lane u = 4h + 2(l/16) + p%2 takes the ql run of p%2, runs p = p%2
//         (positions 0..15) and p%2 + 2 (positions 16..31).
template <int Q>
__device__ __forceinline__ int slot_of(int e, int& pos) {
    if constexpr (Q == 12) {
        const int c = e >> 6, w = e & 63, hi = w >> 5, l = w & 31;
        pos = 16 * hi + (l & 15);
        return 2 * c + (l >> 4);
    } else {
        const int h = e >> 7, w = e & 127, p = w >> 5, l = w & 31;
        pos = 16 * (p >> 1) + (l & 15);
        return 4 * h + 2 * (l >> 4) + (p & 1);
    }
}

// The raw bytes one lane needs from one block.
template <int Q>
struct Raw;
template <>
struct Raw<12> {
    uint4 head, qs;
};
template <>
struct Raw<14> {
    uint4 ql, qh;
    uint32_t sc, d;  // sc: the run's two int8 scales in bytes 0 and 1; d: f16 bits
};

__device__ __forceinline__ void load_raw(const uint8_t* blk, int u, Raw<12>& r) {
    r.head = ld16(blk);
    r.qs = ld16(blk + 16 + 16 * u);
}

// Q6_K blocks are 210 bytes, so they start 2-byte aligned: the 16-byte ql and
// qh runs are read with ld16_a2 (furthest byte: 2 past the qh run, inside
// the block), the two scales and d with byte and half-word loads.
__device__ __forceinline__ void load_raw(const uint8_t* blk, int u, Raw<14>& r) {
    const int h = u >> 2, l0 = 16 * ((u >> 1) & 1), odd = u & 1;
    r.ql = ld16_a2(blk + 64 * h + 32 * odd + l0);
    r.qh = ld16_a2(blk + 128 + 32 * h + l0);
    const int si = 192 + 8 * h + (l0 >> 4) + 2 * odd;
    r.sc = (uint32_t)blk[si] | ((uint32_t)blk[si + 4] << 8);
    r.d = *reinterpret_cast<const uint16_t*>(blk + 208);
}

// Decode a lane's 32 weights into slot order (w[pos]).
__device__ __forceinline__ void decode_raw(const Raw<12>& r, int u, float (&w)[32]) {
    Q4Unit q;
    q4k_decode_unit(r.head, r.qs, u, q);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        w[t] = q.lo[t];
        w[16 + t] = q.hi[t];
    }
}

// value = (d*sc)*(q-32): exact in fp32 (at most 24 significant bits).  With a
// finite d it is computed as one fused multiply-add d*sc*q - 32*d*sc (exact,
// so equal); an infinite or NaN d takes the product form, as the definition.
template <bool kFinite>
__device__ __forceinline__ void q6k_decode_run2(const Raw<14>& r, int shA, float (&w)[32]) {
    const float d = half_bits_to_float(r.d);
    const float dsA = d * (float)(int8_t)(r.sc & 0xFFu);
    const float dsB = d * (float)(int8_t)((r.sc >> 8) & 0xFFu);
    const uint32_t L[4] = {r.ql.x, r.ql.y, r.ql.z, r.ql.w};
    const uint32_t H[4] = {r.qh.x, r.qh.y, r.qh.z, r.qh.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t a = (L[i] & 0x0F0F0F0Fu) | (((H[i] >> shA) & 0x03030303u) << 4);
        uint32_t b = ((L[i] >> 4) & 0x0F0F0F0Fu) | (((H[i] >> (shA + 4)) & 0x03030303u) << 4);
        asm("" : "+v"(a), "+v"(b));  // byte b converts with v_cvt_f32_ubyte<b>
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
            const float qa = (float)((a >> (8 * bt)) & 0xFFu), qb = (float)((b >> (8 * bt)) & 0xFFu);
            w[4 * i + bt] = kFinite ? __builtin_fmaf(dsA, qa, -32.0f * dsA) : dsA * (qa - 32.0f);
            w[16 + 4 * i + bt] = kFinite ? __builtin_fmaf(dsB, qb, -32.0f * dsB) : dsB * (qb - 32.0f);
        }
    }
}

__device__ __forceinline__ void decode_raw(const Raw<14>& r, int u, float (&w)[32]) {
    const int shA = 2 * (u & 1);
    if (half_finite(r.d))
        q6k_decode_run2<true>(r, shA, w);
    else
        q6k_decode_run2<false>(r, shA, w);
}

template <int Q>
constexpr int block_bytes() {
    return Q == 12 ? kQ4Bytes : kQ6Bytes;
}

template <int Q, int MR, int RW, int CB, int WAVES>
__global__ __launch_bounds__(WAVES* kWave) void kgemv_kernel(const uint8_t* __restrict__ blocks, uint32_t n,
                                                             uint32_t nb, const float* __restrict__ x, uint32_t k,
                                                             float* __restrict__ y) {
    constexpr int kThreads = WAVES * kWave;
    constexpr int J = CB / kBlocksPerStep;  // steps per chunk
    extern __shared__ __attribute__((aligned(16))) float xs[];  // [MR][CB][kBlockFloats]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int u = lane & (kLanesPerBlock - 1);  // lane within its block
    const int bl = lane / kLanesPerBlock;       // block within a step
    const uint32_t r0 = (blockIdx.x * WAVES + tid / kWave) * RW;
    const bool active = r0 < n;  // inactive waves still take part in staging and barriers
    const uint8_t* rowp[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const uint32_t r = (r0 + i < n) ? r0 + i : n - 1;  // rows past n re-read the last row, not stored
        rowp[i] = blocks + (size_t)r * nb * block_bytes<Q>();
    }
    float acc[RW][MR];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) acc[i][mi] = 0.0f;

    // weight loads of a chunk (blocks past the chunk re-read its first block)
    auto load_chunk = [&](Raw<Q> (&raw)[J][RW], uint32_t cb0, int nbc) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int b = bl + kBlocksPerStep * j;
            const uint32_t blk = cb0 + (b < nbc ? b : 0);
#pragma unroll
            for (int i = 0; i < RW; ++i) load_raw(rowp[i] + (size_t)blk * block_bytes<Q>(), u, raw[j][i]);
        }
    };
    auto chunk_len = [&](uint32_t cb0) { return (nb - cb0) < (uint32_t)CB ? (int)(nb - cb0) : CB; };

    for (uint32_t cb0 = 0; cb0 < nb; cb0 += CB) {
        const int nbc = chunk_len(cb0);
        Raw<Q> raw[J][RW];
        if (active) load_chunk(raw, cb0, nbc);  // in flight while the activation is staged
        // the activation chunk into the LDS slots
        const int pieces = nbc * (kQK / 4);
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) {
            const float* src = x + (size_t)mi * k + (size_t)cb0 * kQK;
            for (int pc = tid; pc < pieces; pc += kThreads) {
                int pos;
                const int sl = slot_of<Q>((pc & 63) * 4, pos);
                const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * pc);
                *reinterpret_cast<f32x4*>(xs + (mi * CB + (pc >> 6)) * kBlockFloats + sl * kSlotFloats + pos) = v;
            }
        }
        __syncthreads();
        // decode and multiply
        if (active) {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int b = bl + kBlocksPerStep * j;
                if (b < nbc) {
                    float w[RW][32];
#pragma unroll
                    for (int i = 0; i < RW; ++i) decode_raw(raw[j][i], u, w[i]);
                    const float* xl = xs + b * kBlockFloats + u * kSlotFloats;
#pragma unroll
                    for (int mi = 0; mi < MR; ++mi) {
                        float xv[32];
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const f32x4 t4 = *reinterpret_cast<const f32x4*>(xl + mi * CB * kBlockFloats + 4 * c);
                            xv[4 * c] = t4.x;
                            xv[4 * c + 1] = t4.y;
                            xv[4 * c + 2] = t4.z;
                            xv[4 * c + 3] = t4.w;
                        }
#pragma unroll
                        for (int i = 0; i < RW; ++i) {
                            float a = acc[i][mi];
#pragma unroll
                            for (int t = 0; t < 32; ++t) a = __builtin_fmaf(w[i][t], xv[t], a);
                            acc[i][mi] = a;
                        }
                    }
                }
            }
        }
        __syncthreads();  // the next chunk overwrites the slots
    }
    if (active) store_sums<RW, MR>(acc, r0, n, y);
}

// The same product for the smallest batches without LDS or barriers: each
// lane loads its two runs of 16 activation values per block straight from
// global memory (they stay in L2) and uses them for the wave's RW rows; the
// waves of a group are independent.  Lane u of a block covers the same
// weights, in the same order, as in kgemv_kernel, so both give the same sums.
template <int Q>
__device__ __forceinline__ int run_a(int u) {  // first element of the lane's first run
    if constexpr (Q == 12)
        return 64 * (u >> 1) + 16 * (u & 1);
    else
        return 128 * (u >> 2) + 16 * ((u >> 1) & 1) + 32 * (u & 1);
}
template <int Q>
constexpr int run_gap() {  // second run = first + gap
    return Q == 12 ? 32 : 64;
}

template <int Q, int MR, int RW>
__global__ __launch_bounds__(kRegThreads) void kgemv_reg_kernel(const uint8_t* __restrict__ blocks, uint32_t n,
                                                                uint32_t nb, const float* __restrict__ x,
                                                                uint32_t k, float* __restrict__ y) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t r0 = (blockIdx.x * (kRegThreads / kWave) + threadIdx.x / kWave) * RW;
    if (r0 >= n) return;  // whole waves leave; no barriers
    const int u = lane & (kLanesPerBlock - 1);
    const int bl = lane / kLanesPerBlock;
    const int xa = run_a<Q>(u);
    const uint8_t* rowp[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const uint32_t r = (r0 + i < n) ? r0 + i : n - 1;  // rows past n re-read the last row, not stored
        rowp[i] = blocks + (size_t)r * nb * block_bytes<Q>();
    }
    float acc[RW][MR];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) acc[i][mi] = 0.0f;
    for (uint32_t b = bl; b < nb; b += kBlocksPerStep) {
        Raw<Q> raw[RW];
#pragma unroll
        for (int i = 0; i < RW; ++i) load_raw(rowp[i] + (size_t)b * block_bytes<Q>(), u, raw[i]);
        f32x4 xv[MR][8];
#pragma unroll
        for (int mi = 0; mi < MR; ++mi) {
            const float* xb = x + (size_t)mi * k + (size_t)b * kQK + xa;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                xv[mi][c] = *reinterpret_cast<const f32x4*>(xb + 4 * c);
                xv[mi][4 + c] = *reinterpret_cast<const f32x4*>(xb + run_gap<Q>() + 4 * c);
            }
        }
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            float w[32];
            decode_raw(raw[i], u, w);
#pragma unroll
            for (int mi = 0; mi < MR; ++mi) {
                float a = acc[i][mi];
#pragma unroll
                for (int t = 0; t < 32; ++t) a = __builtin_fmaf(w[t], xv[mi][t >> 2][t & 3], a);
                acc[i][mi] = a;
            }
        }
    }
    store_sums<RW, MR>(acc, r0, n, y);
}

// Launch shape (measured at N=4608, K=3584 Q4_K and N=3584, K=18944 Q6_K,
// m = 1 and 4): chunks of 8 blocks (LDS = MR * 9216 B); 4 waves per group,
// 8 for Q6_K at m >= 3; one row per wave except Q4_K at m >= 3 with
// n >= 4096, where two rows per wave halve the activation reads from LDS.
constexpr int kChunkBlocks = 8;

template <int Q, int MR, int RW, int WAVES>
hipError_t launch_q(const uint8_t* blocks, uint32_t n, uint32_t nb, const float* x, uint32_t k, float* y,
                    hipStream_t st) {
    constexpr size_t lds = (size_t)MR * kChunkBlocks * kBlockFloats * sizeof(float);
    auto kern = kgemv_kernel<Q, MR, RW, kChunkBlocks, WAVES>;
    if constexpr (lds > 65536) {
        // m = 8: 72 KB of the 160 KB per CU.  The opt-in is set at every such
        // launch (a host-side attribute, cheap), so it holds on whichever
        // device is current.
        const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr != hipSuccess) return attr;
    }
    const uint32_t waves = (n + RW - 1) / RW;
    const dim3 grid((waves + WAVES - 1) / WAVES), block(WAVES * kWave);
    kern<<<grid, block, lds, st>>>(blocks, n, nb, x, k, y);
    return hipGetLastError();
}

template <int Q, int MR, int RW>
hipError_t launch_reg(const uint8_t* blocks, uint32_t n, uint32_t nb, const float* x, uint32_t k, float* y,
                      hipStream_t st) {
    constexpr uint32_t kWavesPer = kRegThreads / kWave;
    const uint32_t waves = (n + RW - 1) / RW;
    kgemv_reg_kernel<Q, MR, RW><<<(waves + kWavesPer - 1) / kWavesPer, kRegThreads, 0, st>>>(blocks, n, nb, x, k, y);
    return hipGetLastError();
}

// m = 1 (and Q6_K at m = 2) take the register kernel: measured 5.97 against
// 6.52 us (Q4_K, N=4608, K=3584), 17.0 against 22.4 us (Q6_K, N=3584,
// K=18944), 3.7 against 6.4 us (N=512); above that the LDS kernel's shared
// activation reads win.
template <int MR>
hipError_t launch_mr(int qtype, const uint8_t* blocks, uint32_t n, uint32_t nb, const float* x, uint32_t k,
                     float* y, hipStream_t st) {
    if constexpr (MR == 1) {
        if (n < 2048u)  // few rows: one per wave keeps more waves in flight
            return qtype == 12 ? launch_reg<12, 1, 1>(blocks, n, nb, x, k, y, st)
                               : launch_reg<14, 1, 1>(blocks, n, nb, x, k, y, st);
        return qtype == 12 ? launch_reg<12, 1, 2>(blocks, n, nb, x, k, y, st)
                           : launch_reg<14, 1, 2>(blocks, n, nb, x, k, y, st);
    }
    if constexpr (MR == 2) {
        if (qtype == 14) return launch_reg<14, 2, 2>(blocks, n, nb, x, k, y, st);
    }
    if (qtype == 14) return launch_q<14, MR, 1, MR <= 2 ? 4 : 8>(blocks, n, nb, x, k, y, st);
    if (MR >= 3 && n >= 4096u) return launch_q<12, MR, 2, 4>(blocks, n, nb, x, k, y, st);
    return launch_q<12, MR, 1, 4>(blocks, n, nb, x, k, y, st);
}

}  // namespace

hipError_t launch_kquant_gemv(int qtype, const uint8_t* blocks, uint32_t n, uint32_t k, const float* x,
                              uint32_t m, float* y, hipStream_t st) {
    const uint32_t nb = k / kQK;
#define RZ_KGEMV_CASE(MR) \
    case MR:              \
        return launch_mr<MR>(qtype, blocks, n, nb, x, k, y, st);
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
