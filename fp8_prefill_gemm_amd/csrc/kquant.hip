// Q4_K / Q6_K weight kernels: fp32 dequantisation (diagnostic) and the fused
// FP8 weight pack.
//
// Source: realizar 0.8.4 source page cublas_prefill/gemm.rs,
// get_or_cache_fp8_weight (dequantise -> per-tensor absmax -> scale 448/a,
// absmax 0 -> 1 -> scaled E4M3) and launch_dequant_q4k / launch_dequant_q6k
// (one super-block of 256 weights per unit of work, fp32 [N][K] row-major).
//
// The pages stage the dequantised weight in an fp32 scratch tensor (write 4,
// read 4, read 4 bytes per weight) before encoding.  Here the weight is
// dequantised in registers twice instead: pass 1 reduces per-workgroup
// absmax keys, pass 2 reduces those keys, derives the scales and re-decodes
// the blocks straight into E4M3 bytes.  Traffic per weight: 2 x 0.5625 + 1
// bytes (Q4_K), 2 x 0.8203 + 1 (Q6_K).  The decoded values are bit-identical
// in both passes (integer unpacking and exact products).
//
// Thread mapping.  Q4_K: a super-block is 8 units of 16 quant bytes; 8
// consecutive lanes take one block (its 16-byte header plus one 16-byte
// quant slice each), so a wave reads 8 whole consecutive blocks and writes
// their 2 KB of output.  Q6_K: 210-byte blocks are not 16-byte aligned, so a
// workgroup stages 64 consecutive blocks (13440 bytes, 16-byte aligned) into
// LDS with a 224-byte stride, then 4 lanes take one block.
#include "rz_device.h"
#include "rz_internal.h"

namespace rz {
namespace {

constexpr int kThreads = 256;
constexpr int kQ6Chunk = 64;  // Q6_K blocks staged per workgroup iteration

// Calls unit(...) for every decode unit of the tensor, in an order that keeps
// each wave on contiguous memory:
//   Q4_K: unit(b, s, head, qs) for block b and 16-byte quant slice s;
//   Q6_K: unit(b, h, l0, ql_a, ql_b, qh, sc4, dbits) (see q6k_load_unit).
template <int QT, typename F>
__device__ __forceinline__ void visit_units(const uint8_t* __restrict__ blocks, uint64_t nb, uint8_t* lds,
                                            F&& unit) {
    if constexpr (QT == 12) {
        // two units per iteration (g and g + stride), loads issued first
        const uint64_t units = nb * 8;
        const uint64_t stride = (uint64_t)gridDim.x * kThreads;
        for (uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x; g < units; g += 2 * stride) {
            const uint64_t g2 = g + stride;
            const bool two = g2 < units;
            const uint8_t* bp = blocks + (g >> 3) * kQ4Bytes;
            const uint8_t* bp2 = blocks + ((two ? g2 : g) >> 3) * kQ4Bytes;
            const uint4 head = *reinterpret_cast<const uint4*>(bp);
            const uint4 qs = *reinterpret_cast<const uint4*>(bp + 16 + 16 * (int)(g & 7));
            const uint4 head2 = *reinterpret_cast<const uint4*>(bp2);
            const uint4 qs2 = *reinterpret_cast<const uint4*>(bp2 + 16 + 16 * (int)(g2 & 7));
            unit(g >> 3, (int)(g & 7), head, qs);
            if (two) unit(g2 >> 3, (int)(g2 & 7), head2, qs2);
        }
    } else {
        const uint64_t nchunks = (nb + kQ6Chunk - 1) / kQ6Chunk;
        for (uint64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
            const uint64_t b0 = ch * kQ6Chunk;
            const int nbc = (int)((nb - b0) < (uint64_t)kQ6Chunk ? (nb - b0) : kQ6Chunk);
            q6k_stage<kThreads>(blocks + b0 * kQ6Bytes, nbc, lds);
            for (int t = threadIdx.x; t < nbc * 4; t += kThreads) {
                const int bl = t >> 2, h = (t >> 1) & 1, l0 = (t & 1) * 16;
                uint4 ql_a, ql_b, qh;
                uint32_t sc4, dbits;
                q6k_load_unit(lds, bl, h, l0, ql_a, ql_b, qh, sc4, dbits);
                unit(b0 + bl, h, l0, ql_a, ql_b, qh, sc4, dbits);
            }
            __syncthreads();  // LDS is restaged by the next iteration
        }
    }
}

// Calls f(first_element, vals[16]) for every run of 16 consecutive decoded
// weights of the tensor.
template <int QT, typename F>
__device__ __forceinline__ void visit_runs(const uint8_t* __restrict__ blocks, uint64_t nb, uint8_t* lds, F&& f) {
    if constexpr (QT == 12) {
        visit_units<12>(blocks, nb, lds, [&](uint64_t b, int s, uint4 head, uint4 qs) {
            Q4Unit u;
            q4k_decode_unit(head, qs, s, u);
            const uint64_t base = b * kQK + 64 * (s >> 1) + 16 * (s & 1);
            f(base, u.lo);
            f(base + 32, u.hi);
        });
    } else {
        visit_units<14>(blocks, nb, lds,
                        [&](uint64_t b, int h, int l0, uint4 ql_a, uint4 ql_b, uint4 qh, uint32_t sc4, uint32_t dbits) {
                            Q6Unit u;
                            q6k_decode_unit(ql_a, ql_b, qh, sc4, dbits, u);
                            const uint64_t base = b * kQK + 128 * h + l0;
#pragma unroll
                            for (int p = 0; p < 4; ++p) f(base + 32 * p, u.v[p]);
                        });
    }
}

template <int QT>
__global__ __launch_bounds__(kThreads) void dequant_f32_kernel(const uint8_t* __restrict__ blocks,
                                                               uint64_t nb,
                                                               float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[QT == 14 ? kQ6Chunk * kQ6LdsStride : 16];
    visit_runs<QT>(blocks, nb, lds, [&](uint64_t base, const float* v) {
        float4* o = reinterpret_cast<float4*>(out + base);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    });
}

// Pass 1: one absmax key per workgroup (from each unit's extreme quants).
template <int QT>
__global__ __launch_bounds__(kThreads) void pack_absmax_kernel(const uint8_t* __restrict__ blocks,
                                                               uint64_t nb,
                                                               uint32_t* __restrict__ partial) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[QT == 14 ? kQ6Chunk * kQ6LdsStride : 16];
    __shared__ uint32_t red[kThreads / kWave];
    uint32_t key = 0;
    if constexpr (QT == 12) {
        visit_units<12>(blocks, nb, lds, [&](uint64_t, int s, uint4 head, uint4 qs) {
            const uint32_t k = q4k_unit_key(head, qs, s);
            key = key > k ? key : k;
        });
    } else {
        visit_units<14>(blocks, nb, lds,
                        [&](uint64_t, int, int, uint4 ql_a, uint4 ql_b, uint4 qh, uint32_t sc4, uint32_t dbits) {
                            const uint32_t k = q6k_unit_key(ql_a, ql_b, qh, sc4, dbits);
                            key = key > k ? key : k;
                        });
    }
    key = block_max_u32<kThreads>(key, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = key;
}

// Pass 2: reduce the pass-1 keys, derive the scales, encode.  Workgroup 0
// publishes {a, q, dq, 0} to scale_out and, when given, {a, q, dq} to
// host_out (coherent host memory) followed by `ticket` in its fourth word,
// stored with release order at system scope: a host thread that sees the
// ticket there can read the scales while the codes are still being written.
template <int QT>
__global__ __launch_bounds__(kThreads) void pack_encode_kernel(const uint8_t* __restrict__ blocks,
                                                               uint64_t nb,
                                                               const uint32_t* __restrict__ partial,
                                                               int npartial,
                                                               uint8_t* __restrict__ w_fp8,
                                                               float* __restrict__ scale_out,
                                                               float* __restrict__ host_out, uint32_t ticket) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[QT == 14 ? kQ6Chunk * kQ6LdsStride : 16];
    __shared__ uint32_t red[kThreads / kWave];
    const Scales sc = scales_from_key(reduce_partials<kThreads>(partial, npartial, red));
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        scale_out[0] = sc.a;
        scale_out[1] = sc.q;
        scale_out[2] = sc.dq;
        scale_out[3] = 0.0f;
        if (host_out) {
            host_out[0] = sc.a;
            host_out[1] = sc.q;
            host_out[2] = sc.dq;
            __hip_atomic_store(reinterpret_cast<uint32_t*>(host_out) + 3, ticket, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
    const float q = sc.q;
    // With a finite absmax and a unit whose f16 scales are finite, every
    // product is finite and at most 448(1 + 2^-23) in magnitude: the wave
    // takes the short encoder when all its lanes qualify.
    const bool tensor_finite = sc.a <= 3.402823466e38f;
    if constexpr (QT == 12) {
        visit_units<12>(blocks, nb, lds, [&](uint64_t b, int s, uint4 head, uint4 qs) {
            Q4Unit u;
            q4k_decode_unit(head, qs, s, u);
            uint8_t* o = w_fp8 + b * kQK + 64 * (s >> 1) + 16 * (s & 1);
            const bool fast = tensor_finite && half_finite(head.x) && half_finite(head.x >> 16);
            if (__all(fast)) {
                *reinterpret_cast<uint4*>(o) = e4m3_scaled16<true>(u.lo, q);
                *reinterpret_cast<uint4*>(o + 32) = e4m3_scaled16<true>(u.hi, q);
            } else {
                *reinterpret_cast<uint4*>(o) = e4m3_scaled16(u.lo, q);
                *reinterpret_cast<uint4*>(o + 32) = e4m3_scaled16(u.hi, q);
            }
        });
    } else {
        visit_units<14>(blocks, nb, lds,
                        [&](uint64_t b, int h, int l0, uint4 ql_a, uint4 ql_b, uint4 qh, uint32_t sc4, uint32_t dbits) {
                            Q6Unit u;
                            uint8_t* o = w_fp8 + b * kQK + 128 * h + l0;
                            if (__all(tensor_finite && half_finite(dbits))) {
                                q6k_decode_unit<true>(ql_a, ql_b, qh, sc4, dbits, u);
#pragma unroll
                                for (int p = 0; p < 4; ++p)
                                    *reinterpret_cast<uint4*>(o + 32 * p) = e4m3_scaled16<true>(u.v[p], q);
                            } else {
                                q6k_decode_unit(ql_a, ql_b, qh, sc4, dbits, u);
#pragma unroll
                                for (int p = 0; p < 4; ++p)
                                    *reinterpret_cast<uint4*>(o + 32 * p) = e4m3_scaled16(u.v[p], q);
                            }
                        });
    }
}

// Workgroups that cover the tensor once (one pass of the visit loop).
uint64_t groups_for(int qtype, uint64_t nb) {
    return qtype == 12 ? (nb * 8 + kThreads - 1) / kThreads : (nb + kQ6Chunk - 1) / kQ6Chunk;
}

int clamp_groups(uint64_t g, int cap) {
    if (g < 1) g = 1;
    return (int)(g > (uint64_t)cap ? (uint64_t)cap : g);
}

}  // namespace

hipError_t launch_dequant_f32(int qtype, const uint8_t* blocks, uint64_t nb, float* out,
                              hipStream_t st) {
    const int grid = clamp_groups(groups_for(qtype, nb), 1 << 16);
    if (qtype == 12)
        dequant_f32_kernel<12><<<grid, kThreads, 0, st>>>(blocks, nb, out);
    else
        dequant_f32_kernel<14><<<grid, kThreads, 0, st>>>(blocks, nb, out);
    return hipGetLastError();
}

hipError_t launch_pack(int qtype, const uint8_t* blocks, uint64_t nb, uint8_t* w_fp8, uint8_t* ws,
                       float* host_scale, uint32_t ticket, hipStream_t st) {
    uint32_t* partial = reinterpret_cast<uint32_t*>(ws);
    float* scale_out = reinterpret_cast<float*>(ws + kWsScaleOffset);
    const int g1 = clamp_groups(groups_for(qtype, nb), kMaxPartials);
    const int g2 = clamp_groups(groups_for(qtype, nb), kMaxPartials);
    if (qtype == 12) {
        pack_absmax_kernel<12><<<g1, kThreads, 0, st>>>(blocks, nb, partial);
        pack_encode_kernel<12><<<g2, kThreads, 0, st>>>(blocks, nb, partial, g1, w_fp8, scale_out, host_scale, ticket);
    } else {
        pack_absmax_kernel<14><<<g1, kThreads, 0, st>>>(blocks, nb, partial);
        pack_encode_kernel<14><<<g2, kThreads, 0, st>>>(blocks, nb, partial, g1, w_fp8, scale_out, host_scale, ticket);
    }
    return hipGetLastError();
}

}  // namespace rz
