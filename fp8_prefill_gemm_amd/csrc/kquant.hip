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
// absmax keys, one workgroup per weight reduces those keys and publishes
// the scales, and pass 2 re-decodes the blocks straight into E4M3 bytes
// with them.  Traffic per weight: 2 x 0.5625 + 1
// bytes (Q4_K), 2 x 0.8203 + 1 (Q6_K).  The decoded values are bit-identical
// in both passes (integer unpacking and exact products).
//
// Thread mapping.  Q4_K: a super-block is 8 units of 16 quant bytes; 8
// consecutive lanes take one block (its 16-byte header plus one 16-byte
// quant slice each), so a wave reads 8 whole consecutive blocks and writes
// their 2 KB of output.  Q6_K: 4 consecutive lanes take one block (a half
// and a 16-element offset each), so a wave reads 16 consecutive blocks;
// 210-byte blocks start 2-byte aligned, and each 16-byte field is read with
// a 4-byte-aligned load plus byte funnel shifts.  Each thread issues the
// loads of several units before it decodes the first.
#include "rz_device.h"
#include "rz_internal.h"

namespace rz {
namespace {

constexpr int kThreads = 256;
// Q4_K units (32 weights) per thread and loop iteration in the two pack
// passes; Q6_K takes half as many of its 64-weight units.
constexpr int kAbsmaxUnits = 4;
constexpr int kEncodeUnits = 2;

// Calls unit(...) for every decode unit of the tensor, U units per thread
// and iteration (unit g, g + stride, ...; all their loads are issued before
// the first is used), so that each wave stays on contiguous memory:
//   Q4_K: unit(b, s, head, qs) for block b and 16-byte quant slice s (8
//         lanes per block);
//   Q6_K: unit(b, h, l0, ql_a, ql_b, qh, sc4, dbits) for half h and l0 in
//         {0, 16} of block b (4 lanes per block; see q6k_load_unit).
// The tensor is shared by `ngroups` workgroups; this one is number `bid`.
template <int QT, int U, typename F>
__device__ __forceinline__ void visit_units(const uint8_t* __restrict__ blocks, uint64_t nb, int bid, int ngroups,
                                            F&& unit) {
    constexpr int kPer = QT == 12 ? 8 : 4;  // units per block
    const uint64_t units = nb * kPer;
    const uint64_t stride = (uint64_t)ngroups * kThreads;
    for (uint64_t g0 = (uint64_t)bid * kThreads + threadIdx.x; g0 < units; g0 += U * stride) {
        if constexpr (QT == 12) {
            uint4 head[U], qs[U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const uint64_t g = (g0 + i * stride < units) ? g0 + i * stride : g0;
                const uint8_t* bp = blocks + (g >> 3) * kQ4Bytes;
                head[i] = *reinterpret_cast<const uint4*>(bp);
                qs[i] = *reinterpret_cast<const uint4*>(bp + 16 + 16 * (int)(g & 7));
            }
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const uint64_t g = g0 + i * stride;
                if (g < units) unit(g >> 3, (int)(g & 7), head[i], qs[i]);
            }
        } else {
            uint4 ql_a[U], ql_b[U], qh[U];
            uint32_t sc4[U], dbits[U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const uint64_t g = (g0 + i * stride < units) ? g0 + i * stride : g0;
                q6k_load_unit(blocks + (g >> 2) * kQ6Bytes, (int)(g >> 1) & 1, (int)(g & 1) * 16, ql_a[i], ql_b[i],
                              qh[i], sc4[i], dbits[i]);
            }
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const uint64_t g = g0 + i * stride;
                if (g < units) unit(g >> 2, (int)(g >> 1) & 1, (int)(g & 1) * 16, ql_a[i], ql_b[i], qh[i], sc4[i], dbits[i]);
            }
        }
    }
}

// Calls f(first_element, vals[16]) for every run of 16 consecutive decoded
// weights of the tensor.
template <int QT, typename F>
__device__ __forceinline__ void visit_runs(const uint8_t* __restrict__ blocks, uint64_t nb, F&& f) {
    const int bid = blockIdx.x, ngroups = gridDim.x;
    if constexpr (QT == 12) {
        visit_units<12, 2>(blocks, nb, bid, ngroups, [&](uint64_t b, int s, uint4 head, uint4 qs) {
            Q4Unit u;
            q4k_decode_unit(head, qs, s, u);
            const uint64_t base = b * kQK + 64 * (s >> 1) + 16 * (s & 1);
            f(base, u.lo);
            f(base + 32, u.hi);
        });
    } else {
        visit_units<14, 1>(blocks, nb, bid, ngroups,
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
    visit_runs<QT>(blocks, nb, [&](uint64_t base, const float* v) {
        float4* o = reinterpret_cast<float4*>(out + base);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    });
}

// The fp16 weight cache of the FP16 comparator path (gemm.rs page,
// get_or_cache_fp16_weight): every weight dequantised as above, then
// rounded to fp16 (to nearest even, as cvt.rn.f16.f32 on the mod.rs page);
// fp16 [N][K] row-major, 32 bytes per run of 16.
// The pages round twice (the fp32 scratch value, then the fp16 conversion).
// The empty asm makes the fp32 values exist as such: otherwise the compiler
// folds the decode's fused multiply-add and the conversion into one
// v_fma_mix*_f16, which rounds the exact value straight to fp16 and differs
// from the two roundings at fp16 ties of the fp32 value.
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f16x2(float a, float b) {
    asm("" : "+v"(a), "+v"(b));
    return __builtin_bit_cast(uint32_t, (h2v){(_Float16)a, (_Float16)b});
}

template <int QT>
__global__ __launch_bounds__(kThreads) void fp16_pack_kernel(const uint8_t* __restrict__ blocks, uint64_t nb,
                                                             uint16_t* __restrict__ out) {
    visit_runs<QT>(blocks, nb, [&](uint64_t base, const float* v) {
        uint4* o = reinterpret_cast<uint4*>(out + base);
        o[0] = make_uint4(f16x2(v[0], v[1]), f16x2(v[2], v[3]), f16x2(v[4], v[5]), f16x2(v[6], v[7]));
        o[1] = make_uint4(f16x2(v[8], v[9]), f16x2(v[10], v[11]), f16x2(v[12], v[13]), f16x2(v[14], v[15]));
    });
}

// Pass 1 of one weight: this workgroup's absmax key (from each unit's
// extreme quants), reduced over the workgroup.
template <int QT>
__device__ __forceinline__ uint32_t absmax_part(const uint8_t* __restrict__ blocks, uint64_t nb, int bid, int ngroups,
                                                uint32_t* red) {
    uint32_t key = 0;
    if constexpr (QT == 12) {
        visit_units<12, kAbsmaxUnits>(blocks, nb, bid, ngroups, [&](uint64_t, int s, uint4 head, uint4 qs) {
            const uint32_t k = q4k_unit_key(head, qs, s);
            key = key > k ? key : k;
        });
    } else {
        visit_units<14, kAbsmaxUnits / 2>(blocks, nb, bid, ngroups,
                        [&](uint64_t, int, int, uint4 ql_a, uint4 ql_b, uint4 qh, uint32_t sc4, uint32_t dbits) {
                            const uint32_t k = q6k_unit_key(ql_a, ql_b, qh, sc4, dbits);
                            key = key > k ? key : k;
                        });
    }
    return block_max_u32<kThreads>(key, red);
}

// Pass 2 of one weight: re-decode this workgroup's units and encode them
// with the scale q.  With a finite absmax and a unit whose f16 scales are
// finite, every product is finite and at most 448(1 + 2^-23) in magnitude:
// the wave takes the short encoder when all its lanes qualify.
template <int QT>
__device__ __forceinline__ void encode_part(const uint8_t* __restrict__ blocks, uint64_t nb, int bid, int ngroups,
                                            uint8_t* __restrict__ w_fp8, float q, bool tensor_finite) {
    if constexpr (QT == 12) {
        visit_units<12, kEncodeUnits>(blocks, nb, bid, ngroups, [&](uint64_t b, int s, uint4 head, uint4 qs) {
            // each run of 16 encoded as soon as it is decoded (fewer live
            // registers, more waves per SIMD to overlap memory with the ALU)
            uint8_t* o = w_fp8 + b * kQK + 64 * (s >> 1) + 16 * (s & 1);
            const bool fast = tensor_finite && half_finite(head.x) && half_finite(head.x >> 16);
            float v[16];
            if (__all(fast)) {
                q4k_decode_run<false>(head, qs, s, v);
                *reinterpret_cast<uint4*>(o) = e4m3_scaled16<true>(v, q);
                q4k_decode_run<true>(head, qs, s, v);
                *reinterpret_cast<uint4*>(o + 32) = e4m3_scaled16<true>(v, q);
            } else {
                q4k_decode_run<false>(head, qs, s, v);
                *reinterpret_cast<uint4*>(o) = e4m3_scaled16(v, q);
                q4k_decode_run<true>(head, qs, s, v);
                *reinterpret_cast<uint4*>(o + 32) = e4m3_scaled16(v, q);
            }
        });
    } else {
        visit_units<14, kEncodeUnits / 2>(blocks, nb, bid, ngroups,
                        [&](uint64_t b, int h, int l0, uint4 ql_a, uint4 ql_b, uint4 qh, uint32_t sc4, uint32_t dbits) {
                            uint8_t* o = w_fp8 + b * kQK + 128 * h + l0;
                            float v[16];  // one run of 16 at a time
                            if (__all(tensor_finite && half_finite(dbits))) {
#pragma unroll
                                for (int p = 0; p < 4; ++p) {
                                    q6k_decode_run<true>(ql_a, ql_b, qh, sc4, dbits, p, v);
                                    *reinterpret_cast<uint4*>(o + 32 * p) = e4m3_scaled16<true>(v, q);
                                }
                            } else {
#pragma unroll
                                for (int p = 0; p < 4; ++p) {
                                    q6k_decode_run(ql_a, ql_b, qh, sc4, dbits, p, v);
                                    *reinterpret_cast<uint4*>(o + 32 * p) = e4m3_scaled16(v, q);
                                }
                            }
                        });
    }
}

// The weight of set P that workgroup b of a launch belongs to (`start` holds
// the first workgroup of each weight and, at [count], the grid size).
__device__ __forceinline__ int set_member(const int* start, int count, int b) {
    int i = 0;
    while (i + 1 < count && b >= start[i + 1]) ++i;
    return i;
}

// Pass 1 over a set of weights: weight i owns workgroups [g1[i], g1[i+1]),
// and each writes its key to partial[blockIdx.x].  QT = 12 / 14 when every
// weight of the set has that type, 0 for a mixed set (the type is then read
// per weight; it is uniform over a workgroup).
template <int QT>
__global__ __launch_bounds__(kThreads) void pack_absmax_kernel(PackSet P, uint32_t* __restrict__ partial) {
    __shared__ uint32_t red[kThreads / kWave];
    const int i = set_member(P.g1, P.count, blockIdx.x);
    const int bid = blockIdx.x - P.g1[i], ng = P.g1[i + 1] - P.g1[i];
    const int qt = QT ? QT : P.qtype[i];
    uint32_t key;
    if (qt == 12)
        key = absmax_part<12>(P.blocks[i], P.nb[i], bid, ng, red);
    else
        key = absmax_part<14>(P.blocks[i], P.nb[i], bid, ng, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = key;
}

// Workgroup i reduces weight i's pass-1 keys and publishes {a, q, dq, 0} to
// scale_out[4i..] and, when host[i] is given, {a, q, dq} to that coherent
// host memory followed by ticket[i] in its fourth word, stored with release
// order at system scope: a host thread that sees the ticket there can read
// the scales while pass 2 still writes the codes.
__global__ __launch_bounds__(kThreads) void pack_scales_kernel(PackSet P, const uint32_t* __restrict__ partial,
                                                               float* __restrict__ scale_out) {
    __shared__ uint32_t red[kThreads / kWave];
    const int i = blockIdx.x;
    const Scales sc = scales_from_key(reduce_partials<kThreads>(partial + P.g1[i], P.g1[i + 1] - P.g1[i], red));
    if (threadIdx.x == 0) {
        float* so = scale_out + 4 * i;
        so[0] = sc.a;
        so[1] = sc.q;
        so[2] = sc.dq;
        so[3] = 0.0f;
        if (float* ho = P.host[i]) {
            ho[0] = sc.a;
            ho[1] = sc.q;
            ho[2] = sc.dq;
            __hip_atomic_store(reinterpret_cast<uint32_t*>(ho) + 3, P.ticket[i], __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

// Pass 2 over a set of weights: weight i owns workgroups [g2[i], g2[i+1])
// (none when it has no output, w_fp8[i] null) and encodes with the q that
// pack_scales_kernel published in scale_out[4i + 1].
template <int QT>
__global__ __launch_bounds__(kThreads) void pack_encode_kernel(PackSet P, const float* __restrict__ scale_out) {
    const int i = set_member(P.g2, P.count, blockIdx.x);
    const int bid = blockIdx.x - P.g2[i], ng = P.g2[i + 1] - P.g2[i];
    const float a = scale_out[4 * i], q = scale_out[4 * i + 1];
    const bool tensor_finite = a <= 3.402823466e38f;
    const int qt = QT ? QT : P.qtype[i];
    if (qt == 12)
        encode_part<12>(P.blocks[i], P.nb[i], bid, ng, P.w_fp8[i], q, tensor_finite);
    else
        encode_part<14>(P.blocks[i], P.nb[i], bid, ng, P.w_fp8[i], q, tensor_finite);
}

// Workgroups that give every thread `per` units of a Q4_K tensor (`per` / 2
// of a Q6_K one).
uint64_t groups_for(int qtype, uint64_t nb, int per) {
    const uint64_t units = qtype == 12 ? nb * 8 : nb * 4;
    const uint64_t per_thread = qtype == 12 ? per : (per + 1) / 2;
    return (units + kThreads * per_thread - 1) / (kThreads * per_thread);
}

int clamp_groups(uint64_t g, int cap) {
    if (g < 1) g = 1;
    return (int)(g > (uint64_t)cap ? (uint64_t)cap : g);
}

}  // namespace

hipError_t launch_dequant_f32(int qtype, const uint8_t* blocks, uint64_t nb, float* out,
                              hipStream_t st) {
    const int grid = clamp_groups(groups_for(qtype, nb, 2), 1 << 16);
    if (qtype == 12)
        dequant_f32_kernel<12><<<grid, kThreads, 0, st>>>(blocks, nb, out);
    else
        dequant_f32_kernel<14><<<grid, kThreads, 0, st>>>(blocks, nb, out);
    return hipGetLastError();
}

hipError_t launch_fp16_pack(int qtype, const uint8_t* blocks, uint64_t nb, uint16_t* out, hipStream_t st) {
    const int grid = clamp_groups(groups_for(qtype, nb, 2), 1 << 16);
    if (qtype == 12)
        fp16_pack_kernel<12><<<grid, kThreads, 0, st>>>(blocks, nb, out);
    else
        fp16_pack_kernel<14><<<grid, kThreads, 0, st>>>(blocks, nb, out);
    return hipGetLastError();
}

int pack_absmax_groups(int qtype, uint64_t nb) {
    return clamp_groups(groups_for(qtype, nb, kAbsmaxUnits), kMaxPartials);
}

hipError_t launch_pack_set(int count, const int* qtype, const uint8_t* const* blocks, const uint64_t* nb,
                           uint8_t* const* w_fp8, uint8_t* ws, float* const* host_scale, const uint32_t* ticket,
                           hipStream_t st) {
    if (count < 1 || count > kMaxPackSet) return hipErrorInvalidValue;
    PackSet P{};
    P.count = count;
    bool same = true;
    for (int i = 0; i < count; ++i) {
        P.qtype[i] = qtype[i];
        P.blocks[i] = blocks[i];
        P.nb[i] = nb[i];
        P.w_fp8[i] = w_fp8[i];
        P.host[i] = host_scale ? host_scale[i] : nullptr;
        P.ticket[i] = ticket ? ticket[i] : 0u;
        P.g1[i + 1] = P.g1[i] + pack_absmax_groups(qtype[i], nb[i]);
        // pass 2 writes no keys: its grid is not capped at kMaxPartials (an
        // 18944 x 3584 weight takes 4144 workgroups; capped at 2048 the
        // step's pass 2 took 8 us longer)
        P.g2[i + 1] = P.g2[i] + (w_fp8[i] ? clamp_groups(groups_for(qtype[i], nb[i], kEncodeUnits), 1 << 16) : 0);
        same = same && qtype[i] == qtype[0];
    }
    if (P.g1[count] > kWsPartials) return hipErrorInvalidValue;
    uint32_t* partial = reinterpret_cast<uint32_t*>(ws);
    float* scale_out = reinterpret_cast<float*>(ws + kWsScaleOffset);
    const int g1 = P.g1[count], g2 = P.g2[count];
    if (same && qtype[0] == 12)
        pack_absmax_kernel<12><<<g1, kThreads, 0, st>>>(P, partial);
    else if (same)
        pack_absmax_kernel<14><<<g1, kThreads, 0, st>>>(P, partial);
    else
        pack_absmax_kernel<0><<<g1, kThreads, 0, st>>>(P, partial);
    pack_scales_kernel<<<count, kThreads, 0, st>>>(P, partial, scale_out);
    if (g2 == 0) return hipGetLastError();
    if (same && qtype[0] == 12)
        pack_encode_kernel<12><<<g2, kThreads, 0, st>>>(P, scale_out);
    else if (same)
        pack_encode_kernel<14><<<g2, kThreads, 0, st>>>(P, scale_out);
    else
        pack_encode_kernel<0><<<g2, kThreads, 0, st>>>(P, scale_out);
    return hipGetLastError();
}

hipError_t launch_pack(int qtype, const uint8_t* blocks, uint64_t nb, uint8_t* w_fp8, uint8_t* ws,
                       float* host_scale, uint32_t ticket, hipStream_t st) {
    return launch_pack_set(1, &qtype, &blocks, &nb, &w_fp8, ws, &host_scale, &ticket, st);
}

}  // namespace rz
