// Device helpers shared by the rz_fp8 kernels (gfx950, wave64).
//
// Sources: realizar 0.8.4 source pages cublas_prefill/mod.rs (the E4M3
// conversion kernels and ABSMAX_REDUCE_PTX) and cublas_prefill/gemm.rs
// (get_or_cache_fp8_weight, cublas_prefill_fp8_gemm); the Q4_K / Q6_K field
// layouts are the public GGUF K-quant formats (the pages fix only the block
// sizes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rz {

constexpr int kWave = 64;
constexpr int kQK = 256;          // weights per K-quant super-block
constexpr int kQ4Bytes = 144;     // Q4_K super-block bytes
constexpr int kQ6Bytes = 210;     // Q6_K super-block bytes
constexpr int kQ6LdsStride = 224; // Q6_K block stride when staged in LDS (16-aligned)
constexpr float kFp8Max = 448.0f; // largest finite E4M3 value, code 0x7E

// ---------------------------------------------------------------- E4M3
//
// FP32 -> E4M3 as the mod.rs page's conversion kernels define it: zero and
// fp32 subnormals -> 0x00; Inf/NaN -> sign|0x7E; biased exponent E = e-120,
// E < 1 flushes to 0x00 before any rounding, E > 15 saturates to sign|0x7E;
// the 20 dropped fraction bits round to nearest even (round bit 19, sticky
// bits 18..0) with a carry into E; a carry past E = 15 saturates.  A result
// of E = 15, m = 7 (the NaN code in E4M3FN) is saturated to sign|0x7E too.
// Pure integer arithmetic, so the result is bit-identical on any hardware.
__device__ __forceinline__ uint32_t e4m3_from_bits(uint32_t u) {
    const uint32_t s = (u >> 31) << 7;
    const uint32_t e = (u >> 23) & 0xFFu;
    const uint32_t f = u & 0x7FFFFFu;
    int E = (int)e - 120;
    uint32_t m3 = f >> 20;
    const uint32_t rb = (f >> 19) & 1u;
    const uint32_t sticky_or_odd = ((f & 0x7FFFFu) != 0u) | (m3 & 1u);
    m3 += rb & sticky_or_odd;
    E += (int)(m3 >> 3);
    m3 &= 7u;
    const bool sat = (e == 255u) | (E > 15) | ((E == 15) & (m3 == 7u));
    const bool zero = ((int)e - 120) < 1;
    uint32_t out = s | ((uint32_t)(E & 15) << 3) | m3;
    out = sat ? (s | 0x7Eu) : out;
    return zero ? 0u : out;
}

// E4M3 code of RN(x * q).  The product is one IEEE multiply (no contraction:
// there is nothing to fuse it with, and the build uses -ffp-contract=off).
// A NaN product encodes as the positive NaN does, 0x7E.
__device__ __forceinline__ uint32_t e4m3_scaled(float x, float q) {
    const float y = x * q;
    const uint32_t code = e4m3_from_bits(__float_as_uint(y));
    return (y != y) ? 0x7Eu : code;
}

// Pack 16 codes (one per float) into a uint4, byte i of the result = code i.
__device__ __forceinline__ uint4 pack16(const uint32_t c[16]) {
    uint4 r;
    r.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    r.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    r.z = c[8] | (c[9] << 8) | (c[10] << 16) | (c[11] << 24);
    r.w = c[12] | (c[13] << 8) | (c[14] << 16) | (c[15] << 24);
    return r;
}

// ---------------------------------------------------------------- absmax
//
// |x| as an ordered integer key: the bit pattern of |x| compares like the
// float for non-negative values; NaN maps to 0 so it never wins (the
// ABSMAX_REDUCE_PTX float max returns the non-NaN operand).  -0 maps to 0.
__device__ __forceinline__ uint32_t abs_key(float x) {
    const uint32_t a = __float_as_uint(x) & 0x7FFFFFFFu;
    return a > 0x7F800000u ? 0u : a;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
        v = v > o ? v : o;
    }
    return v;
}

// Max over the whole workgroup; every thread gets the result.  `smem` must
// hold one word per wave.  Contains barriers: call from all threads.
template <int kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* smem) {
    constexpr int kWaves = kThreads / kWave;
    v = wave_max_u32(v);
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    if (lane == 0) smem[wid] = v;
    __syncthreads();
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) r = r > smem[i] ? r : smem[i];
    __syncthreads();
    return r;
}

// The scale pair of a per-tensor absmax a (bit key): q = RN(448/a'),
// dq = RN(a'/448), a' = a or 1 when a == 0.  HIP's fp32 division is IEEE
// correctly rounded (the build keeps -fhip-fp32-correctly-rounded-divide-sqrt).
struct Scales {
    float a, q, dq;
};
__device__ __forceinline__ Scales scales_from_key(uint32_t key) {
    Scales s;
    s.a = __uint_as_float(key);
    const float ap = (s.a == 0.0f) ? 1.0f : s.a;
    s.q = kFp8Max / ap;
    s.dq = ap / kFp8Max;
    return s;
}

// Reduce `count` partial keys (written by an earlier kernel on the same
// stream) to one key; every thread gets it.  Contains barriers.
template <int kThreads>
__device__ __forceinline__ uint32_t reduce_partials(const uint32_t* __restrict__ part, int count,
                                                    uint32_t* smem) {
    uint32_t v = 0;
    for (int i = threadIdx.x; i < count; i += kThreads) {
        const uint32_t p = part[i];
        v = v > p ? v : p;
    }
    return block_max_u32<kThreads>(v, smem);
}

// ---------------------------------------------------------------- K-quants

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    _Float16 v;
    const uint16_t b = (uint16_t)h;
    __builtin_memcpy(&v, &b, 2);
    return (float)v;
}

__device__ __forceinline__ uint32_t byte_of(uint4 v, int i) {
    const uint32_t w = (i < 4) ? v.x : (i < 8) ? v.y : (i < 12) ? v.z : v.w;
    return (w >> (8 * (i & 3))) & 0xFFu;
}

// Q4_K: one "unit" is a 16-byte slice s (0..7) of the 128 quant bytes of a
// super-block.  It holds the low nibbles of 16 weights of sub-block 2c and
// the high nibbles of 16 weights of sub-block 2c+1, c = s/2, starting at
// element 64c + 16(s&1) and 64c + 32 + 16(s&1).  `head` is the first 16
// bytes of the block: f16 d, f16 dmin, 12 packed 6-bit scale/min bytes.
struct Q4Unit {
    float lo[16];  // elements 64c + 16(s&1) + t
    float hi[16];  // elements 64c + 32 + 16(s&1) + t
};

__device__ __forceinline__ void q4k_scale_min(uint4 head, int j, uint32_t& sc, uint32_t& mn) {
    // scale bytes start at byte 4 of the head
    if (j < 4) {
        sc = byte_of(head, 4 + j) & 63u;
        mn = byte_of(head, 8 + j) & 63u;
    } else {
        const uint32_t b = byte_of(head, 8 + j);  // scales[j+4]
        sc = (b & 15u) | ((byte_of(head, j) >> 6) << 4);       // top bits of scales[j-4]
        mn = (b >> 4) | ((byte_of(head, 4 + j) >> 6) << 4);    // top bits of scales[j]
    }
}

// value = (d*sc)*q - (dmin*m): both products are exact in fp32 (at most 21
// and 17 significant bits), so the single rounding of the subtraction gives
// the correctly rounded value whatever the evaluation order.
__device__ __forceinline__ void q4k_decode_unit(uint4 head, uint4 qs, int s, Q4Unit& u) {
    const float d = half_bits_to_float(head.x & 0xFFFFu);
    const float dmin = half_bits_to_float(head.x >> 16);
    const int c = s >> 1;
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min(head, 2 * c, sc0, m0);
    q4k_scale_min(head, 2 * c + 1, sc1, m1);
    const float d0 = d * (float)sc0, o0 = dmin * (float)m0;
    const float d1 = d * (float)sc1, o1 = dmin * (float)m1;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const uint32_t b = byte_of(qs, t);
        u.lo[t] = d0 * (float)(b & 15u) - o0;
        u.hi[t] = d1 * (float)(b >> 4) - o1;
    }
}

// Q6_K: one unit is (half h, l0 in {0,16}) of a super-block: 64 weights, four
// runs of 16 at elements 128h + 32p + l0 (p = 0..3).  ql_a = ql[64h+l0..+16],
// ql_b = ql[64h+32+l0..+16], qh = qh[32h+l0..+16], sc4 = the four int8 scales
// scales[8h + l0/16 + 2p] packed in one word (byte p), d = f16 bits.
// value = (d*sc)*(q-32) is exact in fp32 (at most 24 significant bits).
struct Q6Unit {
    float v[4][16];
};

__device__ __forceinline__ void q6k_decode_unit(uint4 ql_a, uint4 ql_b, uint4 qh, uint32_t sc4,
                                                uint32_t dbits, Q6Unit& u) {
    const float d = half_bits_to_float(dbits);
    float ds[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) ds[p] = d * (float)(int8_t)((sc4 >> (8 * p)) & 0xFFu);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const uint32_t a = byte_of(ql_a, t), b = byte_of(ql_b, t), h = byte_of(qh, t);
        const int q0 = (int)((a & 15u) | ((h & 3u) << 4)) - 32;
        const int q1 = (int)((b & 15u) | (((h >> 2) & 3u) << 4)) - 32;
        const int q2 = (int)((a >> 4) | (((h >> 4) & 3u) << 4)) - 32;
        const int q3 = (int)((b >> 4) | (((h >> 6) & 3u) << 4)) - 32;
        u.v[0][t] = ds[0] * (float)q0;
        u.v[1][t] = ds[1] * (float)q1;
        u.v[2][t] = ds[2] * (float)q2;
        u.v[3][t] = ds[3] * (float)q3;
    }
}

// Stage `nb` (<= 64) consecutive Q6_K blocks starting at `src` (16-byte
// aligned: the first block of a 64-block chunk) into LDS with a 224-byte
// stride, so that every 16-byte field of a block is 16-byte aligned in LDS.
// The tail of the tensor is read in 2-byte pieces so nothing past the last
// block is touched.  Must be called by all kThreads threads; ends with a
// barrier.
template <int kThreads>
__device__ __forceinline__ void q6k_stage(const uint8_t* __restrict__ src, int nb, uint8_t* lds) {
    const int bytes = nb * kQ6Bytes;
    const int nvec = (bytes + 15) >> 4;
    uint16_t* l16 = reinterpret_cast<uint16_t*>(lds);
    for (int i = threadIdx.x; i < nvec; i += kThreads) {
        const int p0 = i << 4;
        uint32_t w[4];
        if (p0 + 16 <= bytes) {
            const uint4 v = *reinterpret_cast<const uint4*>(src + p0);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
            const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src + p0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = (p0 + 4 * j < bytes) ? s16[2 * j] : 0u;
                const uint32_t hi = (p0 + 4 * j + 2 < bytes) ? s16[2 * j + 1] : 0u;
                w[j] = lo | (hi << 16);
            }
        }
        int blk = p0 / kQ6Bytes;
        int off = p0 - blk * kQ6Bytes;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (p0 + 2 * j < bytes) {
                l16[(blk * kQ6LdsStride + off) >> 1] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
            }
            off += 2;
            if (off == kQ6Bytes) { off = 0; ++blk; }
        }
    }
    __syncthreads();
}

// Read the unit (h, l0) of staged block `bl` from LDS.
__device__ __forceinline__ void q6k_load_unit(const uint8_t* lds, int bl, int h, int l0, uint4& ql_a,
                                              uint4& ql_b, uint4& qh, uint32_t& sc4, uint32_t& dbits) {
    const uint8_t* b = lds + bl * kQ6LdsStride;
    ql_a = *reinterpret_cast<const uint4*>(b + 64 * h + l0);
    ql_b = *reinterpret_cast<const uint4*>(b + 64 * h + 32 + l0);
    qh = *reinterpret_cast<const uint4*>(b + 128 + 32 * h + l0);
    const uint4 sc = *reinterpret_cast<const uint4*>(b + 192);
    const int base = 8 * h + (l0 >> 4);
    sc4 = byte_of(sc, base) | (byte_of(sc, base + 2) << 8) | (byte_of(sc, base + 4) << 16) |
          (byte_of(sc, base + 6) << 24);
    dbits = *reinterpret_cast<const uint16_t*>(b + 208);
}

}  // namespace rz
