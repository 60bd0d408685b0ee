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
constexpr float kFp8Max = 448.0f; // largest finite E4M3 value, code 0x7E

// ---------------------------------------------------------------- E4M3
//
// FP32 -> E4M3 as the mod.rs page's conversion kernels define it: zero and
// fp32 subnormals -> 0x00; Inf/NaN -> sign|0x7E; biased exponent E = e-120,
// E < 1 (|y| < 2^-6) flushes to 0x00 before any rounding, E > 15 saturates to
// sign|0x7E; the 20 dropped fraction bits round to nearest even with a carry
// into E; a carry past E = 15, or a result of E = 15, m = 7 (the NaN code of
// E4M3FN), saturates to sign|0x7E.  So every |y| >= 448 gives sign|0x7E.
//
// gfx950's v_cvt_pk_fp8_f32 converts to OCP E4M3FN with round-to-nearest-
// even, which is the same map on 2^-6 <= |y| < 448.  Outside that range the
// input is replaced first so that the converter returns the pages' code:
// |y| < 2^-6 (and +-0, subnormals) -> +0 (0x00), |y| >= 448 and +-Inf ->
// +-448 (sign|0x7E), NaN -> +448 (0x7E; the scaled conversions map a NaN
// product to the code of the positive NaN).  The replacement plus the
// converter agree with the bitwise definition above on all 2^32 fp32 bit
// patterns except negative NaNs, which only the scaled path (0x7E) meets.
__device__ __forceinline__ float e4m3_prep(float y) {
    float t = __builtin_amdgcn_fmed3f(y, -kFp8Max, kFp8Max);
    t = (fabsf(y) < 0.015625f) ? 0.0f : t;
    return (y != y) ? kFp8Max : t;
}

// Fast form for values known to be finite with |y| <= 448 * (1 + 2^-23)
// (a finite weight or activation times q = RN(448/a) with |x| <= a): only
// the flush below 2^-6 remains; the converter rounds the rest to at most 448.
__device__ __forceinline__ float e4m3_prep_finite(float y) { return (fabsf(y) < 0.015625f) ? 0.0f : y; }

// Codes of four values in one word (byte i = value i).  The converter writes
// src0 to the low byte of the selected 16-bit half and src1 to the high one.
template <bool kFinite = false>
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    if constexpr (kFinite) {
        a = e4m3_prep_finite(a);
        b = e4m3_prep_finite(b);
        c = e4m3_prep_finite(c);
        d = e4m3_prep_finite(d);
    } else {
        a = e4m3_prep(a);
        b = e4m3_prep(b);
        c = e4m3_prep(c);
        d = e4m3_prep(d);
    }
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// E4M3 code of RN(x * q).  The product is one IEEE multiply (no contraction:
// there is nothing to fuse it with, and the build uses -ffp-contract=off).
__device__ __forceinline__ uint32_t e4m3_scaled(float x, float q) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prep(x * q), 0.0f, 0, false) & 0xFFu;
}

// Codes of RN(v[i] * q), i < 16, byte i of the result = code i.  kFinite:
// every product is known to be finite with |y| <= 448 * (1 + 2^-23).
template <bool kFinite = false>
__device__ __forceinline__ uint4 e4m3_scaled16(const float v[16], float q) {
    uint4 r;
    r.x = e4m3_pack4<kFinite>(v[0] * q, v[1] * q, v[2] * q, v[3] * q);
    r.y = e4m3_pack4<kFinite>(v[4] * q, v[5] * q, v[6] * q, v[7] * q);
    r.z = e4m3_pack4<kFinite>(v[8] * q, v[9] * q, v[10] * q, v[11] * q);
    r.w = e4m3_pack4<kFinite>(v[12] * q, v[13] * q, v[14] * q, v[15] * q);
    return r;
}

// f16 bit pattern (low 16 bits) of a finite value.
__device__ __forceinline__ bool half_finite(uint32_t h) { return (h & 0x7C00u) != 0x7C00u; }

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
// stream) to one key; every thread gets it.  Contains barriers.  Each
// thread issues the loads of up to 8 keys before it compares any, so the
// common case (count <= 8 * kThreads) waits for one round trip instead of
// one per key (a single workgroup runs this: measured 4.6 us per call with
// the loads one after another).
template <int kThreads>
__device__ __forceinline__ uint32_t reduce_partials(const uint32_t* __restrict__ part, int count,
                                                    uint32_t* smem) {
    constexpr int kPer = 8;
    uint32_t v = 0;
    for (int i0 = threadIdx.x; i0 < count; i0 += kPer * kThreads) {
        uint32_t p[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = i0 + u * kThreads;
            p[u] = i < count ? part[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) v = v > p[u] ? v : p[u];
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
    const uint32_t w[4] = {qs.x, qs.y, qs.z, qs.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // quant bytes 4i..4i+3: low nibbles -> lo, high nibbles -> hi (one
        // byte-to-float conversion per value)
        uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
        asm("" : "+v"(lo), "+v"(hi));  // keep the masks: byte b converts with v_cvt_f32_ubyte<b>
        // d0*q is exact (an 11-bit f16 significand times a 6-bit scale times a
        // 4-bit quant), so the fused multiply-add rounds exactly once, as
        // the multiply and the subtraction do
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            u.lo[4 * i + b] = __builtin_fmaf(d0, (float)((lo >> (8 * b)) & 0xFFu), -o0);
            u.hi[4 * i + b] = __builtin_fmaf(d1, (float)((hi >> (8 * b)) & 0xFFu), -o1);
        }
    }
}

// One run of q4k_decode_unit: u.lo (kHi false) or u.hi (kHi true) alone,
// the same values (for callers that encode a run as soon as it is decoded).
template <bool kHi>
__device__ __forceinline__ void q4k_decode_run(uint4 head, uint4 qs, int s, float (&v)[16]) {
    const float d = half_bits_to_float(head.x & 0xFFFFu);
    const float dmin = half_bits_to_float(head.x >> 16);
    uint32_t sc, mn;
    q4k_scale_min(head, 2 * (s >> 1) + (kHi ? 1 : 0), sc, mn);
    const float d0 = d * (float)sc, o0 = dmin * (float)mn;
    const uint32_t w[4] = {qs.x, qs.y, qs.z, qs.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t x = kHi ? (w[i] >> 4) & 0x0F0F0F0Fu : w[i] & 0x0F0F0F0Fu;
        asm("" : "+v"(x));  // byte b converts with v_cvt_f32_ubyte<b>
#pragma unroll
        for (int b = 0; b < 4; ++b) v[4 * i + b] = __builtin_fmaf(d0, (float)((x >> (8 * b)) & 0xFFu), -o0);
    }
}

// Running per-byte maximum and minimum of the four bytes of w (each < 256)
// with packed 16-bit integer max/min: bytes 0 and 2 go to the two 16-bit
// halves of one operand, bytes 1 and 3 to the other.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void byte_minmax(uint32_t w, u16x2& mx, u16x2& mn) {
    const u16x2 e = __builtin_bit_cast(u16x2, w & 0x00FF00FFu);
    const u16x2 o = __builtin_bit_cast(u16x2, (w >> 8) & 0x00FF00FFu);
    mx = __builtin_elementwise_max(mx, __builtin_elementwise_max(e, o));
    mn = __builtin_elementwise_min(mn, __builtin_elementwise_min(e, o));
}
__device__ __forceinline__ uint32_t u16x2_max(u16x2 v) { return v.x > v.y ? v.x : v.y; }
__device__ __forceinline__ uint32_t u16x2_min(u16x2 v) { return v.x < v.y ? v.x : v.y; }

// max abs_key over the 32 decoded values of a unit, without decoding them:
// d*sc*q is exact, so q -> RN(d*sc*q - dmin*m) is monotone in q and |value|
// peaks at the smallest or the largest nibble of each half (NaN products
// only occur where every value of the half is NaN or at q = 0 next to Inf
// values, so the endpoint keys still give the maximum).
__device__ __forceinline__ uint32_t q4k_unit_key(uint4 head, uint4 qs, int s) {
    const float d = half_bits_to_float(head.x & 0xFFFFu);
    const float dmin = half_bits_to_float(head.x >> 16);
    const int c = s >> 1;
    uint32_t sc0, m0, sc1, m1;
    q4k_scale_min(head, 2 * c, sc0, m0);
    q4k_scale_min(head, 2 * c + 1, sc1, m1);
    const float d0 = d * (float)sc0, o0 = dmin * (float)m0;
    const float d1 = d * (float)sc1, o1 = dmin * (float)m1;
    const uint32_t w[4] = {qs.x, qs.y, qs.z, qs.w};
    u16x2 lmx = {0, 0}, lmn = {15, 15}, hmx = {0, 0}, hmn = {15, 15};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
        byte_minmax(lo, lmx, lmn);
        byte_minmax(hi, hmx, hmn);
    }
    const float lmax = (float)u16x2_max(lmx), lmin = (float)u16x2_min(lmn);
    const float hmax = (float)u16x2_max(hmx), hmin = (float)u16x2_min(hmn);
    const uint32_t k0 = abs_key(d0 * lmax - o0), k1 = abs_key(d0 * lmin - o0);
    const uint32_t k2 = abs_key(d1 * hmax - o1), k3 = abs_key(d1 * hmin - o1);
    const uint32_t a = k0 > k1 ? k0 : k1, b = k2 > k3 ? k2 : k3;
    return a > b ? a : b;
}

// Q6_K: one unit is (half h, l0 in {0,16}) of a super-block: 64 weights, four
// runs of 16 at elements 128h + 32p + l0 (p = 0..3).  ql_a = ql[64h+l0..+16],
// ql_b = ql[64h+32+l0..+16], qh = qh[32h+l0..+16], sc4 = the four int8 scales
// scales[8h + l0/16 + 2p] packed in one word (byte p), d = f16 bits.
// value = (d*sc)*(q-32) is exact in fp32 (at most 24 significant bits).
struct Q6Unit {
    float v[4][16];
};

// kFinite: the caller knows d is finite, so ds*(q-32), which is exact, can
// be computed as ds*q - 32*ds in one fused multiply-add (with an infinite d
// that form would give NaN where the product gives an infinity).
template <bool kFinite = false>
__device__ __forceinline__ void q6k_decode_unit(uint4 ql_a, uint4 ql_b, uint4 qh, uint32_t sc4,
                                                uint32_t dbits, Q6Unit& u) {
    const float d = half_bits_to_float(dbits);
    float ds[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) ds[p] = d * (float)(int8_t)((sc4 >> (8 * p)) & 0xFFu);
    const uint32_t A[4] = {ql_a.x, ql_a.y, ql_a.z, ql_a.w};
    const uint32_t B[4] = {ql_b.x, ql_b.y, ql_b.z, ql_b.w};
    const uint32_t H[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // the 6-bit quants of bytes 4i..4i+3, one per byte lane
        uint32_t q[4];
        q[0] = (A[i] & 0x0F0F0F0Fu) | ((H[i] & 0x03030303u) << 4);
        q[1] = (B[i] & 0x0F0F0F0Fu) | (((H[i] >> 2) & 0x03030303u) << 4);
        q[2] = ((A[i] >> 4) & 0x0F0F0F0Fu) | (((H[i] >> 4) & 0x03030303u) << 4);
        q[3] = ((B[i] >> 4) & 0x0F0F0F0Fu) | (((H[i] >> 6) & 0x03030303u) << 4);
        asm("" : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]));
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float qf = (float)((q[p] >> (8 * b)) & 0xFFu);
                u.v[p][4 * i + b] = kFinite ? __builtin_fmaf(ds[p], qf, -32.0f * ds[p]) : ds[p] * (qf - 32.0f);
            }
    }
}

// Run p of q6k_decode_unit alone (u.v[p]), the same values.
template <bool kFinite = false>
__device__ __forceinline__ void q6k_decode_run(uint4 ql_a, uint4 ql_b, uint4 qh, uint32_t sc4, uint32_t dbits, int p,
                                               float (&v)[16]) {
    const float d = half_bits_to_float(dbits);
    const float ds = d * (float)(int8_t)((sc4 >> (8 * p)) & 0xFFu);
    const uint32_t A[4] = {ql_a.x, ql_a.y, ql_a.z, ql_a.w};
    const uint32_t B[4] = {ql_b.x, ql_b.y, ql_b.z, ql_b.w};
    const uint32_t H[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (p & 1) ? B[i] : A[i];
        uint32_t q = ((p & 2) ? (lo >> 4) : lo) & 0x0F0F0F0Fu;
        q |= ((H[i] >> (2 * p)) & 0x03030303u) << 4;
        asm("" : "+v"(q));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float qf = (float)((q >> (8 * b)) & 0xFFu);
            v[4 * i + b] = kFinite ? __builtin_fmaf(ds, qf, -32.0f * ds) : ds * (qf - 32.0f);
        }
    }
}

// max abs_key over the 64 decoded values of a unit, from the smallest and
// largest 6-bit quant of each run of 16 (d*sc*(q-32) is exact and monotone
// in q).
__device__ __forceinline__ uint32_t q6k_unit_key(uint4 ql_a, uint4 ql_b, uint4 qh, uint32_t sc4, uint32_t dbits) {
    const float d = half_bits_to_float(dbits);
    const uint32_t A[4] = {ql_a.x, ql_a.y, ql_a.z, ql_a.w};
    const uint32_t B[4] = {ql_b.x, ql_b.y, ql_b.z, ql_b.w};
    const uint32_t H[4] = {qh.x, qh.y, qh.z, qh.w};
    u16x2 mx[4], mn[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        mx[p] = (u16x2){0, 0};
        mn[p] = (u16x2){63, 63};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        byte_minmax((A[i] & 0x0F0F0F0Fu) | ((H[i] & 0x03030303u) << 4), mx[0], mn[0]);
        byte_minmax((B[i] & 0x0F0F0F0Fu) | (((H[i] >> 2) & 0x03030303u) << 4), mx[1], mn[1]);
        byte_minmax(((A[i] >> 4) & 0x0F0F0F0Fu) | (((H[i] >> 4) & 0x03030303u) << 4), mx[2], mn[2]);
        byte_minmax(((B[i] >> 4) & 0x0F0F0F0Fu) | (((H[i] >> 6) & 0x03030303u) << 4), mx[3], mn[3]);
    }
    float qmax[4], qmin[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        qmax[p] = (float)u16x2_max(mx[p]);
        qmin[p] = (float)u16x2_min(mn[p]);
    }
    uint32_t key = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float ds = d * (float)(int8_t)((sc4 >> (8 * p)) & 0xFFu);
        const uint32_t k0 = abs_key(ds * (qmax[p] - 32.0f)), k1 = abs_key(ds * (qmin[p] - 32.0f));
        key = key > k0 ? key : k0;
        key = key > k1 ? key : k1;
    }
    return key;
}

// 16 bytes at a 2-byte-aligned global address p (a field of a 210-byte
// Q6_K block): one 16-byte load at p rounded down to 4 bytes plus one more
// word, recombined with byte funnel shifts.  Every byte read lies in
// [p - 2, p + 18): the caller guarantees p + 18 stays inside the buffer when
// p is not 4-byte aligned (the extra word is then needed); when p is, the
// extra word read is the load's own last word.
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

// Load the Q6_K decode unit (half h, l0 in {0, 16}) of the block at blk
// straight from global memory (see q6k_decode_unit).  The furthest byte
// read is 2 past the qh run (offset <= 194), inside the block.
__device__ __forceinline__ void q6k_load_unit(const uint8_t* blk, int h, int l0, uint4& ql_a, uint4& ql_b,
                                              uint4& qh, uint32_t& sc4, uint32_t& dbits) {
    ql_a = ld16_a2(blk + 64 * h + l0);
    ql_b = ld16_a2(blk + 64 * h + 32 + l0);
    qh = ld16_a2(blk + 128 + 32 * h + l0);
    const uint8_t* sc = blk + 192 + 8 * h + (l0 >> 4);
    sc4 = (uint32_t)sc[0] | ((uint32_t)sc[2] << 8) | ((uint32_t)sc[4] << 16) | ((uint32_t)sc[6] << 24);
    dbits = *reinterpret_cast<const uint16_t*>(blk + 208);
}

}  // namespace rz
