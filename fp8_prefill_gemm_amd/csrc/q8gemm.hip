// The integer path: Q8_1 activation blocks times Q4_K weights.
//
// Source: realizar 0.8.4 source page cublas_prefill/gemm.rs,
// launch_dp4a_q4k_gemm (and the DP4A_GEMM_PREFILL branch of
// cublas_prefill_gemm): the fp32 activation is quantised to Q8_1, 36 bytes
// per 32 values (f16 d, f16 s, 32 int8 codes), then a GEMM multiplies the
// Q4_K weight blocks by the Q8_1 blocks with 8-bit integer dot products and
// writes fp32.  The pages print the launches only; the operation is the
// product of the two dequantised tensors:
//   y[m][n] = sum_k (f16(d8) * q8[m][k]) * (d*sc*q4[n][k] - dmin*mn)
//
// gfx950 design.  Within one 32-value sub-block (one Q8_1 block, one Q4_K
// sub-block) every factor but the two int8 codes is constant, so
//   y = sum_j f16(d8)[m][j] * (d*sc_j)[n] * P_j[m][n]
//     - sum_j (f16(d8)*S)[m][j] * (dmin*mn_j)[n]
// with P_j = sum q8*q4 (exact, the int8 matrix cores: one
// v_mfma_i32_32x32x32_i8 per 32x32 output block and sub-block) and
// S = sum q8.  The first sum needs a per-element rescale of every
// sub-block's integer block on the vector ALU (convert, scale product,
// fused multiply-add: three operations per output and sub-block), which
// bounds this path; the second is a plain product of a [M][K/32] by a
// [K/32][N] matrix of fp32 values and runs on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32, two sub-blocks per instruction), accumulating
// into the same fp32 accumulators.
//
// Each wave computes a 64 (n) x 64 (m) output tile on its own (no LDS
// operand staging, no workgroup barrier): lane l holds output column
// n = l % 32 of each 32x32 block (the weight is the MFMA B side), so the
// weight's scale factors are per-lane scalars, decoded once per
// super-block from the lane's own block header; the activation scales of
// the 16 rows a lane holds pass through a small wave-private LDS table.
// Operand fragments come straight from global memory (L2): the weight's
// 16-byte quant slice holds one lane's 16 codes of two sub-blocks (low and
// high nibbles), the Q8_1 block one lane's 16 codes at byte 4 + 16*(l/32).
#include "rz_device.h"
#include "rz_internal.h"

namespace rz {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kQ8Block = 36;  // bytes per Q8_1 block of 32 values
constexpr int kThreads = 256;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint64_t bytes) {
    const uint32_t r = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)r, 0x00020000);
}

// ---------------------------------------------------------------- Q8_1
//
// Eight lanes per block of 32 values (four each).  d = RN(a/127) with a the
// block's max |x| (NaN ignored), id = RN(1/d) (0 when d == 0), code =
// nearest integer to RN(x*id), halves away from zero, clamped to +-127, 0
// for a NaN product; stored f16(d), f16(RN(d*sum codes)) and the codes.
__global__ __launch_bounds__(kThreads) void q8_1_quant_kernel(const float* __restrict__ x, uint64_t nblocks,
                                                              uint8_t* __restrict__ out) {
    const uint64_t stride = (uint64_t)gridDim.x * (kThreads / 8);
    const int sub = threadIdx.x & 7;
    for (uint64_t b = (uint64_t)blockIdx.x * (kThreads / 8) + (threadIdx.x >> 3); b < nblocks; b += stride) {
        const float4 v = reinterpret_cast<const float4*>(x + b * 32)[sub];
        uint32_t key = abs_key(v.x);
        key = key > abs_key(v.y) ? key : abs_key(v.y);
        key = key > abs_key(v.z) ? key : abs_key(v.z);
        key = key > abs_key(v.w) ? key : abs_key(v.w);
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
            const uint32_t t = (uint32_t)__shfl_xor((int)key, o, 8);
            key = key > t ? key : t;
        }
        const float a = __uint_as_float(key);
        const float d = a / 127.0f;  // IEEE division (the build keeps it correctly rounded)
        const float id = d != 0.0f ? 1.0f / d : 0.0f;
        const float xs[4] = {v.x, v.y, v.z, v.w};
        int q[4];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = xs[i] * id;
            const float r = __builtin_roundf(p);  // halves away from zero
            const float c = __builtin_amdgcn_fmed3f(r, -127.0f, 127.0f);
            q[i] = p == p ? (int)c : 0;
            sum += q[i];
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) sum += __shfl_xor(sum, o, 8);
        uint8_t* blk = out + b * kQ8Block;
        const uint32_t codes = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) |
                               ((uint32_t)(q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24);
        reinterpret_cast<uint32_t*>(blk + 4)[sub] = codes;
        if (sub == 0) {
            float s = d * (float)sum;  // one rounded product (|sum| <= 4064 is exact)
            float dd = d;
            asm("" : "+v"(s), "+v"(dd));  // round to fp32 first, then to f16 (no fused conversion)
            const _Float16 d16 = (_Float16)dd, s16 = (_Float16)s;
            reinterpret_cast<uint32_t*>(blk)[0] =
                (uint32_t)__builtin_bit_cast(uint16_t, d16) | ((uint32_t)__builtin_bit_cast(uint16_t, s16) << 16);
        }
    }
}

// ---------------------------------------------------------------- GEMM

// The two sub-blocks 2c and 2c+1 of a Q4_K slice: low and high nibbles of
// the 16 bytes a lane holds, one int8 code per byte.
__device__ __forceinline__ v4i nibbles(v4i s, bool high) {
    v4i r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = high ? (int)(((uint32_t)s[i] >> 4) & 0x0F0F0F0Fu) : (s[i] & 0x0F0F0F0F);
    return r;
}

// sum of the 16 int8 codes a lane holds
__device__ __forceinline__ int code_sum(v4i a) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = __builtin_amdgcn_sdot4(a[i], 0x01010101, s, false);
    return s;
}

// Workgroup = 4 independent waves on a 128 (n) x 128 (m) block of the
// output (waves 2x2, 64 x 64 each), workgroups in an XCD-aware grouped order.
__global__ __launch_bounds__(kThreads, 2) void q8_q4k_gemm_kernel(const uint8_t* __restrict__ q8,
                                                                  const uint8_t* __restrict__ w,
                                                                  float* __restrict__ y, int M, int N, int K,
                                                                  int tiles_m, int tiles_n, int group_m) {
    __shared__ __attribute__((aligned(16))) float d8tab[kThreads / 64][2][32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 31, h = lane >> 5;

    // tile of this workgroup: XCD x takes a contiguous range of the grouped order
    const int T = tiles_m * tiles_n;
    const int tall = T / 8, trem = T % 8, x = blockIdx.x % 8, loc = blockIdx.x / 8;
    if (loc >= tall + (x < trem ? 1 : 0)) return;
    const int t = x * tall + (x < trem ? x : trem) + loc;
    const int per_group = group_m * tiles_n;
    const int gi = t / per_group, first_m = gi * group_m;
    const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int tin = t - gi * per_group;
    const int n0 = (tin / gm) * 128 + (wave & 1) * 64;
    const int m0 = (first_m + tin % gm) * 128 + (wave >> 1) * 64;

    const int nsb = K / 256, nb32 = K / 32;
    // rows past N / M lie outside the resources: their loads return zero
    const __amdgpu_buffer_rsrc_t wrs = rsrc(w, (uint64_t)N * nsb * kQ4Bytes);
    const __amdgpu_buffer_rsrc_t ars = rsrc(q8, (uint64_t)M * nb32 * kQ8Block);
    uint32_t wrow[2], arow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t nr = (uint32_t)(n0 + 32 * i + r), mr = (uint32_t)(m0 + 32 * i + r);
        wrow[i] = nr < (uint32_t)N ? nr * (uint32_t)nsb * kQ4Bytes : 0xFFFFFFF0u;
        arow[i] = mr < (uint32_t)M ? mr * (uint32_t)nb32 * kQ8Block : 0xFFFFFFF0u;
    }
    float* tab = d8tab[wave][0];

    v16f acc[2][2];  // [tm][tn]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (v16f){};

    // activation fragments of the current sub-block, loaded one sub-block ahead
    v4i an[2];
    uint32_t dn[2];
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
        an[tm] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, arow[tm] + 4u + 16u * h, 0, 0));
        dn[tm] = __builtin_amdgcn_raw_buffer_load_b32(ars, arow[tm], 0, 0);
    }
    for (int sb = 0; sb < nsb; ++sb) {
        // the lanes' weight rows: header and the four 16-byte quant slices of this half
        float tp[2][8], mp[2][8];
        v4i qs[2][4];
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
            const uint32_t off = wrow[tn] + (uint32_t)sb * kQ4Bytes;
            const v4i hv = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0));
#pragma unroll
            for (int c = 0; c < 4; ++c)
                qs[tn][c] = __builtin_bit_cast(
                    v4i, __builtin_amdgcn_raw_buffer_load_b128(wrs, off + 16u + 32u * c + 16u * h, 0, 0));
            const uint4 head = __builtin_bit_cast(uint4, hv);
            const float d = half_bits_to_float(head.x & 0xFFFFu), dmin = half_bits_to_float(head.x >> 16);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint32_t sc, mn;
                q4k_scale_min(head, j, sc, mn);
                tp[tn][j] = d * (float)sc;    // exact (11 x 6 bits)
                mp[tn][j] = -dmin * (float)mn;  // exact; negated for the min term
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float sig[2][2];  // [tm][sub-block of the pair]: f16(d8) * S of the lane's own row
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                const int j = 2 * c + hi;
                v4i a[2];
                float d8[2];
#pragma unroll
                for (int tm = 0; tm < 2; ++tm) {
                    a[tm] = an[tm];
                    d8[tm] = half_bits_to_float(dn[tm] & 0xFFFFu);
                }
                // the next sub-block's activation fragments (the first of the next
                // super-block after j = 7; past the end they read zero, unused)
                {
                    const uint32_t nblk = (uint32_t)(sb * 8 + j + 1) * kQ8Block;
#pragma unroll
                    for (int tm = 0; tm < 2; ++tm) {
                        an[tm] = __builtin_bit_cast(
                            v4i, __builtin_amdgcn_raw_buffer_load_b128(ars, arow[tm] + nblk + 4u + 16u * h, 0, 0));
                        dn[tm] = __builtin_amdgcn_raw_buffer_load_b32(ars, arow[tm] + nblk, 0, 0);
                    }
                }
                v4i b[2];
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) b[tn] = nibbles(qs[tn][c], hi != 0);
#pragma unroll
                for (int tm = 0; tm < 2; ++tm) {
                    // the row sum of the codes (both halves of the block) and the
                    // activation scale of each row this lane's outputs hold
                    int s = code_sum(a[tm]);
                    s += __shfl_xor(s, 32, 64);
                    sig[tm][hi] = d8[tm] * (float)s;  // exact (11 + 12 bits)
                    tab[tm * 32 + r] = d8[tm];  // both half-waves write the same value
                }
                __builtin_amdgcn_wave_barrier();
                float rs[2][16];
#pragma unroll
                for (int tm = 0; tm < 2; ++tm)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 v = *reinterpret_cast<const float4*>(tab + tm * 32 + 8 * g + 4 * h);
                        rs[tm][4 * g] = v.x;
                        rs[tm][4 * g + 1] = v.y;
                        rs[tm][4 * g + 2] = v.z;
                        rs[tm][4 * g + 3] = v.w;
                    }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int tm = 0; tm < 2; ++tm)
#pragma unroll
                    for (int tn = 0; tn < 2; ++tn) {
                        const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[tm], b[tn], (v16i){}, 0, 0, 0);
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            acc[tm][tn][e] = __builtin_fmaf((float)p[e], rs[tm][e] * tp[tn][j], acc[tm][tn][e]);
                    }
            }
            // the min term of sub-blocks 2c, 2c+1: rows supply f16(d8)*S, columns -dmin*mn
            float mpv[2], sgv[2];  // this lane's K index of the pair (h): two-way selects
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                mpv[i] = h ? mp[i][2 * c + 1] : mp[i][2 * c];
                sgv[i] = h ? sig[i][1] : sig[i][0];
            }
#pragma unroll
            for (int tm = 0; tm < 2; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(sgv[tm], mpv[tn], acc[tm][tn], 0, 0, 0);
        }
    }
    // acc[tm][tn][e]: row m0 + 32tm + 8(e/4) + 4h + e%4, column n0 + 32tn + r
    const __amdgpu_buffer_rsrc_t ys = rsrc(y, (uint64_t)M * (uint64_t)N * 4u);
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
            const uint32_t col = (uint32_t)(n0 + 32 * tn + r);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t row = (uint32_t)(m0 + 32 * tm + 8 * (e >> 2) + 4 * h + (e & 3));
                const uint32_t off = row < (uint32_t)M && col < (uint32_t)N ? (row * (uint32_t)N + col) * 4u
                                                                           : 0xFFFFFFF0u;
                // (a vector element read into a scalar first: __builtin_bit_cast of the
                // element lvalue itself reads element 0)
                const float v = acc[tm][tn][e];
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ys, off, 0, 0);
            }
        }
}

}  // namespace

hipError_t launch_q8_1_quant(const float* x, uint64_t count, uint8_t* out, hipStream_t st) {
    const uint64_t nblocks = count / 32;
    uint64_t g = (nblocks + (kThreads / 8) - 1) / (kThreads / 8);
    if (g < 1) g = 1;
    if (g > 16384) g = 16384;
    q8_1_quant_kernel<<<(int)g, kThreads, 0, st>>>(x, nblocks, out);
    return hipGetLastError();
}

hipError_t launch_q8_q4k_gemm(const uint8_t* q8, uint32_t m, const uint8_t* blocks, uint32_t n, uint32_t k,
                              float* y, hipStream_t st) {
    const int tiles_m = (int)((m + 127u) / 128u), tiles_n = (int)((n + 127u) / 128u);
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    const int T = tiles_m * tiles_n;
    const int grid = 8 * ((T + 7) / 8);
    q8_q4k_gemm_kernel<<<grid, kThreads, 0, st>>>(q8, blocks, y, (int)m, (int)n, (int)k, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

}  // namespace rz
