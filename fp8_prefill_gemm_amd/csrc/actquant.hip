// Activation quantisation and the element-wise diagnostics.
//
// Source: realizar 0.8.4 source pages cublas_prefill/gemm.rs,
// cublas_prefill_fp8_gemm (device absmax over the m*k real elements, then a
// device-scaled E4M3 conversion; no host synchronisation; M padded to 16),
// and cublas_prefill/mod.rs, ABSMAX_REDUCE_PTX, F32_TO_E4M3_DEVICE_SCALED_PTX
// and F32_TO_E4M3_SCALED_PTX.
//
// The pages reduce with a shared-memory tree and a global atomic max into a
// word that must first be zeroed by a host-to-device copy.  Here the
// reduction is atomic-free: pass 1 writes one key per workgroup (wave
// shuffles + LDS), one workgroup reduces those keys and publishes
// {absmax, absmax'/448} for the GEMM and the encode scale 448/absmax', and
// pass 2 (the encoder) reads that record (for inputs with few keys every
// encoder workgroup reduces them itself instead): no zeroing, nothing left
// over between calls.  HBM traffic: read x twice (4 + 4 bytes per element) and
// write 1 byte.
#include <mutex>

#include "rz_device.h"
#include "rz_internal.h"

// Scratch of rz_fp8_quant_act_noalloc: the partial absmax keys of one
// activation quantisation (at most kMaxPartials of them), then the scale
// record.  One copy per GPU, held until the process ends; host code reaches
// it only through the address hipGetSymbolAddress returns for the current
// device (quant_scratch_ptr), never through this name.
static __device__ __align__(256) uint32_t scratch[rz::kQuantScratchBytes / 4];

namespace rz {
namespace {

constexpr int kThreads = 256;

// Pass 1 over fp32 data: per-workgroup max key.  x is 16-byte aligned.
// Each workgroup iteration covers kU*kThreads consecutive float4 (thread t
// reads t, t + kThreads, ...), all issued before any is used, so every thread
// keeps kU loads in flight.  The last count % 4 elements are read one at a
// time by workgroup 0.
constexpr int kU = 8;
__global__ __launch_bounds__(kThreads) void absmax_partial_kernel(const float* __restrict__ x,
                                                                  uint64_t count,
                                                                  uint32_t* __restrict__ partial) {
    __shared__ uint32_t red[kThreads / kWave];
    const float4* x4 = reinterpret_cast<const float4*>(x);
    const uint64_t n4 = count >> 2;
    const uint64_t step = (uint64_t)gridDim.x * kThreads * kU;
    uint32_t k = 0;
    for (uint64_t i0 = (uint64_t)blockIdx.x * kThreads * kU + threadIdx.x; i0 < n4; i0 += step) {
        float4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint64_t i = i0 + (uint64_t)u * kThreads;
            v[u] = i < n4 ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            uint32_t t;
            t = abs_key(v[u].x); k = k > t ? k : t;
            t = abs_key(v[u].y); k = k > t ? k : t;
            t = abs_key(v[u].z); k = k > t ? k : t;
            t = abs_key(v[u].w); k = k > t ? k : t;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (count & 3)) {
        const uint32_t t = abs_key(x[(n4 << 2) + threadIdx.x]);
        k = k > t ? k : t;
    }
    const uint32_t key = block_max_u32<kThreads>(k, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = key;
}

// One workgroup: reduces the npartial keys and publishes {a, dq} to
// act_scale and {a, q, dq, 0} to rec for the encode pass.
__global__ __launch_bounds__(kThreads) void act_scales_kernel(const uint32_t* __restrict__ partial, int npartial,
                                                              float* __restrict__ act_scale, float* __restrict__ rec) {
    __shared__ uint32_t red[kThreads / kWave];
    const Scales sc = scales_from_key(reduce_partials<kThreads>(partial, npartial, red));
    if (threadIdx.x == 0) {
        rec[0] = sc.a;
        rec[1] = sc.q;
        rec[2] = sc.dq;
        rec[3] = 0.0f;
        act_scale[0] = sc.a;
        act_scale[1] = sc.dq;
    }
}

// Pass 2 of the activation path.  count_real = m*k (a multiple of 256),
// count_total = pad_m(m)*k; groups of 16 elements at or past count_real are
// pad rows and are written as zero bytes.
__device__ __forceinline__ void act_encode_body(const float* __restrict__ x, uint64_t count_real,
                                                uint64_t count_total, float q, uint8_t* __restrict__ out) {
    const uint64_t groups = count_total >> 4;
    const uint64_t real_groups = count_real >> 4;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    uint4* o16 = reinterpret_cast<uint4*>(out);
    for (uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x; g < groups; g += stride) {
        if (g < real_groups) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 a = x4[4 * g + j];
                v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
            }
            o16[g] = e4m3_scaled16(v, q);
        } else {
            o16[g] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
}

// rec: the {a, q, dq, 0} act_scales_kernel published.
__global__ __launch_bounds__(kThreads) void act_encode_kernel(
    const float* __restrict__ x, uint64_t count_real, uint64_t count_total,
    const float* __restrict__ rec, uint8_t* __restrict__ out) {
    act_encode_body(x, count_real, count_total, rec[1], out);
}

// The same pass for an input with at most kFusedPartials partial keys (up to
// 32 MB of fp32): every workgroup reduces the keys itself (4 KB at most, one
// load per thread, read from the L2 by all but the first workgroups) and
// workgroup 0 publishes {a, dq} to act_scale, in place of act_scales_kernel:
// one launch less for the same values.
constexpr int kFusedPartials = 1024;
__global__ __launch_bounds__(kThreads) void act_encode_reduce_kernel(
    const float* __restrict__ x, uint64_t count_real, uint64_t count_total, const uint32_t* __restrict__ partial,
    int npartial, float* __restrict__ act_scale, uint8_t* __restrict__ out) {
    __shared__ uint32_t red[kThreads / kWave];
    const Scales sc = scales_from_key(reduce_partials<kThreads>(partial, npartial, red));
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        act_scale[0] = sc.a;
        act_scale[1] = sc.dq;
    }
    act_encode_body(x, count_real, count_total, sc.q, out);
}

// fp32 -> fp16 (to nearest even) of the activation for the FP16 comparator
// path (gemm.rs page, cublas_prefill_hgemm; mod.rs page, F32_TO_F16_PTX):
// 8 elements per thread and iteration; groups at or past count_real (a
// multiple of 256) are the pad rows and are written as zeros.
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, (h2v){(_Float16)a, (_Float16)b});
}

__global__ __launch_bounds__(kThreads) void act_to_f16_kernel(const float* __restrict__ x, uint64_t count_real,
                                                              uint64_t count_total, uint16_t* __restrict__ out) {
    const uint64_t groups = count_total >> 3, real_groups = count_real >> 3;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    uint4* o = reinterpret_cast<uint4*>(out);
    for (uint64_t g = (uint64_t)blockIdx.x * kThreads + threadIdx.x; g < groups; g += stride) {
        if (g < real_groups) {
            const float4 a = x4[2 * g], b = x4[2 * g + 1];
            o[g] = make_uint4(f16x2(a.x, a.y), f16x2(a.z, a.w), f16x2(b.x, b.y), f16x2(b.z, b.w));
        } else {
            o[g] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
}

// Final reduction for the absmax diagnostic: one workgroup.
__global__ __launch_bounds__(kThreads) void absmax_final_kernel(const uint32_t* __restrict__ partial,
                                                                int npartial, float* __restrict__ out) {
    __shared__ uint32_t red[kThreads / kWave];
    const uint32_t key = reduce_partials<kThreads>(partial, npartial, red);
    if (threadIdx.x == 0) out[0] = __uint_as_float(key);
}

// Host-scaled encode of `count` elements (16 per thread; scalar tail).
__global__ __launch_bounds__(kThreads) void encode_kernel(const float* __restrict__ x, uint64_t count,
                                                          float q, uint8_t* __restrict__ out) {
    const uint64_t groups = count >> 4;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    const uint64_t tid = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    const float4* x4 = reinterpret_cast<const float4*>(x);
    for (uint64_t g = tid; g < groups; g += stride) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 a = x4[4 * g + j];
            v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
        }
        reinterpret_cast<uint4*>(out)[g] = e4m3_scaled16(v, q);
    }
    const uint64_t tail = count & 15;
    if (tid < tail) {
        const uint64_t i = (groups << 4) + tid;
        out[i] = (uint8_t)e4m3_scaled(x[i], q);
    }
}

__global__ __launch_bounds__(kThreads) void scales_kernel(const float* __restrict__ a, uint64_t count,
                                                          float* __restrict__ q,
                                                          float* __restrict__ dq) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += stride) {
        const float v = a[i];
        const float ap = (v == 0.0f) ? 1.0f : v;
        q[i] = kFp8Max / ap;
        dq[i] = ap / kFp8Max;
    }
}

int grid_for(uint64_t work_items, int cap) {
    uint64_t g = (work_items + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    return (int)(g > (uint64_t)cap ? (uint64_t)cap : g);
}

// Partial workgroups for an absmax over `count` floats: at least one
// iteration of kU float4 per thread, at most kMaxPartials.
int absmax_groups(uint64_t count) { return grid_for(((count >> 2) + kU - 1) / kU, kMaxPartials); }

}  // namespace

hipError_t launch_quant_act(const float* x, uint64_t count_real, uint64_t count_total,
                            uint8_t* a_fp8, float* act_scale, uint32_t* partial, uint8_t* tail, hipStream_t st) {
    const int g1 = absmax_groups(count_real);
    float* rec = reinterpret_cast<float*>(tail);
    absmax_partial_kernel<<<g1, kThreads, 0, st>>>(x, count_real, partial);
    const int g2 = grid_for(count_total >> 4, 4096);
    if (count_total && g1 <= kFusedPartials) {
        act_encode_reduce_kernel<<<g2, kThreads, 0, st>>>(x, count_real, count_total, partial, g1, act_scale, a_fp8);
        return hipGetLastError();
    }
    act_scales_kernel<<<1, kThreads, 0, st>>>(partial, g1, act_scale, rec);
    if (count_total) act_encode_kernel<<<g2, kThreads, 0, st>>>(x, count_real, count_total, rec, a_fp8);
    return hipGetLastError();
}

int quant_act_partials(uint64_t count_real) { return absmax_groups(count_real); }

hipError_t quant_scratch_ptr(uint8_t** ptr) {
    constexpr int kDevs = 64;
    static std::mutex mu;
    static void* addr[kDevs];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDevs) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = static_cast<uint8_t*>(addr[dev]);
    return hipSuccess;
}

hipError_t launch_fp16_convert(const float* x, uint64_t count_real, uint64_t count_total, uint16_t* out,
                               hipStream_t st) {
    act_to_f16_kernel<<<grid_for(count_total >> 3, 8192), kThreads, 0, st>>>(x, count_real, count_total, out);
    return hipGetLastError();
}

hipError_t launch_absmax(const float* x, uint64_t count, float* out, uint8_t* ws, hipStream_t st) {
    uint32_t* partial = reinterpret_cast<uint32_t*>(ws);
    const int g1 = absmax_groups(count);
    absmax_partial_kernel<<<g1, kThreads, 0, st>>>(x, count, partial);
    absmax_final_kernel<<<1, kThreads, 0, st>>>(partial, g1, out);
    return hipGetLastError();
}

hipError_t launch_encode(const float* x, uint64_t count, float scale, uint8_t* out,
                         hipStream_t st) {
    encode_kernel<<<grid_for((count >> 4) + 1, 8192), kThreads, 0, st>>>(x, count, scale, out);
    return hipGetLastError();
}

hipError_t launch_scales(const float* a, uint64_t count, float* q, float* dq, hipStream_t st) {
    scales_kernel<<<grid_for(count, 4096), kThreads, 0, st>>>(a, count, q, dq);
    return hipGetLastError();
}

}  // namespace rz
