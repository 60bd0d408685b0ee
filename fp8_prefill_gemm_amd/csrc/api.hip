// C ABI of librz_fp8 (declared in include/rz_fp8.h): argument validation,
// device check and launch sequencing.  Validation runs before any HIP call,
// so every error path can be exercised without a GPU.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <chrono>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rz_fp8.h"
#include "rz_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(RZ_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool qtype_ok(int q) { return q == RZ_Q4_K || q == RZ_Q6_K; }

// The kernels are built for gfx950 only; refuse any other device up front
// (checked once per device ordinal).
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDevices];  // 0 unknown, 1 ok, -1 unsupported
int g_dev_cus[kMaxDevices];    // compute units of each checked device

int check_device(const char* fn) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (dev < 0 || dev >= kMaxDevices) return fail(RZ_ERR_HIP, "%s: device ordinal %d out of range", fn, dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, fn);
        g_dev_state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_dev_cus[dev] = prop.multiProcessorCount;
        if (g_dev_state[dev] < 0)
            return fail(RZ_ERR_HIP, "%s: device %d is %s; this library is built for gfx950 only", fn,
                        dev, prop.gcnArchName);
    }
    if (g_dev_state[dev] < 0) return fail(RZ_ERR_HIP, "%s: device %d is not gfx950", fn, dev);
    return RZ_OK;
}

// Compute units of the current device for GEMM planning (MI355X: 256).  Used
// only to size persistent grids; falls back to 256 when no device answers.
int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (g_dev_cus[dev] > 0) return g_dev_cus[dev];
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) {
            g_dev_cus[dev] = cus;
            return cus;
        }
    }
    return 256;
}

int check_k(const char* fn, uint32_t k) {
    if (k == 0 || (k % 256u) != 0)
        return fail(RZ_ERR_SHAPE, "%s: k=%u must be a positive multiple of 256", fn, k);
    return RZ_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

size_t rz_block_bytes(int qtype) {
    return qtype == RZ_Q4_K ? 144u : qtype == RZ_Q6_K ? 210u : 0u;
}

size_t rz_weight_bytes(int qtype, uint32_t n, uint32_t k) {
    if (!qtype_ok(qtype) || k % 256u != 0) return 0;
    return (size_t)n * (k / 256u) * rz_block_bytes(qtype);
}

uint32_t rz_pad_m(uint32_t m) { return (m + 15u) & ~15u; }

size_t rz_workspace_bytes(void) { return rz::kWsBytes; }

const char* rz_status_string(int status) {
    switch (status) {
        case RZ_OK: return "ok";
        case RZ_ERR_NULL: return "null pointer";
        case RZ_ERR_QTYPE: return "unsupported weight type";
        case RZ_ERR_SHAPE: return "invalid shape";
        case RZ_ERR_ALIGN: return "misaligned pointer";
        case RZ_ERR_HIP: return "HIP error";
        case RZ_ERR_VALUE: return "invalid value";
        default: return "unknown status";
    }
}

const char* rz_last_error_string(void) { return g_last_error.c_str(); }

const char* rz_version(void) { return "rz_fp8 0.1.0 gfx950"; }

// Per-thread slot of fine-grained (coherent) pinned host memory that the
// pack's scale kernel writes the scales into, followed by the call's ticket
// (below), so the host scale needs neither a device-to-host copy nor a
// stream synchronisation.  Allocated on first use, kept until the process
// ends; null if the allocation fails (then the scales are copied back and
// the stream synchronised).  A call returns only after its kernel has
// written its ticket, the slot's last write from that kernel, so one slot
// per thread is enough.
static float* host_scale_slot() {
    thread_local float* slot = nullptr;
    thread_local bool tried = false;
    if (!tried) {
        tried = true;
        void* p = nullptr;
        if (hipHostMalloc(&p, 64, hipHostMallocCoherent | hipHostMallocPortable) == hipSuccess) {
            void* dp = nullptr;
            if (hipHostGetDevicePointer(&dp, p, 0) == hipSuccess && dp == p) slot = static_cast<float*>(p);
        }
        (void)hipGetLastError();  // a failed attempt leaves no error behind
    }
    return slot;
}

// Waits until `ticket` appears at *tag (written by the pack's scale kernel
// with release order once the scales are in the slot).  After the first
// millisecond the stream is queried once a millisecond, so a stream that
// finishes, or fails, without publishing the ticket ends the wait with an
// error instead of a hang.  Not sooner: each query costs the GPU a few
// microseconds between the kernels queued around it (measured: the gap
// between the pack and the next launch fell from 5.7 to 0 us when the
// query every 256 polls went).
static hipError_t wait_for_ticket(const uint32_t* tag, uint32_t ticket, hipStream_t st) {
    using clock = std::chrono::steady_clock;
    const clock::time_point t0 = clock::now();
    clock::time_point next_query = t0 + std::chrono::milliseconds(1);
    for (uint32_t i = 1;; ++i) {
        if (__atomic_load_n(tag, __ATOMIC_ACQUIRE) == ticket) return hipSuccess;
        if ((i & 4095u) == 0 && clock::now() >= next_query) {
            const hipError_t q = hipStreamQuery(st);
            if (q == hipSuccess)
                return __atomic_load_n(tag, __ATOMIC_ACQUIRE) == ticket ? hipSuccess : hipErrorUnknown;
            if (q != hipErrorNotReady) return q;
            next_query = clock::now() + std::chrono::milliseconds(1);
        }
        __builtin_ia32_pause();
    }
}

// One weight through the pack's two passes; w_fp8 null: scales only.
// sc receives {a, q, dq}.
static int pack_one(const char* fn, int qtype, const void* blocks, uint32_t n, uint32_t k, uint8_t* w_fp8,
                    float sc[3], void* ws, void* stream) {
    if (!qtype_ok(qtype)) return fail(RZ_ERR_QTYPE, "%s: unsupported qtype %d", fn, qtype);
    if (int r = check_k(fn, k)) return r;
    if (n == 0) return fail(RZ_ERR_SHAPE, "%s: n must be positive", fn);
    if ((uint64_t)n * k > RZ_MAX_ELEMS) return fail(RZ_ERR_SHAPE, "%s: n*k too large", fn);
    if (!aligned16(blocks) || (w_fp8 && !aligned16(w_fp8)) || !aligned16(ws))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipStream_t st = as_stream(stream);
    const uint64_t nb = (uint64_t)n * (k / 256u);
    float* slot = host_scale_slot();
    thread_local uint32_t last_ticket = 0;
    const uint32_t ticket = ++last_ticket == 0 ? ++last_ticket : last_ticket;  // never 0
    hipError_t e = rz::launch_pack(qtype, static_cast<const uint8_t*>(blocks), nb, w_fp8,
                                   static_cast<uint8_t*>(ws), slot, ticket, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (slot) {
        e = wait_for_ticket(reinterpret_cast<const uint32_t*>(slot) + 3, ticket, st);
        if (e != hipSuccess) return hip_fail(e, fn);
        const volatile float* v = slot;  // written by the device before the ticket
        for (int i = 0; i < 3; ++i) sc[i] = v[i];
    } else {  // no pinned slot: copy the scales back
        float out[4];
        e = hipMemcpyAsync(out, static_cast<uint8_t*>(ws) + rz::kWsScaleOffset, sizeof out,
                           hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, fn);
        for (int i = 0; i < 3; ++i) sc[i] = out[i];
    }
    return RZ_OK;
}

int rz_fp8_pack_weight(int qtype, const void* blocks, uint32_t n, uint32_t k, uint8_t* w_fp8,
                       float* w_scale_host, float* w_absmax_host, void* ws, void* stream) {
    static const char* fn = "rz_fp8_pack_weight";
    if (!blocks || !w_fp8 || !w_scale_host || !ws) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    float sc[3];
    if (int r = pack_one(fn, qtype, blocks, n, k, w_fp8, sc, ws, stream)) return r;
    *w_scale_host = sc[2];
    if (w_absmax_host) *w_absmax_host = sc[0];
    return RZ_OK;
}

int rz_kquant_weight_scale(int qtype, const void* blocks, uint32_t n, uint32_t k, float* w_q_host,
                           float* w_dq_host, float* w_absmax_host, void* ws, void* stream) {
    static const char* fn = "rz_kquant_weight_scale";
    if (!blocks || !w_q_host || !w_dq_host || !ws) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    float sc[3];
    if (int r = pack_one(fn, qtype, blocks, n, k, nullptr, sc, ws, stream)) return r;
    *w_q_host = sc[1];
    *w_dq_host = sc[2];
    if (w_absmax_host) *w_absmax_host = sc[0];
    return RZ_OK;
}

// Per-thread array of `count` four-float slots of coherent pinned host memory
// for rz_fp8_pack_weights (grown on demand, kept until the process ends);
// null if the allocation fails.
static float* host_scale_slots(uint32_t count) {
    thread_local float* slots = nullptr;
    thread_local uint32_t cap = 0;
    if (count > cap) {
        uint32_t want = cap ? cap : 256u;
        while (want < count) want *= 2u;
        void* p = nullptr;
        if (hipHostMalloc(&p, (size_t)want * 4 * sizeof(float), hipHostMallocCoherent | hipHostMallocPortable) !=
            hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        void* dp = nullptr;
        if (hipHostGetDevicePointer(&dp, p, 0) != hipSuccess || dp != p) {
            (void)hipGetLastError();
            (void)hipHostFree(p);
            return nullptr;
        }
        if (slots) (void)hipHostFree(slots);  // no kernel of this thread still writes the old array
        slots = static_cast<float*>(p);
        cap = want;
    }
    return slots;
}

int rz_fp8_pack_weights(uint32_t count, const int* qtypes, const void* const* blocks, const uint32_t* n,
                        const uint32_t* k, uint8_t* const* w_fp8, float* w_scale_host, float* w_absmax_host,
                        void* ws, void* stream) {
    static const char* fn = "rz_fp8_pack_weights";
    if (count == 0) return RZ_OK;
    if (!qtypes || !blocks || !n || !k || !w_fp8 || !w_scale_host || !ws)
        return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (count > (1u << 24)) return fail(RZ_ERR_SHAPE, "%s: count=%u too large", fn, count);
    for (uint32_t i = 0; i < count; ++i) {
        if (!blocks[i] || !w_fp8[i]) return fail(RZ_ERR_NULL, "%s: weight %u: null pointer", fn, i);
        if (!qtype_ok(qtypes[i])) return fail(RZ_ERR_QTYPE, "%s: weight %u: unsupported qtype %d", fn, i, qtypes[i]);
        if (k[i] == 0 || k[i] % 256u != 0)
            return fail(RZ_ERR_SHAPE, "%s: weight %u: k=%u must be a positive multiple of 256", fn, i, k[i]);
        if (n[i] == 0) return fail(RZ_ERR_SHAPE, "%s: weight %u: n must be positive", fn, i);
        if ((uint64_t)n[i] * k[i] > RZ_MAX_ELEMS) return fail(RZ_ERR_SHAPE, "%s: weight %u: n*k too large", fn, i);
        if (!aligned16(blocks[i]) || !aligned16(w_fp8[i]))
            return fail(RZ_ERR_ALIGN, "%s: weight %u: device pointers must be 16-byte aligned", fn, i);
    }
    if (!aligned16(ws)) return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    float* slots = host_scale_slots(count);
    if (!slots) {  // no pinned slots: one weight at a time, each with its own wait
        for (uint32_t i = 0; i < count; ++i) {
            const int r = rz_fp8_pack_weight(qtypes[i], blocks[i], n[i], k[i], w_fp8[i], w_scale_host + i,
                                             w_absmax_host ? w_absmax_host + i : nullptr, ws, stream);
            if (r != RZ_OK) return r;
        }
        return RZ_OK;
    }
    hipStream_t st = as_stream(stream);
    // Consecutive weights whose pass-1 workgroups fit the workspace's partial
    // keys together (up to 8 weights) share one launch per pass: a whole
    // layer of the 7B-class model, so the kernels' latencies and tails overlap.
    thread_local uint32_t last_ticket = 0x80000000u;  // apart from rz_fp8_pack_weight's tickets
    std::vector<uint32_t> tickets(count);
    for (uint32_t i = 0; i < count;) {
        int qt[rz::kMaxPackSet];
        const uint8_t* bl[rz::kMaxPackSet];
        uint64_t nbv[rz::kMaxPackSet];
        uint8_t* wo[rz::kMaxPackSet];
        float* hs[rz::kMaxPackSet];
        uint32_t tk[rz::kMaxPackSet];
        int cnt = 0, groups = 0;
        while (i + cnt < count && cnt < rz::kMaxPackSet) {
            const uint32_t j = i + (uint32_t)cnt;
            const uint64_t nbj = (uint64_t)n[j] * (k[j] / 256u);
            const int gj = rz::pack_absmax_groups(qtypes[j], nbj);
            if (cnt > 0 && groups + gj > rz::kWsPartials) break;
            groups += gj;
            tickets[j] = ++last_ticket == 0 ? ++last_ticket : last_ticket;  // never 0
            reinterpret_cast<volatile uint32_t*>(slots + 4 * j)[3] = 0;        // not yet this call's ticket
            qt[cnt] = qtypes[j];
            bl[cnt] = static_cast<const uint8_t*>(blocks[j]);
            nbv[cnt] = nbj;
            wo[cnt] = w_fp8[j];
            hs[cnt] = slots + 4 * j;
            tk[cnt] = tickets[j];
            ++cnt;
        }
        const hipError_t e = rz::launch_pack_set(cnt, qt, bl, nbv, wo, static_cast<uint8_t*>(ws), hs, tk, st);
        if (e != hipSuccess) {
            // the weights before i are enqueued: wait for their scales so that no
            // kernel still writes the slots, then report the failure
            for (uint32_t j = 0; j < i; ++j)
                (void)wait_for_ticket(reinterpret_cast<const uint32_t*>(slots + 4 * j) + 3, tickets[j], st);
            return hip_fail(e, fn);
        }
        i += (uint32_t)cnt;
    }
    for (uint32_t i = 0; i < count; ++i) {
        const hipError_t e = wait_for_ticket(reinterpret_cast<const uint32_t*>(slots + 4 * i) + 3, tickets[i], st);
        if (e != hipSuccess) return hip_fail(e, fn);
        const volatile float* v = slots + 4 * i;  // written by the device before the ticket
        w_scale_host[i] = v[2];
        if (w_absmax_host) w_absmax_host[i] = v[0];
    }
    return RZ_OK;
}

int rz_fp8_quant_act(const float* x, uint32_t m, uint32_t k, uint8_t* a_fp8, float* act_scale_dev,
                     void* ws, void* stream) {
    static const char* fn = "rz_fp8_quant_act";
    // x and a_fp8 may be NULL when m == 0 (nothing is read or written there)
    if ((m != 0 && (!x || !a_fp8)) || !act_scale_dev || !ws)
        return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (int r = check_k(fn, k)) return r;
    if ((uint64_t)rz_pad_m(m) * k > RZ_MAX_ELEMS || m > 0xFFFFFFF0u)
        return fail(RZ_ERR_SHAPE, "%s: m*k too large", fn);
    if ((m != 0 && (!aligned16(x) || !aligned16(a_fp8))) || !aligned16(ws) ||
        ((uintptr_t)act_scale_dev & 3u))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    uint8_t* w = static_cast<uint8_t*>(ws);
    hipError_t e = rz::launch_quant_act(x, (uint64_t)m * k, (uint64_t)rz_pad_m(m) * k, a_fp8, act_scale_dev,
                                        reinterpret_cast<uint32_t*>(w), w + rz::kWsQuantOffset, as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

static_assert(rz::kQuantScratchBytes == RZ_QUANT_SCRATCH_BYTES, "scratch size in the header");

int rz_fp8_quant_act_noalloc(const float* x, uint32_t m, uint32_t k, uint8_t* a_fp8, float* act_scale_dev,
                             void* stream) {
    static const char* fn = "rz_fp8_quant_act_noalloc";
    if ((m != 0 && (!x || !a_fp8)) || !act_scale_dev) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (int r = check_k(fn, k)) return r;
    if ((uint64_t)rz_pad_m(m) * k > RZ_MAX_ELEMS || m > 0xFFFFFFF0u)
        return fail(RZ_ERR_SHAPE, "%s: m*k too large", fn);
    // the partial keys, then the scale record at a fixed offset
    const uint64_t need = 4 * (uint64_t)rz::quant_act_partials((uint64_t)m * k);
    if (need > 4 * (uint64_t)rz::kMaxPartials)
        return fail(RZ_ERR_SHAPE, "%s: %llu bytes of partial keys needed, %u available", fn,
                    (unsigned long long)need, (unsigned)(4 * rz::kMaxPartials));
    if ((m != 0 && (!aligned16(x) || !aligned16(a_fp8))) || ((uintptr_t)act_scale_dev & 3u))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    uint8_t* scratch = nullptr;
    hipError_t e = rz::quant_scratch_ptr(&scratch);
    if (e != hipSuccess) return hip_fail(e, fn);
    e = rz::launch_quant_act(x, (uint64_t)m * k, (uint64_t)rz_pad_m(m) * k, a_fp8, act_scale_dev,
                             reinterpret_cast<uint32_t*>(scratch), scratch + 4 * (size_t)rz::kMaxPartials,
                             as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_fp8_gemm(const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n, uint32_t k,
                const float* act_scale_dev, float w_scale, float* y, void* ws, size_t ws_bytes,
                void* stream) {
    static const char* fn = "rz_fp8_gemm";
    if (int r = check_k(fn, k)) return r;
    if (k > RZ_MAX_GEMM_K) return fail(RZ_ERR_SHAPE, "%s: k=%u exceeds %u", fn, k, (unsigned)RZ_MAX_GEMM_K);
    if (m == 0 || n == 0) return RZ_OK;  // empty product: nothing to read or write
    if (!a_fp8 || !w_fp8 || !act_scale_dev || !y) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if ((uint64_t)n * k > RZ_MAX_ELEMS || (uint64_t)rz_pad_m(m) * k > RZ_MAX_ELEMS ||
        (uint64_t)m * n > RZ_MAX_ELEMS || m > 0x7FFFFFF0u || n > 0x7FFFFFF0u)
        return fail(RZ_ERR_SHAPE, "%s: operand too large", fn);
    if (!aligned16(a_fp8) || !aligned16(w_fp8) || !aligned16(y) || ((uintptr_t)act_scale_dev & 3u) ||
        (ws && !aligned16(ws)))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (w_scale != w_scale || w_scale - w_scale != 0.0f)
        return fail(RZ_ERR_VALUE, "%s: w_scale must be finite", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_gemm(a_fp8, w_fp8, m, n, k, act_scale_dev, w_scale, y, ws, ws ? ws_bytes : 0,
                                   device_cus(), as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_fp8_gemm_group(const uint8_t* a_fp8, uint32_t m, uint32_t k, const float* act_scale_dev, uint32_t count,
                      const uint8_t* const* w_fp8, const uint32_t* n, const float* w_scale, float* const* y,
                      void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "rz_fp8_gemm_group";
    if (int r = check_k(fn, k)) return r;
    if (k > RZ_MAX_GEMM_K) return fail(RZ_ERR_SHAPE, "%s: k=%u exceeds %u", fn, k, (unsigned)RZ_MAX_GEMM_K);
    if (count > RZ_GEMM_GROUP_MAX) return fail(RZ_ERR_SHAPE, "%s: count=%u exceeds %u", fn, count, (unsigned)RZ_GEMM_GROUP_MAX);
    if (count == 0 || m == 0) return RZ_OK;  // nothing to read or write
    if (!w_fp8 || !n || !w_scale || !y) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (!a_fp8 || !act_scale_dev) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if ((uint64_t)rz_pad_m(m) * k > RZ_MAX_ELEMS || m > 0x7FFFFFF0u) return fail(RZ_ERR_SHAPE, "%s: operand too large", fn);
    if (!aligned16(a_fp8) || ((uintptr_t)act_scale_dev & 3u) || (ws && !aligned16(ws)))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    uint64_t ntot = 0;
    bool whole = true;  // every width a multiple of 256: the GEMMs can share one launch
    for (uint32_t i = 0; i < count; ++i) {
        if (n[i] == 0) continue;
        if (!w_fp8[i] || !y[i]) return fail(RZ_ERR_NULL, "%s: gemm %u: null pointer", fn, i);
        if ((uint64_t)n[i] * k > RZ_MAX_ELEMS || (uint64_t)m * n[i] > RZ_MAX_ELEMS || n[i] > 0x7FFFFFF0u)
            return fail(RZ_ERR_SHAPE, "%s: gemm %u: operand too large", fn, i);
        if (!aligned16(w_fp8[i]) || !aligned16(y[i]))
            return fail(RZ_ERR_ALIGN, "%s: gemm %u: device pointers must be 16-byte aligned", fn, i);
        if (w_scale[i] != w_scale[i] || w_scale[i] - w_scale[i] != 0.0f)
            return fail(RZ_ERR_VALUE, "%s: gemm %u: w_scale must be finite", fn, i);
        whole = whole && n[i] % 256u == 0;
        ntot += n[i];
    }
    if (ntot == 0) return RZ_OK;
    if (int r = check_device(fn)) return r;
    hipStream_t st = as_stream(stream);
    const int cus = device_cus();
    if (whole && ntot < (1u << 21)) {
        const rz::GemmPlan p = rz::plan_gemm(m, (uint32_t)ntot, k, cus, true);
        if (p.kind == rz::kGemmTiles) {  // one launch over the concatenated widths
            rz::GemmGroups G = {};
            int end = 0;
            for (uint32_t i = 0; i < count; ++i) {
                if (n[i] == 0) continue;
                end += (int)n[i];
                G.n_end[G.count] = end;
                G.w[G.count] = w_fp8[i];
                G.y[G.count] = y[i];
                G.w_scale[G.count] = w_scale[i];
                ++G.count;
            }
            const hipError_t e = rz::launch_interior(p, a_fp8, G, m, (uint32_t)ntot, k, act_scale_dev, st, false);
            return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
        }
    }
    for (uint32_t i = 0; i < count; ++i) {  // one launch per GEMM, in order on the stream
        if (n[i] == 0) continue;
        const hipError_t e = rz::launch_gemm(a_fp8, w_fp8[i], m, n[i], k, act_scale_dev, w_scale[i], y[i], ws,
                                             ws ? ws_bytes : 0, cus, st);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    return RZ_OK;
}

int rz_fp16_pack_weight(int qtype, const void* blocks, uint32_t n, uint32_t k, uint16_t* w_f16, void* stream) {
    static const char* fn = "rz_fp16_pack_weight";
    if (!blocks || !w_f16) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (!qtype_ok(qtype)) return fail(RZ_ERR_QTYPE, "%s: unsupported qtype %d", fn, qtype);
    if (int r = check_k(fn, k)) return r;
    if (n == 0) return fail(RZ_ERR_SHAPE, "%s: n must be positive", fn);
    if ((uint64_t)n * k > RZ_MAX_ELEMS) return fail(RZ_ERR_SHAPE, "%s: n*k too large", fn);
    if (!aligned16(blocks) || !aligned16(w_f16))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_fp16_pack(qtype, static_cast<const uint8_t*>(blocks), (uint64_t)n * (k / 256u), w_f16,
                                        as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_fp16_convert_act(const float* x, uint32_t m, uint32_t k, uint16_t* a_f16, void* stream) {
    static const char* fn = "rz_fp16_convert_act";
    if (int r = check_k(fn, k)) return r;
    if (m == 0) return RZ_OK;  // nothing to read or write
    if (!x || !a_f16) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if ((uint64_t)rz_pad_m(m) * k > RZ_MAX_ELEMS || m > 0xFFFFFFF0u) return fail(RZ_ERR_SHAPE, "%s: m*k too large", fn);
    if (!aligned16(x) || !aligned16(a_f16))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_fp16_convert(x, (uint64_t)m * k, (uint64_t)rz_pad_m(m) * k, a_f16, as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_fp16_gemm(const uint16_t* a_f16, const uint16_t* w_f16, uint32_t m, uint32_t n, uint32_t k, float* y,
                 void* stream) {
    static const char* fn = "rz_fp16_gemm";
    if (int r = check_k(fn, k)) return r;
    if (k > RZ_MAX_GEMM_K / 2) return fail(RZ_ERR_SHAPE, "%s: k=%u exceeds %u", fn, k, (unsigned)(RZ_MAX_GEMM_K / 2));
    if (m == 0 || n == 0) return RZ_OK;  // empty product: nothing to read or write
    if (!a_f16 || !w_f16 || !y) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if ((uint64_t)n * k > RZ_MAX_ELEMS || (uint64_t)rz_pad_m(m) * k > RZ_MAX_ELEMS || (uint64_t)m * n > RZ_MAX_ELEMS ||
        m > 0x7FFFFFF0u || n > 0x7FFFFFF0u)
        return fail(RZ_ERR_SHAPE, "%s: operand too large", fn);
    if (!aligned16(a_f16) || !aligned16(w_f16) || !aligned16(y))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_fp16_gemm(a_f16, w_f16, m, n, k, y, device_cus(), as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

size_t rz_q8_1_bytes(uint32_t m, uint32_t k) {
    if (k == 0 || k % 256u != 0) return 0;
    return (size_t)m * (k / 32u) * 36u;
}

int rz_q8_1_quant(const float* x, uint32_t m, uint32_t k, uint8_t* q8, void* stream) {
    static const char* fn = "rz_q8_1_quant";
    if (int r = check_k(fn, k)) return r;
    if (m == 0) return RZ_OK;  // nothing to read or write
    if (!x || !q8) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if ((uint64_t)m * k > RZ_MAX_ELEMS) return fail(RZ_ERR_SHAPE, "%s: m*k too large", fn);
    if (!aligned16(x) || !aligned16(q8)) return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_q8_1_quant(x, (uint64_t)m * k, q8, as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_q8_q4k_gemm(const uint8_t* q8, uint32_t m, const void* blocks, uint32_t n, uint32_t k, float* y,
                   void* stream) {
    static const char* fn = "rz_q8_q4k_gemm";
    if (int r = check_k(fn, k)) return r;
    if (m == 0 || n == 0) return RZ_OK;  // empty product: nothing to read or write
    if (!q8 || !blocks || !y) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    // the kernel addresses every operand and the output with 32-bit byte offsets
    const uint64_t lim = 0xFFFFFF00ull;
    if ((uint64_t)m * n * 4u > lim || (uint64_t)n * (k / 256u) * 144u > lim || (uint64_t)m * (k / 32u) * 36u > lim)
        return fail(RZ_ERR_SHAPE, "%s: operand or output beyond 4 GB", fn);
    if (!aligned16(q8) || !aligned16(blocks) || !aligned16(y))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_q8_q4k_gemm(q8, m, static_cast<const uint8_t*>(blocks), n, k, y, as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_route_kquant_gemv(uint32_t m) { return m >= 1u && m <= RZ_KGEMV_ROUTE_MAX_M ? 1 : 0; }

int rz_kquant_fp8_gemm(const uint8_t* a_fp8, uint32_t m, const float* act_scale_dev, int qtype, const void* blocks,
                       uint32_t n, uint32_t k, float w_q, float w_dq, float* y, void* stream) {
    static const char* fn = "rz_kquant_fp8_gemm";
    if (!qtype_ok(qtype)) return fail(RZ_ERR_QTYPE, "%s: unsupported qtype %d", fn, qtype);
    if (int r = check_k(fn, k)) return r;
    if (k > RZ_MAX_GEMM_K) return fail(RZ_ERR_SHAPE, "%s: k=%u exceeds %u", fn, k, (unsigned)RZ_MAX_GEMM_K);
    if (m == 0 || n == 0) return RZ_OK;  // empty product: nothing to read or write
    if (!a_fp8 || !blocks || !act_scale_dev || !y) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if ((uint64_t)n * k > RZ_MAX_ELEMS || (uint64_t)rz_pad_m(m) * k > RZ_MAX_ELEMS ||
        (uint64_t)m * n > RZ_MAX_ELEMS || m > 0x7FFFFFF0u || n > 0x7FFFFFF0u)
        return fail(RZ_ERR_SHAPE, "%s: operand too large", fn);
    if (!aligned16(a_fp8) || !aligned16(blocks) || !aligned16(y) || ((uintptr_t)act_scale_dev & 3u))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (w_q != w_q || w_q - w_q != 0.0f || w_dq != w_dq || w_dq - w_dq != 0.0f)
        return fail(RZ_ERR_VALUE, "%s: w_q and w_dq must be finite", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_kquant_fp8_gemm(a_fp8, m, act_scale_dev, qtype, static_cast<const uint8_t*>(blocks), n,
                                              k, w_q, w_dq, y, as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

size_t rz_fp8_gemm_workspace_bytes(uint32_t m, uint32_t n, uint32_t k) {
    if (k == 0 || k % 256u != 0 || m == 0 || n == 0) return 0;
    return rz::plan_gemm(m, n, k, device_cus(), true).ws_bytes;
}

int rz_fp8_gemm_plan(uint32_t m, uint32_t n, uint32_t k, int32_t* cfg_out) {
    static const char* fn = "rz_fp8_gemm_plan";
    if (!cfg_out) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (int r = check_k(fn, k)) return r;
    const rz::GemmPlan p = rz::plan_gemm(m, n, k, device_cus(), true);
    cfg_out[0] = p.bn;
    cfg_out[1] = p.bm;
    cfg_out[2] = p.threads;
    cfg_out[3] = (m == 0 || n == 0) ? 0 : p.workgroups;
    return RZ_OK;
}

int rz_kquant_gemv(int qtype, const void* blocks, uint32_t n, uint32_t k, const float* x, uint32_t m,
                   float* y, void* stream) {
    static const char* fn = "rz_kquant_gemv";
    if (!qtype_ok(qtype)) return fail(RZ_ERR_QTYPE, "%s: unsupported qtype %d", fn, qtype);
    if (int r = check_k(fn, k)) return r;
    if (m > RZ_KGEMV_MAX_M) return fail(RZ_ERR_SHAPE, "%s: m=%u exceeds %u", fn, m, (unsigned)RZ_KGEMV_MAX_M);
    if (m == 0 || n == 0) return RZ_OK;  // empty product: nothing to read or write
    if (!blocks || !x || !y) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if ((uint64_t)n * k > RZ_MAX_ELEMS || n > 0x7FFFFFF0u) return fail(RZ_ERR_SHAPE, "%s: n*k too large", fn);
    if (!aligned16(blocks) || !aligned16(x) || !aligned16(y))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_kquant_gemv(qtype, static_cast<const uint8_t*>(blocks), n, k, x, m, y,
                                          as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_dequant_f32(int qtype, const void* blocks, uint32_t n, uint32_t k, float* out_dev,
                   void* stream) {
    static const char* fn = "rz_dequant_f32";
    if (!blocks || !out_dev) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (!qtype_ok(qtype)) return fail(RZ_ERR_QTYPE, "%s: unsupported qtype %d", fn, qtype);
    if (int r = check_k(fn, k)) return r;
    if (n == 0) return fail(RZ_ERR_SHAPE, "%s: n must be positive", fn);
    if ((uint64_t)n * k > RZ_MAX_ELEMS) return fail(RZ_ERR_SHAPE, "%s: n*k too large", fn);
    if (!aligned16(blocks) || !aligned16(out_dev))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_dequant_f32(qtype, static_cast<const uint8_t*>(blocks),
                                          (uint64_t)n * (k / 256u), out_dev, as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_absmax_f32(const float* x, uint64_t count, float* out_dev, void* ws, void* stream) {
    static const char* fn = "rz_absmax_f32";
    if ((count != 0 && !x) || !out_dev || !ws) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (count > RZ_MAX_ELEMS) return fail(RZ_ERR_SHAPE, "%s: count too large", fn);
    if ((count != 0 && !aligned16(x)) || !aligned16(ws) || ((uintptr_t)out_dev & 3u))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_absmax(x, count, out_dev, static_cast<uint8_t*>(ws), as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_e4m3_encode(const float* x, uint64_t count, float scale, uint8_t* out, void* stream) {
    static const char* fn = "rz_e4m3_encode";
    if (count == 0) return RZ_OK;
    if (!x || !out) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (count > RZ_MAX_ELEMS) return fail(RZ_ERR_SHAPE, "%s: count too large", fn);
    if (!aligned16(x) || !aligned16(out))
        return fail(RZ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_encode(x, count, scale, out, as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

int rz_fp8_scales(const float* absmax_dev, uint64_t count, float* q_out_dev, float* dq_out_dev,
                  void* stream) {
    static const char* fn = "rz_fp8_scales";
    if (count == 0) return RZ_OK;
    if (!absmax_dev || !q_out_dev || !dq_out_dev) return fail(RZ_ERR_NULL, "%s: null pointer", fn);
    if (count > RZ_MAX_ELEMS) return fail(RZ_ERR_SHAPE, "%s: count too large", fn);
    if (((uintptr_t)absmax_dev | (uintptr_t)q_out_dev | (uintptr_t)dq_out_dev) & 3u)
        return fail(RZ_ERR_ALIGN, "%s: pointers must be 4-byte aligned", fn);
    if (int r = check_device(fn)) return r;
    hipError_t e = rz::launch_scales(absmax_dev, count, q_out_dev, dq_out_dev, as_stream(stream));
    return e == hipSuccess ? RZ_OK : hip_fail(e, fn);
}

}  // extern "C"
