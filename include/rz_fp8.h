/*
 * rz_fp8 — FP8 (E4M3) prefill matmul path for GGUF K-quant weights on
 * AMD Instinct MI355X (gfx950).
 *
 * The path (realizar 0.8.4 source pages, cublas_prefill/gemm.rs and
 * cublas_prefill/mod.rs):
 *   1. once per weight: Q4_K/Q6_K super-blocks -> fp32 -> per-tensor absmax
 *      -> E4M3 bytes of RN(w * RN(448/absmax)) (absmax 0 treated as 1),
 *      kept with the host scale RN(absmax/448)       [rz_fp8_pack_weight]
 *   2. per distinct activation: device absmax and E4M3 conversion with no
 *      host synchronisation, reused by every GEMM that reads the same input
 *                                                     [rz_fp8_quant_act]
 *   3. FP8 x FP8 GEMM with fp32 accumulation and an epilogue that multiplies
 *      by (act_absmax/448) * (w_absmax/448), fp32 output  [rz_fp8_gemm]
 *
 * Conventions shared by every entry point:
 *   - Every pointer named *_dev / device is device memory owned by the
 *     caller; *_host is host memory owned by the caller.  The library keeps
 *     no persistent device allocation of its own.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is ordered on it.  No call synchronises it; only
 *     rz_fp8_pack_weight waits on the host, for its scale (below).
 *   - Arguments are validated before anything is launched.  Errors return a
 *     negative rz_status and leave outputs untouched; nothing aborts.
 *     rz_last_error_string() gives a message for the calling thread.
 *   - Device pointers to tensors and to `ws` must be 16-byte aligned; pointers
 *     to scalars (act_scale_dev, absmax/scale arrays) 4-byte aligned
 *     (RZ_ERR_ALIGN otherwise).
 *   - K (the reduction dimension) must be a positive multiple of 256, the
 *     K-quant super-block length (RZ_ERR_SHAPE otherwise).
 *   - `ws` is a caller-provided device workspace of rz_workspace_bytes()
 *     bytes (any contents: every call writes what it reads).  Calls that
 *     use the same `ws` must be ordered (same stream).
 */
#ifndef RZ_FP8_H
#define RZ_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GGML tensor type ids of the supported weight formats. */
typedef enum { RZ_Q4_K = 12, RZ_Q6_K = 14 } rz_qtype;

typedef enum {
    RZ_OK = 0,
    RZ_ERR_NULL = -1,   /* a required pointer is NULL */
    RZ_ERR_QTYPE = -2,  /* weight type other than Q4_K / Q6_K */
    RZ_ERR_SHAPE = -3,  /* k not a positive multiple of 256, n == 0, size limits */
    RZ_ERR_ALIGN = -4,  /* a device pointer is not 16-byte aligned */
    RZ_ERR_HIP = -5,    /* a HIP runtime call failed, or the device is not gfx950 */
    RZ_ERR_VALUE = -6   /* a scalar argument is not finite where it must be */
} rz_status;

/* Largest accepted n*k (weights) and m*k (activations): 2^36 elements. */
#define RZ_MAX_ELEMS ((uint64_t)1 << 36)

/* Largest K rz_fp8_gemm accepts (its tile loads use 32-bit byte offsets
 * over 256 rows of K bytes). */
#define RZ_MAX_GEMM_K ((uint32_t)(1u << 24) - 256u)

/* Bytes per super-block of 256 weights: 144 (Q4_K, 0.5625 B/weight, as the
 * gemm.rs page states) or 210 (Q6_K); 0 for any other type. */
size_t rz_block_bytes(int qtype);

/* Bytes of a [n][k] K-quant weight: n * (k/256) * rz_block_bytes(qtype);
 * 0 if the type or k is invalid. */
size_t rz_weight_bytes(int qtype, uint32_t n, uint32_t k);

/* M rounded up to a multiple of 16 — the row count of the FP8 activation
 * buffer (gemm.rs page, cublas_prefill_fp8_gemm: M is padded to 16). */
uint32_t rz_pad_m(uint32_t m);

/* Size in bytes of the device workspace `ws` (a constant, about 32 KB). */
size_t rz_workspace_bytes(void);

/*
 * Pack one K-quant weight into FP8 E4M3 (gemm.rs page,
 * get_or_cache_fp8_weight; mod.rs page, F32_TO_E4M3_SCALED_PTX and
 * ABSMAX_REDUCE_PTX).
 *
 *   blocks        device, n*(k/256) super-blocks, row-major: row r of the
 *                 weight is blocks r*(k/256) .. r*(k/256)+k/256-1
 *   w_fp8         device out, uint8 [n][k] row-major E4M3 codes of
 *                 RN(w * RN(448/a')), where a = max|w| (NaN ignored) and
 *                 a' = a, or 1 when a == 0
 *   w_scale_host  host out, RN(a'/448): the weight's dequantisation scale
 *   w_absmax_host host out (may be NULL): a
 *   ws            device workspace of rz_workspace_bytes()
 * The dequantised fp32 weight is never materialised.  Returns once the
 * scale is known on the host: the second kernel publishes it to pinned host
 * memory before it encodes, and the call waits for that, not for the codes.
 * w_fp8 is complete for later work on `stream`; other streams and the host
 * must synchronise `stream` before reading it.  If the stream ends or fails
 * without publishing the scale, the call returns RZ_ERR_HIP.
 */
int rz_fp8_pack_weight(int qtype, const void* blocks, uint32_t n, uint32_t k,
                       uint8_t* w_fp8, float* w_scale_host, float* w_absmax_host,
                       void* ws, void* stream);

/*
 * Pack `count` K-quant weights, each exactly as rz_fp8_pack_weight packs it,
 * with one host wait for all their scales instead of one per weight
 * (gemm.rs page, get_or_cache_fp8_weight, for every weight of a model: the
 * pages pack on first use, one weight at a time).
 *
 *   qtypes, blocks, n, k, w_fp8   host arrays of `count` entries: weight i
 *                 is described as the same-named arguments of
 *                 rz_fp8_pack_weight (device pointers, caller-owned)
 *   w_scale_host  host out, float[count]
 *   w_absmax_host host out, float[count] (may be NULL)
 *   ws            device workspace of rz_workspace_bytes(), reused by the
 *                 weights in stream order
 * Every entry is validated before anything is launched (the message names
 * the first bad weight).  The kernels of all weights are enqueued back to
 * back; the call returns once every scale is on the host (the codes of the
 * last weight may still be being written, ordered before later work on
 * `stream`).  count == 0 is a no-op.  Per-thread pinned host memory for the
 * scales grows to the largest count seen and is kept until the process ends.
 */
int rz_fp8_pack_weights(uint32_t count, const int* qtypes, const void* const* blocks,
                        const uint32_t* n, const uint32_t* k, uint8_t* const* w_fp8,
                        float* w_scale_host, float* w_absmax_host, void* ws, void* stream);

/*
 * Quantise an fp32 activation to FP8 on the device, with no host
 * synchronisation (gemm.rs page, cublas_prefill_fp8_gemm steps 1-2; mod.rs
 * page, F32_TO_E4M3_DEVICE_SCALED_PTX).
 *
 *   x             device, fp32 [m][k] row-major
 *   a_fp8         device out, uint8 [rz_pad_m(m)][k]: rows < m hold the E4M3
 *                 codes of RN(x * RN(448/a')), a = max|x| over the m*k real
 *                 elements (NaN ignored); rows m..rz_pad_m(m)-1 are zero
 *   act_scale_dev device out, float[2] = { a, RN(a'/448) }
 * m == 0 is allowed (writes {0, RN(1/448)} and no codes; x and a_fp8 may
 * then be NULL).  The outputs may
 * be passed to any number of rz_fp8_gemm calls that read the same input.
 */
int rz_fp8_quant_act(const float* x, uint32_t m, uint32_t k, uint8_t* a_fp8,
                     float* act_scale_dev, void* ws, void* stream);

/* Bytes of the device scratch array rz_fp8_quant_act_noalloc uses on each
 * GPU (2048 partial absmax keys and the scale record). */
#define RZ_QUANT_SCRATCH_BYTES 8224u

/*
 * rz_fp8_quant_act without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and error behaviour as rz_fp8_quant_act, minus `ws`.
 *
 * Its scratch (the partial absmax keys and the scale record) is a fixed
 * array of
 * RZ_QUANT_SCRATCH_BYTES in the library's device image, one copy per GPU,
 * held until the process ends; its address is looked up on the first call
 * on each device.  A quantisation needs at most 2048 keys whatever m*k
 * (the reduction caps its grid), so every size accepted by rz_fp8_quant_act
 * fits; a size that would need more is rejected with RZ_ERR_SHAPE.  Nothing
 * in the scratch needs to start at zero: every call writes the keys and the
 * record it reads.  All calls on one GPU share the array, so calls that overlap in
 * time on one GPU (different streams, or other host threads) race and must
 * be ordered by the caller; calls on one stream are ordered by the stream.
 * Calls no hipMalloc, hipFree or allocating library routine.
 */
int rz_fp8_quant_act_noalloc(const float* x, uint32_t m, uint32_t k, uint8_t* a_fp8,
                             float* act_scale_dev, void* stream);

/*
 * FP8 GEMM with fused dequantisation epilogue (gemm.rs page,
 * cublas_prefill_fp8_gemm steps 3-4; mod.rs page, F16_TO_F32_ACT_SCALED_PTX).
 *
 *   y[i][j] = (sum_k dec(a_fp8[i][kk]) * dec(w_fp8[j][kk]))
 *             * act_scale_dev[1] * w_scale          for i < m, j < n
 *
 *   a_fp8         device, uint8 [rz_pad_m(m)][k] from rz_fp8_quant_act
 *   w_fp8         device, uint8 [n][k] from rz_fp8_pack_weight
 *   act_scale_dev device, float[2] from rz_fp8_quant_act
 *   w_scale       the host scale from rz_fp8_pack_weight
 *   y             device out, fp32 [m][n] row-major (only rows < m written)
 *   ws, ws_bytes  optional device workspace (may be NULL / 0) of at least
 *                 rz_fp8_gemm_workspace_bytes(m, n, k) bytes, zero-filled
 *                 before its first use; every call leaves it reusable by
 *                 the next, whatever that call's shape.  It
 *                 holds partial sums and arrival counters when a shape with
 *                 few output tiles (small or medium m, narrow n) splits K
 *                 to keep the compute units busy; without it (or when it is
 *                 too small) every tile runs over the whole K.  Calls that
 *                 share a workspace must be ordered (same stream).
 * Products are accumulated in fp32 on the matrix cores (no fp16 stage); the
 * summation order may differ between calls with and without a workspace.
 * k <= RZ_MAX_GEMM_K.  m == 0 or n == 0 is a no-op (any pointer may then
 * be NULL).
 */
int rz_fp8_gemm(const uint8_t* a_fp8, const uint8_t* w_fp8, uint32_t m, uint32_t n,
                uint32_t k, const float* act_scale_dev, float w_scale, float* y,
                void* ws, size_t ws_bytes, void* stream);

/* Largest number of GEMMs one rz_fp8_gemm_group call takes. */
#define RZ_GEMM_GROUP_MAX 4u

/*
 * Several FP8 GEMMs on one quantised activation (gemm.rs page,
 * cublas_prefill_fp8_gemm: the Q/K/V projections, and the FFN gate and up
 * projections, share one activation conversion), as `count` rz_fp8_gemm
 * calls would compute them:
 *
 *   y[g][i][j] = (sum_k dec(a_fp8[i][kk]) * dec(w_fp8[g][j][kk]))
 *                * act_scale_dev[1] * w_scale[g]      for i < m, j < n[g]
 *
 *   a_fp8, m, k, act_scale_dev   the shared activation, as for rz_fp8_gemm
 *   w_fp8, n, w_scale, y         host arrays of `count` (<= RZ_GEMM_GROUP_MAX)
 *                 entries: weight g (device, uint8 [n[g]][k]), its host
 *                 scale, and its output (device, fp32 [m][n[g]]); n[g] == 0
 *                 skips that GEMM (its pointers may then be NULL)
 *   ws, ws_bytes  as for rz_fp8_gemm (used only when the GEMMs run one by one)
 * When every n[g] is a multiple of 256 and the combined width takes the
 * 256x256 interior-tile kernel, all the GEMMs run as one launch (their
 * tiles share the rounds of the compute units, so the partial last round is
 * paid once); each output element is then computed exactly as rz_fp8_gemm's
 * interior kernel computes it.  Otherwise the GEMMs run one after another
 * as rz_fp8_gemm would run them.  m == 0 or count == 0 is a no-op.
 */
int rz_fp8_gemm_group(const uint8_t* a_fp8, uint32_t m, uint32_t k, const float* act_scale_dev,
                      uint32_t count, const uint8_t* const* w_fp8, const uint32_t* n,
                      const float* w_scale, float* const* y, void* ws, size_t ws_bytes,
                      void* stream);

/* Workspace rz_fp8_gemm can use for this shape on the current device
 * (0 when it would not split). */
size_t rz_fp8_gemm_workspace_bytes(uint32_t m, uint32_t n, uint32_t k);

/* Largest batch rz_kquant_gemv accepts. */
#define RZ_KGEMV_MAX_M 8u

/*
 * Batched GEMV straight from the K-quant weight, for small batches
 * (cublas_prefill/mod.rs page, the note on cublas_gemm_threshold: below a
 * threshold of 4 rows by default the pages run GEMV kernels instead of the
 * FP8 GEMM; q6k_gemv_indexed.rs page, the q4k_gemv_into and
 * q6k_gemv_indexed_async dispatchers, fp32 in, K-quant weight, fp32 out):
 *
 *   y[i][j] = sum_kk x[i][kk] * w[j][kk]        for i < m, j < n
 *
 * where w is the weight decoded exactly as rz_dequant_f32 decodes it.  No
 * FP8 conversion and no scales are involved; nothing is packed or cached.
 *
 *   blocks  device, n*(k/256) super-blocks, row-major as for
 *           rz_fp8_pack_weight (read once, at 0.5625 / 0.8203 B per weight)
 *   x       device, fp32 [m][k] row-major
 *   y       device out, fp32 [m][n] row-major
 * 1 <= m <= RZ_KGEMV_MAX_M (RZ_ERR_SHAPE otherwise; m == 0 or n == 0 is a
 * no-op and any pointer may then be NULL).  Products are exact fp32
 * multiply-adds accumulated in fp32, so each output is within
 * gamma_k * sum_kk |x[i][kk] * w[j][kk]| of the exact sum (gamma_k =
 * k u / (1 - k u), u = 2^-24).  No workspace, no host synchronisation.
 */
int rz_kquant_gemv(int qtype, const void* blocks, uint32_t n, uint32_t k, const float* x,
                   uint32_t m, float* y, void* stream);

/* Largest batch routed to rz_kquant_gemv by rz_route_kquant_gemv. */
#define RZ_KGEMV_ROUTE_MAX_M 4u

/*
 * Batch-size routing between the two ways to multiply by a K-quant weight
 * (cublas_prefill/mod.rs page, cublas_gemm_threshold: the pages take the
 * GEMV route for fewer rows than a threshold, 4 by default):
 *   returns 1 when 1 <= m <= RZ_KGEMV_ROUTE_MAX_M (take rz_kquant_gemv),
 *   0 otherwise (take rz_fp8_quant_act + rz_fp8_gemm; m == 0 is a no-op on
 *   either route).
 * The bound comes from a measurement on MI355X and agrees with the pages'
 * 4, except that m = 4 itself takes the GEMV: at N=4608, K=3584 (Q4_K) the
 * GEMV takes 6.0 / 6.5 / 8.1 / 9.5 us at m = 1 / 2 / 3 / 4 against
 * 11.7-12.1 us for activation quantisation plus FP8 GEMM, and the FP8 route
 * wins at m = 8.  Host only; no device needed.
 */
int rz_route_kquant_gemv(uint32_t m);

/*
 * The weight's scale pair without its FP8 codes, for rz_kquant_fp8_gemm
 * (gemm.rs page, get_or_cache_fp8_weight: per-tensor absmax a of the
 * dequantised weight, a' = a or 1 when a == 0, q = RN(448/a'),
 * dq = RN(a'/448)).  One read of the blocks; nothing of size n*k is written.
 *
 *   qtype, blocks, n, k, ws, stream   as for rz_fp8_pack_weight
 *   w_q_host      host out, q (the value the weight is multiplied by before
 *                 its E4M3 encoding)
 *   w_dq_host     host out, dq (the value rz_fp8_pack_weight returns as
 *                 w_scale_host)
 *   w_absmax_host host out (may be NULL): a
 * Returns once the scales are on the host (the same pinned-memory handshake
 * and error behaviour as rz_fp8_pack_weight).
 */
int rz_kquant_weight_scale(int qtype, const void* blocks, uint32_t n, uint32_t k, float* w_q_host,
                           float* w_dq_host, float* w_absmax_host, void* ws, void* stream);

/*
 * FP8 GEMM straight from the K-quant weight (gemm.rs page,
 * cublas_prefill_fp8_gemm on the codes get_or_cache_fp8_weight would cache,
 * made here inside the GEMM so that no FP8 copy of the weight exists):
 *
 *   y[i][j] = (sum_kk dec(a_fp8[i][kk]) * dec(E4M3(RN(w[j][kk] * w_q))))
 *             * act_scale_dev[1] * w_dq                 for i < m, j < n
 *
 * where w is the weight decoded exactly as rz_dequant_f32 decodes it.  With
 * w_q, w_dq from rz_kquant_weight_scale the weight codes are the bytes
 * rz_fp8_pack_weight writes, so y equals rz_fp8_gemm on the packed weight up
 * to the order of the fp32 accumulation.
 *
 *   a_fp8, m, act_scale_dev   the activation, as for rz_fp8_gemm
 *   qtype, blocks, n, k       the weight, as for rz_fp8_pack_weight
 *   w_q, w_dq     host, finite (RZ_ERR_VALUE otherwise)
 *   y             device out, fp32 [m][n] row-major
 * k <= RZ_MAX_GEMM_K.  m == 0 or n == 0 is a no-op (any pointer may then be
 * NULL).  No workspace, no host synchronisation.
 */
int rz_kquant_fp8_gemm(const uint8_t* a_fp8, uint32_t m, const float* act_scale_dev, int qtype,
                       const void* blocks, uint32_t n, uint32_t k, float w_q, float w_dq, float* y,
                       void* stream);

/* ---------------------------------------------------------------------
 * Integer path: Q8_1 activation blocks times Q4_K weights (gemm.rs page,
 * launch_dp4a_q4k_gemm and the DP4A_GEMM_PREFILL branch of
 * cublas_prefill_gemm: the activation quantised to Q8_1, 36 bytes per 32
 * values, then an 8-bit integer GEMM against the Q4_K blocks, fp32 out).
 * --------------------------------------------------------------------- */

/* Bytes of the Q8_1 form of an [m][k] activation: m * (k/32) * 36 (0 if k
 * is not a positive multiple of 256). */
size_t rz_q8_1_bytes(uint32_t m, uint32_t k);

/*
 * Q8_1 quantisation: for every 32 consecutive values x of a row, a =
 * max |x| (NaN ignored), d = RN(a/127), id = RN(1/d) (0 when d == 0),
 * q = the nearest integer to RN(x * id), halves away from zero, clamped to
 * [-127, 127], 0 for a NaN product; the block is f16(d), f16(RN(d * sum q))
 * (both to nearest even, little-endian), then the 32 codes as int8.
 *   x   device, fp32 [m][k] row-major
 *   q8  device out, rz_q8_1_bytes(m, k) bytes: row i is blocks i*(k/32) ...
 * m == 0 is a no-op.  No workspace, no host synchronisation.
 */
int rz_q8_1_quant(const float* x, uint32_t m, uint32_t k, uint8_t* q8, void* stream);

/*
 * y[i][j] = sum_kk (f16(d)[i][kk/32] * q[i][kk]) * w[j][kk]   for i < m, j < n
 * where the first factor is the Q8_1 value and w the exact Q4_K value
 * d*sc*q4 - dmin*mn (as rz_dequant_f32 decodes it, before its fp32
 * rounding).  Integer dot products of each 32-value sub-block on the
 * matrix cores, scaled and accumulated in fp32.
 *   q8      device, Q8_1 blocks of the activation (rz_q8_1_quant)
 *   blocks  device, Q4_K weight [n][k], as for rz_fp8_pack_weight
 *   y       device out, fp32 [m][n] row-major
 * Q4_K only (the pages' integer path takes Q4_K weights).  m*n*4 bytes and
 * both operands must each stay below 4 GB (RZ_ERR_SHAPE).  m == 0 or n == 0
 * is a no-op.  No workspace, no host synchronisation.  Non-finite block
 * scales give non-finite outputs.
 */
int rz_q8_q4k_gemm(const uint8_t* q8, uint32_t m, const void* blocks, uint32_t n, uint32_t k, float* y,
                   void* stream);

/* ---------------------------------------------------------------------
 * FP16 comparator: the cached-fp16-weight GEMM the FP8 path replaced
 * (gemm.rs page, get_or_cache_fp16_weight and cublas_prefill_hgemm; mod.rs
 * page, F32_TO_F16_PTX and the module note on the tensor-core speed-up).
 * Kept to measure the FP8 path's speed and accuracy against it.
 * --------------------------------------------------------------------- */

/*
 * The fp16 weight cache: w_f16[j][kk] = fp16(w[j][kk]) with w the weight
 * decoded exactly as rz_dequant_f32 decodes it and fp16() the
 * round-to-nearest-even conversion (|w| >= 65520 gives +-Inf).
 *   blocks  device, n*(k/256) super-blocks, row-major (as rz_fp8_pack_weight)
 *   w_f16   device out, fp16 bit patterns [n][k] row-major (2 bytes each)
 * No workspace, no host synchronisation.
 */
int rz_fp16_pack_weight(int qtype, const void* blocks, uint32_t n, uint32_t k, uint16_t* w_f16,
                        void* stream);

/*
 * The fp16 activation: a_f16[i][kk] = fp16(x[i][kk]) (round to nearest even)
 * for i < m; rows m..rz_pad_m(m)-1 are zero.
 *   x       device, fp32 [m][k] row-major
 *   a_f16   device out, fp16 [rz_pad_m(m)][k] row-major
 * m == 0 is a no-op (x and a_f16 may then be NULL).
 */
int rz_fp16_convert_act(const float* x, uint32_t m, uint32_t k, uint16_t* a_f16, void* stream);

/*
 * y[i][j] = sum_kk a_f16[i][kk] * w_f16[j][kk] for i < m, j < n: fp16
 * operands, products exact, accumulated in fp32 on the matrix cores, fp32
 * output [m][n] row-major; no scale factors.
 *   a_f16   device, fp16 [rz_pad_m(m)][k] from rz_fp16_convert_act
 *   w_f16   device, fp16 [n][k] from rz_fp16_pack_weight
 * k <= RZ_MAX_GEMM_K / 2.  m == 0 or n == 0 is a no-op.  No workspace.
 */
int rz_fp16_gemm(const uint16_t* a_f16, const uint16_t* w_f16, uint32_t m, uint32_t n, uint32_t k,
                 float* y, void* stream);

/* ---------------------------------------------------------------------
 * Diagnostics: the individual steps, exposed so that each can be checked
 * against the oracle.  Same conventions as above.
 * --------------------------------------------------------------------- */

/* Dequantise a K-quant weight to fp32 [n][k] row-major (gemm.rs page,
 * launch_dequant_q4k / launch_dequant_q6k).  Each value is the correctly
 * rounded fp32 of the format's exact value. */
int rz_dequant_f32(int qtype, const void* blocks, uint32_t n, uint32_t k,
                   float* out_dev, void* stream);

/* out_dev[0] = max |x| over `count` fp32 values, NaN ignored, 0 when
 * count == 0 (x may then be NULL) (mod.rs page, ABSMAX_REDUCE_PTX). */
int rz_absmax_f32(const float* x, uint64_t count, float* out_dev, void* ws,
                  void* stream);

/* out[i] = E4M3 code of RN(x[i] * scale) for i < count (mod.rs page,
 * F32_TO_E4M3_SCALED_PTX; with scale 1 the plain F32_TO_E4M3_PTX up to the
 * sign of NaN, which the multiply makes positive).  count == 0 is a no-op. */
int rz_e4m3_encode(const float* x, uint64_t count, float scale, uint8_t* out,
                   void* stream);

/* For each of `count` absmax values a: q_out = RN(448/a'), dq_out =
 * RN(a'/448) with a' = a or 1 when a == 0 (mod.rs page,
 * F32_TO_E4M3_DEVICE_SCALED_PTX; gemm.rs page, get_or_cache_fp8_weight).
 * count == 0 is a no-op. */
int rz_fp8_scales(const float* absmax_dev, uint64_t count, float* q_out_dev,
                  float* dq_out_dev, void* stream);

/* GEMM tile configuration rz_fp8_gemm would launch for this shape (with a
 * large enough workspace): writes {BN, BM, threads, workgroups} to
 * cfg_out[4] (host); workgroups is the grid of the one launch: one per
 * compute unit for the persistent 256x256 kernel (which also runs half
 * tiles of 128 activation rows), otherwise tiles, or tiles times K chunks
 * when K is split. */
int rz_fp8_gemm_plan(uint32_t m, uint32_t n, uint32_t k, int32_t* cfg_out);

const char* rz_status_string(int status);
const char* rz_last_error_string(void);

/* Library version, e.g. "rz_fp8 0.1.0 gfx950". */
const char* rz_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RZ_FP8_H */
