/*
 * sparse_mla.h -- C ABI of the MI355X (gfx950) sparse MLA prefill forward.
 *
 * The operation is the DeepSeek-V4 sparse MLA prefill attention described on
 * "[Triton/Gluon] [GFX950][DSV4] Sparse MLA training backward" (aiter PR #4766),
 * section "Contract", whose forward is added by "[TRITON][GLUON] Add DSv4
 * sparse MLA prefill Triton and unified with MLA Gluon kernel on GFX950"
 * (aiter PR #3833):
 *
 *   for each token t and head h, over the valid slots s of row t of
 *   topk_indices (valid iff 0 <= topk_indices[t,s] < num_kv):
 *     x_s  = scale * dot(q[t,h,:], kv[topk_indices[t,s],:])        (K == V == kv)
 *     o[t,h,:] = sum_s softmax_s * kv[topk_indices[t,s],:]
 *   where the softmax denominator also holds exp(attn_sink[h]) (a logit with
 *   no value row, not multiplied by scale), and
 *     lse[t,h] = ln( sum_s exp(x_s) + exp(attn_sink[h]) )            (natural log)
 *   A (t,h) with no valid slot gets o = 0 and lse = attn_sink[h] (or -inf
 *   without a sink). attn_sink[h] == -inf is the same as no sink.
 *
 * This header is plain C: no HIP or torch types. Link against
 * libsparse_mla.so.
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Head dimension of q, kv and o. Fixed: the operation's contract fixes it at 512. */
#define SPARSE_MLA_HEAD_DIM 512

/* Status codes. Every nonzero status is returned before anything is enqueued,
 * except SMLA_ERR_LAUNCH, which reports a failed kernel launch. */
typedef enum {
  SMLA_OK = 0,
  SMLA_ERR_NULL_POINTER = -1, /* a buffer with nonzero size is NULL                       */
  SMLA_ERR_BAD_SIZE = -2,     /* T < 0, H < 1, num_kv < 0, topk < 0, or a size overflows   */
  SMLA_ERR_MISALIGNED = -3,   /* q, kv or out not 16-byte aligned; lse, sink, int32 topk
                                 not 4; int64 topk not 8                                   */
  SMLA_ERR_BAD_SCALE = -4,    /* scale is NaN or infinite                                  */
  SMLA_ERR_NO_DEVICE = -5,    /* no usable HIP device is current                           */
  SMLA_ERR_LAUNCH = -6,       /* the kernel launch failed (hipGetLastError)                */
  SMLA_ERR_NO_MEMORY = -7,    /* device scratch could not be had (int64 rows, backward, or
                                 the no-allocation entry point's array)                    */
  SMLA_ERR_SCRATCH_LIMIT = -8 /* sparse_mla_prefill_noalloc: the call's split partials do not
                                 fit SPARSE_MLA_NOALLOC_SCRATCH_BYTES                      */
} smla_status_t;

/* Size of the device array that sparse_mla_prefill_noalloc keeps its split
 * partials in (64 MiB per device that calls it). */
#define SPARSE_MLA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * sparse_mla_prefill -- enqueue the forward on `stream` and return.
 *
 * Arguments (all device pointers on the current HIP device, caller-owned):
 *   q             bf16 [T, H, 512], contiguous, 16-byte aligned.
 *   kv            bf16 [num_kv, 512], contiguous, 16-byte aligned. K == V: one
 *                 gathered row serves both the score and the value. May be NULL
 *                 when num_kv == 0.
 *   topk_indices  int32 [T, topk], contiguous. Any value outside [0, num_kv)
 *                 (-1 by convention) marks an invalid slot whose row is never
 *                 read. Order within a row does not matter; a repeated valid
 *                 index counts once per occurrence.
 *   attn_sink     fp32 [H] or NULL (no sink).
 *   scale         any finite float; 1/sqrt(512) by convention.
 *   out           bf16 [T, H, 512], contiguous, 16-byte aligned; fully written.
 *   lse           fp32 [T, H], contiguous; fully written; natural log,
 *                 sink-inclusive.
 *   T, H, num_kv, topk   sizes; T == 0 returns SMLA_OK without a launch.
 *   stream        a hipStream_t, or NULL for the default stream.
 *
 * out and lse must not alias any input (not checked). The call never
 * synchronises: results are ready when `stream` reaches this point. Faults
 * during execution surface at the caller's next synchronisation, as usual for
 * HIP. Results are bitwise-deterministic: the same inputs give the same bits
 * on every call. Thread-safe and reentrant.
 *
 * Calls with few (token, head group) units -- fewer than the device has
 * compute units -- and top-k rows of at least 128 entries split each row over
 * several workgroups and merge the partial results in a second kernel (the
 * review of "[Triton/Gluon] [CI] [gfx942] Tuned sparse MLA prefill for
 * DSv4.1-Flash TP4; fix attn_sink in Triton fallback" (aiter PR #6002) notes
 * that a per-token grid leaves the GPU idle for decode-sized calls). The
 * partials live in stream-ordered scratch taken from a memory pool the library
 * creates once per device and keeps until the process ends (it retains its
 * high-water mark: 2 KiB per (unit, split, head), under 140 MB in all; a few
 * MiB for decode-sized calls). If that scratch cannot
 * be had, the call runs the single-pass path instead; the result differs only
 * by floating-point rounding order. Apart from that, only the int64-row, fp8
 * (when it decodes its pool) and backward entry points take scratch.
 */
int sparse_mla_prefill(const void* q, const void* kv, const int32_t* topk_indices, const float* attn_sink,
                       float scale, void* out, float* lse, int64_t T, int64_t H, int64_t num_kv,
                       int64_t topk, void* stream);

/*
 * sparse_mla_prefill_noalloc -- sparse_mla_prefill for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, same kernels, same results
 * bit for bit (the same split decision is taken), but the call itself never
 * calls hipMalloc, hipFree or an allocating routine.
 *
 * Where sparse_mla_prefill would split each top-k row (few (token, head group)
 * units, rows of >= 128 entries), the partial results go to one static device
 * array of SPARSE_MLA_NOALLOC_SCRATCH_BYTES per device instead of the pool; it
 * is reserved when the library's code is first loaded on that device and held
 * until the process ends. A call whose partials need more than that returns
 * SMLA_ERR_SCRATCH_LIMIT before anything is enqueued (2056 bytes per (unit,
 * split, head): e.g. 16 tokens at H = 16 or H = 128 fit, 100 tokens at H = 128
 * with 512-entry rows do not). Every partial a call reads is written by the same
 * call, so the array needs no clearing; but all calls on one device share it,
 * so two calls whose execution overlaps on one device (different streams, or
 * host threads) race on it and must be ordered by the caller. Calls that do
 * not split use no scratch at all.
 */
int sparse_mla_prefill_noalloc(const void* q, const void* kv, const int32_t* topk_indices, const float* attn_sink,
                               float scale, void* out, float* lse, int64_t T, int64_t H, int64_t num_kv,
                               int64_t topk, void* stream);

/*
 * sparse_mla_prefill_fp8 -- the same operation on a pool of OCP FP8 E4M3
 * ("e4m3fn") codes: kv is uint8 [num_kv, 512], contiguous, 16-byte aligned,
 * and K == V == code value * kv_scale (one fp32 dequant scale for the pool;
 * any finite value). Codes decode exactly (exponent bias 7, subnormals at
 * exponent 0, NaN at S.1111.111, no infinity); a NaN code in a referenced row
 * propagates to that (t,h) like a NaN in a bf16 row. Every other argument as
 * for sparse_mla_prefill (int32 rows). The forward pages only mention fp8
 * caches, as a type their Triton path could not take ("[Triton/Gluon] [CI]
 * [gfx942] Tuned sparse MLA prefill for DSv4.1-Flash TP4; fix attn_sink in
 * Triton fallback" (aiter PR #6002), description and review). SMLA_ERR_BAD_SCALE
 * if kv_scale or scale * kv_scale is not finite.
 *
 * Two ways to run it, chosen per call (see sparse_mla_set_fp8_pool_decode):
 * the fp8 kernels gather the codes (half the bytes of a bf16 row) and convert
 * them in registers; or the whole pool is first decoded into bf16 copies of
 * its code values (exact) in stream-ordered scratch of num_kv KiB, taken from
 * the same pool as the split path's and freed stream-ordered after the call,
 * and the bf16 kernels run on that copy with the dequant scale folded in. The
 * second is faster when the call gathers many times the pool's rows; by
 * default it is taken when num_kv <= 262144 (256 MiB of copy) and
 * T * topk >= 8 num_kv, and when its scratch cannot be had the fp8 kernels
 * run. Results of the two agree to floating-point rounding order.
 */
int sparse_mla_prefill_fp8(const void* q, const void* kv, float kv_scale, const int32_t* topk_indices,
                           const float* attn_sink, float scale, void* out, float* lse, int64_t T, int64_t H,
                           int64_t num_kv, int64_t topk, void* stream);

/* How sparse_mla_prefill_fp8 treats the pool (process-wide; the default is AUTO). */
#define SMLA_FP8_POOL_DECODE_NEVER 0  /* always the fp8 kernels                                   */
#define SMLA_FP8_POOL_DECODE_AUTO 1   /* decode to a bf16 copy when it pays (sizes as above)       */
#define SMLA_FP8_POOL_DECODE_ALWAYS 2 /* decode whenever the scratch can be had                    */

/*
 * sparse_mla_set_fp8_pool_decode -- set the mode above for every later
 * sparse_mla_prefill_fp8 call of the process (all devices, all threads; calls
 * already enqueued are not affected). Returns the previous mode, or -1 (and
 * changes nothing) for a value that is not one of the three.
 */
int sparse_mla_set_fp8_pool_decode(int mode);

/*
 * sparse_mla_fp8_pool_decoded -- 1 if a sparse_mla_prefill_fp8 call of these
 * sizes would decode the pool under the current mode (given its scratch can be
 * had), else 0. No device is needed.
 */
int sparse_mla_fp8_pool_decoded(int64_t T, int64_t topk, int64_t num_kv);

/*
 * sparse_mla_prefill_i64 -- the same operation with int64 top-k rows
 * (topk_indices: int64 [T, topk], contiguous, 8-byte aligned; every other
 * argument as above).
 *
 * "[Triton/Gluon] [CI] [gfx942] Tuned sparse MLA prefill for DSv4.1-Flash
 * TP4; fix attn_sink in Triton fallback" (aiter PR #6002), description: int64
 * slot indices are kept as int64, because a cast to int32 wrapped slots at or
 * past 2^31 onto valid rows. Here every index is compared as a 64-bit value:
 * valid iff 0 <= idx < num_kv, anything else (2^32 + r included) is an
 * invalid slot. At H <= 16 in a single pass (T at least the device's compute
 * units, or rows under 128 entries) the forward kernel reads the int64 rows
 * itself. Otherwise a first kernel maps the rows to int32 row numbers (-1 for
 * invalid) in stream-ordered scratch of 4 * T * topk bytes from the library's
 * per-device pool (SMLA_ERR_NO_MEMORY if that cannot be had) and the forward
 * runs as for int32 rows. Either way results are bitwise those of
 * sparse_mla_prefill on the equivalent int32 rows.
 */
int sparse_mla_prefill_i64(const void* q, const void* kv, const int64_t* topk_indices, const float* attn_sink,
                           float scale, void* out, float* lse, int64_t T, int64_t H, int64_t num_kv,
                           int64_t topk, void* stream);

/*
 * sparse_mla_backward -- gradients of sparse_mla_prefill ("[Triton/Gluon]
 * [GFX950][DSV4] Sparse MLA training backward" (aiter PR #4766), sections
 * "Contract" and "Structure"). With x_s = scale q[t,h] . kv[r_s] over the
 * valid slots s of token t (r_s its row, validity as in the forward),
 * P_s = exp(x_s - lse[t,h]) and delta = sum_d o[t,h,d] dout[t,h,d]:
 *   dS_s = P_s (dout[t,h] . kv[r_s] - delta)
 *   dq[t,h] = scale sum_s dS_s kv[r_s]
 *   dkv[r]  = sum over (t, h, s) with r_s == r of scale dS_s q[t,h] + P_s dout[t,h]
 *   d_sink[h] = -sum_t exp(attn_sink[h] - lse[t,h]) delta        (K == V)
 *
 * q, dout, o   bf16 [T, H, 512], contiguous, 16-byte aligned (o and lse
 *              are the forward's outputs; lse is sink-inclusive, natural log)
 * kv           bf16 [num_kv, 512], contiguous, 16-byte aligned
 * lse          fp32 [T, H]
 * topk_indices int32 [T, topk]; slots outside [0, num_kv) are invalid
 * attn_sink    fp32 [H] or NULL; d_sink is required with it, ignored without
 * dq           bf16 [T, H, 512] out;  dkv bf16 [num_kv, 512] out (rows no slot
 *              holds are written 0);  d_sink fp32 [H] out
 * H <= 128 (SMLA_ERR_BAD_SIZE above), num_kv < 2^31, T * round_up(topk, 32) < 2^31.
 *
 * Enqueued on `stream`. dkv is deterministic: each row sums its contributors
 * in (token, slot) order, with no atomics. The work runs in passes over
 * consecutive tokens (the bound the page's R_CHUNK option serves, here over
 * tokens: dq of a token is then complete within one pass); P, dS, the sort
 * keys and the per-slot dkv terms exist for one pass at a time, about
 * round_up(topk, 32) * (4 H + 1104) bytes per token of the pass. This entry
 * point sizes the passes so that one pass's scratch stays under 4 GiB (one
 * pass for T=4096, H=128, topk=512 at 3.4 GB; four for topk=1024 at T=8192);
 * with more than one pass, dkv is summed in an fp32 accumulator of
 * num_kv * 2 KiB and rounded to bf16 at the end (otherwise each row is rounded
 * once from its fp32 sum directly). Scratch in all: the pass buffers, the sort's counts, 4 T H +
 * 4 (num_kv + 1) bytes and that accumulator, stream-ordered from the library's
 * per-device pool (the forward's split path uses the same pool, which keeps at
 * most 4.5 GiB between calls) and returned before the call's work ends;
 * SMLA_ERR_NO_MEMORY if it cannot be had, before any launch. The inverted
 * index is a stable radix sort of the library's own that sets no memory, so
 * the call can be captured into a HIP graph (its scratch then becomes the
 * graph's allocation nodes).
 */
int sparse_mla_backward(const void* q, const void* kv, const void* dout, const void* o, const float* lse,
                        const int32_t* topk_indices, const float* attn_sink, float scale, void* dq, void* dkv,
                        float* d_sink, int64_t T, int64_t H, int64_t num_kv, int64_t topk, void* stream);

/*
 * sparse_mla_backward_chunked -- sparse_mla_backward with the pass size given:
 * chunk_tokens > 0 tokens per pass (the last pass may be shorter), 0 as
 * sparse_mla_backward chooses; SMLA_ERR_BAD_SIZE if negative. Same outputs up
 * to the fp32 summation order of dkv across passes.
 */
int sparse_mla_backward_chunked(const void* q, const void* kv, const void* dout, const void* o, const float* lse,
                                const int32_t* topk_indices, const float* attn_sink, float scale, void* dq, void* dkv,
                                float* d_sink, int64_t T, int64_t H, int64_t num_kv, int64_t topk,
                                int64_t chunk_tokens, void* stream);

/*
 * sparse_mla_backward_i64 -- sparse_mla_backward_chunked with int64 top-k rows
 * (int64 [T, topk], contiguous, 8-byte aligned; validity as for
 * sparse_mla_prefill_i64: 0 <= idx < num_kv compared in 64 bits). The rows are
 * first mapped to int32 row numbers (-1 for invalid) in stream-ordered scratch
 * of 4 * T * topk bytes from the library's per-device pool; the gradients are
 * then bitwise those of the int32 backward on the equivalent rows. Argument
 * errors return before anything is enqueued; SMLA_ERR_NO_MEMORY may also come
 * after the mapping (the backward's own scratch), with no output written.
 */
int sparse_mla_backward_i64(const void* q, const void* kv, const void* dout, const void* o, const float* lse,
                            const int64_t* topk_indices, const float* attn_sink, float scale, void* dq, void* dkv,
                            float* d_sink, int64_t T, int64_t H, int64_t num_kv, int64_t topk, int64_t chunk_tokens,
                            void* stream);

/*
 * sparse_mla_backward_fp8 -- sparse_mla_backward_chunked on a pool of OCP FP8
 * E4M3 codes (kv: uint8 [num_kv, 512], 16-byte aligned) with one fp32 dequant
 * scale: K == V == code value * kv_scale, as in sparse_mla_prefill_fp8, and
 * dkv (bf16 [num_kv, 512]) is the gradient with respect to those values. The
 * pool is first decoded into bf16 copies of its code values (exact) in
 * stream-ordered scratch of num_kv KiB from the library's per-device pool;
 * the backward then folds kv_scale into the logits, dP = dout . kv and dq.
 * SMLA_ERR_BAD_SCALE if kv_scale or scale * kv_scale is not finite. Argument
 * errors return before anything is enqueued; SMLA_ERR_NO_MEMORY may also come
 * after the decoding (the backward's own scratch), with no output written.
 */
int sparse_mla_backward_fp8(const void* q, const void* kv, float kv_scale, const void* dout, const void* o,
                            const float* lse, const int32_t* topk_indices, const float* attn_sink, float scale,
                            void* dq, void* dkv, float* d_sink, int64_t T, int64_t H, int64_t num_kv, int64_t topk,
                            int64_t chunk_tokens, void* stream);

/* Human-readable text for a status code (static storage; never NULL). */
const char* sparse_mla_status_string(int status);

/*
 * Name of the kernel that sparse_mla_prefill (kv_fp8 == 0) launches for H
 * heads and top-k rows of `topk` entries when the call is not split over the
 * top-k row, or (kv_fp8 != 0) the kernel that reads an fp8 pool's codes
 * directly; an fp8 call that decodes its pool (sparse_mla_fp8_pool_decoded)
 * launches the kv_fp8 == 0 kernel after the decoding. Static storage, as the
 * name appears in profiler traces; NULL when H < 1 or topk < 0. Pure host
 * function: no device access.
 */
const char* sparse_mla_kernel_name(int64_t H, int64_t topk, int kv_fp8);

/* Library version, major * 10000 + minor * 100 + patch. */
int sparse_mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H */
