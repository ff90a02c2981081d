/*
 * CPU oracle for the sparse MLA prefill forward (DeepSeek-V4).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition that the GPU path is checked against. Only the test suite, the
 * package smoke check and the benchmark's CPU-baseline leg may load it. It
 * shares no code, header, table or helper with the HIP library, and the
 * product path never calls it.
 *
 * What it computes (the operation's contract as stated on the page
 * "[Triton/Gluon] [GFX950][DSV4] Sparse MLA training backward" (aiter PR
 * #4766), section "Contract"): for every token t and head h,
 *
 *   valid slots  V_t = { s : 0 <= topk[t,s] < num_kv }      (order kept)
 *   logits       x_s = scale * sum_d q[t,h,d] * kv[topk[t,s], d]
 *   sink logit   the per-head attn_sink[h], unscaled, with no value row; it
 *                enters the softmax max and denominator only
 *   m   = max({x_s} U {sink})           Z = sum_s exp(x_s - m) + exp(sink - m)
 *   o   = sum_s exp(x_s - m) * kv[topk[t,s], :] / Z        (then bf16, RNE)
 *   lse = m + ln Z                                           (natural log)
 *
 * Readings of the pages that this follows:
 *  - Any index outside [0, num_kv) is invalid and its row is never read (the
 *    page "Tuned sparse MLA prefill for DSv4.1-Flash TP4; fix attn_sink in
 *    Triton fallback" (aiter PR #6002): invalid KV rows are never loaded, and
 *    its test note masks slots outside [0, len(kv)) -- -1, exactly num_kv,
 *    and values up to the int32 maximum).
 *  - The sink is folded into the running max as well as the denominator (the
 *    review of the reference forward on the backward page asks for
 *    m = max(max(s), sink)); lse is therefore sink-inclusive, as that page's
 *    "Contract" section says of the forward's lse.
 *  - A row with no valid slot and no sink gives o = 0 and lse = -inf (a commit
 *    note on the backward page); with a finite sink, o = 0 and lse = sink.
 *    attn_sink[h] == -inf behaves exactly like having no sink.
 *  - Each valid slot is its own softmax term; a repeated index counts twice.
 *  - Indices may be int32 or int64; an int64 index is compared as is (the
 *    DSv4.1-Flash TP4 page's description: int64 slots at or past 2^31 used
 *    to wrap onto valid rows when cast to int32, and are kept as int64 now),
 *    so such a slot is simply invalid.
 *  - NaN anywhere in a referenced row or in q propagates to that (t,h).
 *
 * KV pools may also hold OCP FP8 E4M3 ("e4m3fn") codes with one fp32 dequant
 * scale for the whole pool (the forward pages only mention fp8 caches, as a
 * type the Triton path rejected; reading: K == V == code value * kv_scale).
 * Each code is decoded exactly from the format's definition: sign bit,
 * 4-bit exponent with bias 7, 3-bit mantissa; exponent 0 is subnormal
 * (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN; there is no infinity.
 *
 * Precision: inputs are bf16 widened exactly; every sum, exp and log is done
 * in double. o is returned both unrounded (double) and rounded to bf16
 * (double -> float -> bf16, each round to nearest even).
 *
 * Tokens are independent, so the loop over them runs under OpenMP; the
 * arithmetic inside one (t,h) is a plain sequential loop.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SMLA_ORACLE_D 512

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) return 0x7FC0u; /* NaN */
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* One OCP FP8 E4M3 code, exactly. */
static double e4m3_to_double(uint8_t c) {
  const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return sgn ? -v : v;
}

/* Element d of pool row r: bf16 bits, or an fp8 code times kv_scale. */
static double kv_at(const void* kv, int kv_fp8, double kv_scale, int64_t r, int d) {
  if (kv_fp8) return e4m3_to_double(((const uint8_t*)kv)[r * SMLA_ORACLE_D + d]) * kv_scale;
  return bf16_to_double(((const uint16_t*)kv)[r * SMLA_ORACLE_D + d]);
}

/* The same element for the backward oracle beside this file (one decoding of
 * the pool for both directions). */
double smla_oracle_kv_value(const void* kv, int kv_fp8, double kv_scale, int64_t r, int d) {
  return kv_at(kv, kv_fp8, kv_scale, r, d);
}

/* Index s of a top-k row of 4- or 8-byte signed integers. */
static int64_t idx_at(const void* row, int idx64, int64_t s) {
  return idx64 ? ((const int64_t*)row)[s] : (int64_t)((const int32_t*)row)[s];
}

/* One (t, h) pair, written straight from the definition above. */
static void one_head(const uint16_t* qrow, const void* kv, int kv_fp8, double kv_scale, const void* idx_row, int idx64,
                     int64_t topk, int64_t num_kv, int has_sink, double sink, double scale,
                     double* x /* scratch [topk] */, double* acc /* scratch [D] */,
                     double* o_exact, uint16_t* o_bf16, double* lse_out) {
  const int D = SMLA_ORACLE_D;
  /* Pass 1: logits of the valid slots and their maximum. */
  double m = -INFINITY;
  for (int64_t s = 0; s < topk; ++s) {
    int64_t r = idx_at(idx_row, idx64, s);
    if (r < 0 || r >= num_kv) continue;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += bf16_to_double(qrow[d]) * kv_at(kv, kv_fp8, kv_scale, r, d);
    double xs = scale * dot;
    x[s] = xs;
    if (!(xs <= m)) m = xs; /* a NaN logit makes m NaN */
  }
  if (has_sink && !(sink <= m)) m = sink;

  if (m == -INFINITY) { /* no valid slot, no sink */
    for (int d = 0; d < D; ++d) {
      if (o_exact) o_exact[d] = 0.0;
      if (o_bf16) o_bf16[d] = 0;
    }
    *lse_out = -INFINITY;
    return;
  }

  /* Pass 2: weights, denominator and the weighted sum of the value rows. */
  for (int d = 0; d < D; ++d) acc[d] = 0.0;
  double Z = 0.0;
  for (int64_t s = 0; s < topk; ++s) {
    int64_t r = idx_at(idx_row, idx64, s);
    if (r < 0 || r >= num_kv) continue;
    double w = exp(x[s] - m);
    Z += w;
    for (int d = 0; d < D; ++d) acc[d] += w * kv_at(kv, kv_fp8, kv_scale, r, d);
  }
  if (has_sink) Z += exp(sink - m);
  for (int d = 0; d < D; ++d) {
    double od = acc[d] / Z;
    if (o_exact) o_exact[d] = od;
    if (o_bf16) o_bf16[d] = float_to_bf16_rne((float)od);
  }
  *lse_out = m + log(Z);
}

/*
 * q      bf16 bits [T, H, 512]          kv  bf16 bits [num_kv, 512]
 * topk   [T, topk_n] of idx_bytes-byte signed integers (4 or 8)
 * sink   fp32 [H] or NULL
 * tokens int64 [n_tokens] token ids to evaluate, or NULL for 0..T-1
 * o_exact double [n_tokens, H, 512] or NULL;  o_bf16 uint16 [n_tokens, H, 512] or NULL
 * lse    double [n_tokens, H] (required)
 * n_valid int64 [n_tokens] or NULL: number of valid slots of each token
 * nthreads <= 0: OpenMP default.  Returns 0, or -1 on a bad argument.
 */
int smla_oracle_forward_kv(const uint16_t* q, const void* kv, int kv_fp8, double kv_scale, const void* topk,
                           int idx_bytes, const float* sink, double scale, int64_t T, int64_t H, int64_t num_kv,
                           int64_t topk_n, const int64_t* tokens, int64_t n_tokens, double* o_exact,
                           uint16_t* o_bf16, double* lse, int64_t* n_valid, int nthreads) {
  const int D = SMLA_ORACLE_D;
  if (T < 0 || H < 1 || num_kv < 0 || topk_n < 0 || n_tokens < 0 || !lse) return -1;
  if (idx_bytes != 4 && idx_bytes != 8) return -1;
  const int idx64 = idx_bytes == 8;
  if (!tokens && n_tokens != T) return -1;
  if (n_tokens > 0 && (!q || !topk || (num_kv > 0 && !kv))) return -1;
  for (int64_t i = 0; tokens && i < n_tokens; ++i)
    if (tokens[i] < 0 || tokens[i] >= T) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int bad = 0;
#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)(topk_n > 0 ? topk_n : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!x || !acc) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_tokens; ++i) {
      if (!x || !acc) continue;
      int64_t t = tokens ? tokens[i] : i;
      const void* idx_row = (const char*)topk + (size_t)(t * topk_n) * (size_t)idx_bytes;
      if (n_valid) {
        int64_t c = 0;
        for (int64_t s = 0; s < topk_n; ++s) {
          const int64_t r = idx_at(idx_row, idx64, s);
          c += (r >= 0 && r < num_kv);
        }
        n_valid[i] = c;
      }
      for (int64_t h = 0; h < H; ++h) {
        int has_sink = 0;
        double sk = 0.0;
        if (sink) {
          sk = (double)sink[h];
          has_sink = !(sk == -INFINITY);
        }
        one_head(q + (t * H + h) * D, kv, kv_fp8, kv_scale, idx_row, idx64, topk_n, num_kv, has_sink, sk, scale, x,
                 acc,
                 o_exact ? o_exact + (i * H + h) * D : NULL, o_bf16 ? o_bf16 + (i * H + h) * D : NULL,
                 lse + i * H + h);
      }
    }
    free(x);
    free(acc);
  }
  return bad ? -2 : 0;
}

/* bf16 pool, int32 or int64 indices. */
int smla_oracle_forward_ix(const uint16_t* q, const uint16_t* kv, const void* topk, int idx_bytes,
                           const float* sink, double scale, int64_t T, int64_t H, int64_t num_kv, int64_t topk_n,
                           const int64_t* tokens, int64_t n_tokens, double* o_exact, uint16_t* o_bf16,
                           double* lse, int64_t* n_valid, int nthreads) {
  return smla_oracle_forward_kv(q, kv, 0, 1.0, topk, idx_bytes, sink, scale, T, H, num_kv, topk_n, tokens, n_tokens,
                                o_exact, o_bf16, lse, n_valid, nthreads);
}

/* int32 indices. */
int smla_oracle_forward(const uint16_t* q, const uint16_t* kv, const int32_t* topk, const float* sink,
                        double scale, int64_t T, int64_t H, int64_t num_kv, int64_t topk_n,
                        const int64_t* tokens, int64_t n_tokens, double* o_exact, uint16_t* o_bf16,
                        double* lse, int64_t* n_valid, int nthreads) {
  return smla_oracle_forward_ix(q, kv, topk, 4, sink, scale, T, H, num_kv, topk_n, tokens, n_tokens, o_exact,
                                o_bf16, lse, n_valid, nthreads);
}

int smla_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
