/*
 * CPU oracle for the sparse MLA backward (DeepSeek-V4).
 *
 * TEST INFRASTRUCTURE ONLY, like smla_oracle.c beside it: the plain, slow,
 * obviously correct definition that the GPU backward is checked against.
 * It shares no code with the HIP library, and the product path never calls it.
 *
 * The operation is the forward of smla_oracle.c; the page "[Triton/Gluon]
 * [GFX950][DSV4] Sparse MLA training backward" (aiter PR #4766), sections
 * "Contract" and "Structure", fixes its backward's inputs and outputs: given
 * q, kv, the output gradient dO, the forward's o and sink-inclusive lse, the
 * top-k rows and the optional sink, produce dq, dkv and d_sink. Writing
 * x_s = scale * q[t,h] . kv[r_s] for the valid slots s of token t (r_s its
 * row), the forward is o = sum_s P_s kv[r_s] with P_s = exp(x_s - lse) and
 * lse = ln(sum_s exp(x_s) + exp(sink[h])). Differentiating that (K == V, so
 * a row collects both its key and its value gradient):
 *
 *   delta[t,h] = sum_d o[t,h,d] dO[t,h,d]                 (the page's rowsum(O*dO))
 *   dP_s       = dO[t,h] . kv[r_s]
 *   dS_s       = P_s (dP_s - delta[t,h])
 *   dq[t,h]   += scale dS_s kv[r_s]
 *   dkv[r_s]  += scale dS_s q[t,h] + P_s dO[t,h]          (summed over t, h, s)
 *   d_sink[h] += -exp(sink[h] - lse[t,h]) delta[t,h]       (summed over t)
 *
 * Readings:
 *  - P is recomputed from the lse passed in, as the page's composition of the
 *    forward's lse with the backward says; o is the o passed in (the
 *    forward's rounded output, or an exact one).
 *  - Slots are valid as in the forward (0 <= idx < num_kv); invalid slots
 *    contribute nothing, a repeated index contributes once per slot.
 *  - A sink of -inf contributes nothing to d_sink; without a sink there is
 *    no d_sink.
 *
 * Precision: bf16 inputs widened exactly; o and lse taken as double; every
 * sum in double, in index order.
 *
 * The pool may also hold OCP FP8 E4M3 codes with one dequant scale: every
 * kv element above is then code value * kv_scale, decoded as the forward
 * oracle decodes it (smla_oracle_kv_value), and dkv is the gradient with
 * respect to those values.
 *
 * dq is evaluated per (t, h) for a list of tokens; dkv for a list of rows,
 * each row scanning every (t, s) for the slots that hold it (plain, and
 * independent of how any index is built); d_sink over all tokens.
 *
 * Optionally, for each output element, the sum of the absolute values of the
 * terms added into it (dq_mag, dkv_mag, dsink_mag): the scale of the rounding
 * error of any evaluation that rounds its terms (a test tolerance derives
 * from it); it does not enter the gradients.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BWD_D 512

static double bw_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int bw_valid(int32_t r, int64_t num_kv) { return r >= 0 && (int64_t)r < num_kv; }

/* element d of pool row r (bf16 bits, or an fp8 code times kv_scale): smla_oracle.c */
double smla_oracle_kv_value(const void* kv, int kv_fp8, double kv_scale, int64_t r, int d);

typedef struct {
  const void* kv;
  int fp8;
  double scale;
} BwPool;

static double bw_kv(const BwPool* pool, int64_t r, int d) { return smla_oracle_kv_value(pool->kv, pool->fp8, pool->scale, r, d); }

/* scale * q[t,h] . kv[r] and dO[t,h] . kv[r] */
static void bw_dots(const uint16_t* qrow, const uint16_t* dorow, const BwPool* pool, int64_t r, double scale,
                    double* x, double* dp) {
  double a = 0.0, b = 0.0;
  for (int d = 0; d < BWD_D; ++d) {
    const double k = bw_kv(pool, r, d);
    a += bw_bf16(qrow[d]) * k;
    b += bw_bf16(dorow[d]) * k;
  }
  *x = scale * a;
  *dp = b;
}

/*
 * q, dout bf16 bits [T, H, 512]; kv bf16 bits [num_kv, 512] (kv_fp8 == 0) or
 * OCP FP8 E4M3 codes [num_kv, 512] with kv_scale (kv_fp8 != 0); o, lse double
 * [T, H, 512] / [T, H]; topk int32 [T, topk_n]; sink fp32 [H] or NULL.
 * tokens int64 [n_tokens] (NULL: all T, then n_tokens must be T) -> dq double
 * [n_tokens, H, 512] (NULL: skipped). rows int64 [n_rows] -> dkv double
 * [n_rows, 512] (NULL: skipped). d_sink double [H] (NULL: skipped; zeros
 * without a sink). Returns 0, -1 on a bad argument, -2 out of memory.
 */
int smla_oracle_backward(const uint16_t* q, const void* kv, int kv_fp8, double kv_scale, const uint16_t* dout,
                         const double* o,
                         const double* lse, const int32_t* topk, const float* sink, double scale, int64_t T, int64_t H,
                         int64_t num_kv, int64_t topk_n, const int64_t* tokens, int64_t n_tokens, double* dq,
                         const int64_t* rows, int64_t n_rows, double* dkv, double* d_sink, double* dq_mag,
                         double* dkv_mag, double* dsink_mag, int nthreads) {
  const int D = BWD_D;
  const BwPool pool = {kv, kv_fp8, kv_scale};
  if (T < 0 || H < 1 || num_kv < 0 || topk_n < 0 || n_tokens < 0 || n_rows < 0) return -1;
  if (T > 0 && (!q || !dout || !o || !lse || (topk_n > 0 && !topk))) return -1;
  if (!tokens && dq && n_tokens != T) return -1;
  for (int64_t i = 0; tokens && i < n_tokens; ++i)
    if (tokens[i] < 0 || tokens[i] >= T) return -1;
  for (int64_t i = 0; rows && i < n_rows; ++i)
    if (rows[i] < 0 || rows[i] >= num_kv) return -1;
  if (dkv && n_rows > 0 && !rows) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

  /* delta for every (t, h) */
  double* delta = (double*)malloc(sizeof(double) * (size_t)(T * H > 0 ? T * H : 1));
  if (!delta) return -2;
#pragma omp parallel for schedule(static)
  for (int64_t th = 0; th < T * H; ++th) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += o[th * D + d] * bw_bf16(dout[th * D + d]);
    delta[th] = acc;
  }

  /* dq */
  if (dq) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_tokens; ++i) {
      const int64_t t = tokens ? tokens[i] : i;
      for (int64_t h = 0; h < H; ++h) {
        double* g = dq + (i * H + h) * D;
        double* gm = dq_mag ? dq_mag + (i * H + h) * D : NULL;
        for (int d = 0; d < D; ++d) g[d] = 0.0;
        if (gm)
          for (int d = 0; d < D; ++d) gm[d] = 0.0;
        const uint16_t* qrow = q + (t * H + h) * D;
        const uint16_t* dorow = dout + (t * H + h) * D;
        for (int64_t s = 0; s < topk_n; ++s) {
          const int32_t r = topk[t * topk_n + s];
          if (!bw_valid(r, num_kv)) continue;
          double x, dp;
          bw_dots(qrow, dorow, &pool, r, scale, &x, &dp);
          const double p = exp(x - lse[t * H + h]);
          const double ds = p * (dp - delta[t * H + h]);
          for (int d = 0; d < D; ++d) g[d] += scale * ds * bw_kv(&pool, r, d);
          if (gm)
            for (int d = 0; d < D; ++d) gm[d] += fabs(scale * ds * bw_kv(&pool, r, d));
        }
      }
    }
  }

  /* dkv, one requested row at a time: every slot of every token that holds it */
  if (dkv) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
      const int64_t r = rows[i];
      double* g = dkv + i * D;
      double* gm = dkv_mag ? dkv_mag + i * D : NULL;
      for (int d = 0; d < D; ++d) g[d] = 0.0;
      if (gm)
        for (int d = 0; d < D; ++d) gm[d] = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        for (int64_t s = 0; s < topk_n; ++s) {
          if ((int64_t)topk[t * topk_n + s] != r) continue;
          for (int64_t h = 0; h < H; ++h) {
            const uint16_t* qrow = q + (t * H + h) * D;
            const uint16_t* dorow = dout + (t * H + h) * D;
            double x, dp;
            bw_dots(qrow, dorow, &pool, r, scale, &x, &dp);
            const double p = exp(x - lse[t * H + h]);
            const double ds = p * (dp - delta[t * H + h]);
            for (int d = 0; d < D; ++d) g[d] += scale * ds * bw_bf16(qrow[d]) + p * bw_bf16(dorow[d]);
            if (gm)
              for (int d = 0; d < D; ++d) gm[d] += fabs(scale * ds * bw_bf16(qrow[d])) + fabs(p * bw_bf16(dorow[d]));
          }
        }
      }
    }
  }

  /* d_sink */
  if (d_sink) {
    for (int64_t h = 0; h < H; ++h) {
      double acc = 0.0, mag = 0.0;
      const double sk = sink ? (double)sink[h] : -INFINITY;
      if (sk != -INFINITY)
        for (int64_t t = 0; t < T; ++t) {
          acc -= exp(sk - lse[t * H + h]) * delta[t * H + h];
          mag += fabs(exp(sk - lse[t * H + h]) * delta[t * H + h]);
        }
      d_sink[h] = acc;
      if (dsink_mag) dsink_mag[h] = mag;
    }
  }
  free(delta);
  return 0;
}
