/*
 * gdn_oracle.c -- float64 CPU oracle for the Gated DeltaNet token mixer.
 *
 * TEST INFRASTRUCTURE: plain, slow and sequential on purpose. It is the
 * definition of what the GPU library computes, written out token by token,
 * and it shares no code with the GPU library. Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load it.
 *
 * Pins (tests/test_oracle_*.py check this file against values that it does
 * not compute itself): a dense closed form solved with LAPACK, the chunked
 * WY form at several chunk sizes, the spec matrix form, beta = 0 decay,
 * exact retrieval with orthonormal keys, exact rational arithmetic in the
 * scalar case, numpy.convolve for the conv, and library sigmoid / softplus
 * for the gates. Nothing here is "parity unpinned".
 *
 * Page citations are listed in gdn_oracle.h.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdn_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static int check_cu(int64_t num_seqs, const int64_t* cu) {
  if (num_seqs < 0 || cu == NULL || cu[0] != 0) return -1;
  for (int64_t n = 0; n < num_seqs; ++n)
    if (cu[n + 1] < cu[n]) return -1;
  return 0;
}

/*
 * One recurrent step per token, per (sequence, V head) chain.
 *
 * The state H is [dk][dv] ("key_dim x value_dim", [MoE report] §3.3 stage 3;
 * the spec S is its transpose). Per token t, following the order of the
 * read / error / write steps in [xiwon notes] "DeltaNet" and "Gated DeltaNet"
 * and the decode code there (state multiplied by exp(g) first, then
 * delta = (v - kv_mem) * beta):
 *   H     <- exp(g_t) * H                       decay
 *   kv_j  <- sum_i H[i][j] k_t[i]               read the memory at key k_t
 *   u_j   <- beta_t * (v_t[j] - kv_j)           prediction error times strength
 *   H     <- H + k_t u^T                         rank-1 write
 *   o_t   <- scale * H^T q_t                     read-out with the query
 * GQA: V head h uses QK head h / (hv / hqk), the repeat_interleave along the
 * head axis in [xiwon notes] "Qwen3_5MoeGatedDeltaNet" and [MoE report] §3.4.
 */
int gdn_oracle_recurrent(int64_t num_seqs, const int64_t* cu, int64_t hqk, int64_t hv,
                         int64_t dk, int64_t dv, const double* q, const double* k,
                         const double* v, const double* g, const double* beta,
                         const double* h0, double scale, double* o, double* ht) {
  if (check_cu(num_seqs, cu) != 0) return -1;
  if (hqk <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || hv % hqk != 0) return -1;
  const int64_t group = hv / hqk;
  const int64_t chains = num_seqs * hv;
  int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t c = 0; c < chains; ++c) {
    const int64_t n = c / hv, h = c % hv, m = h / group;
    double* H = (double*)malloc(sizeof(double) * (size_t)(dk * dv));
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    if (H == NULL || u == NULL) {
      free(H);
      free(u);
#pragma omp atomic write
      bad = 1;
      continue;
    }
    if (h0 != NULL)
      memcpy(H, h0 + (n * hv + h) * dk * dv, sizeof(double) * (size_t)(dk * dv));
    else
      memset(H, 0, sizeof(double) * (size_t)(dk * dv));

    for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
      const double* qt = q + (t * hqk + m) * dk;
      const double* kt = k + (t * hqk + m) * dk;
      const double* vt = v + (t * hv + h) * dv;
      const double alpha = exp(g[t * hv + h]);
      const double bt = beta[t * hv + h];
      for (int64_t i = 0; i < dk * dv; ++i) H[i] *= alpha;
      for (int64_t j = 0; j < dv; ++j) {
        double kv = 0.0;
        for (int64_t i = 0; i < dk; ++i) kv += H[i * dv + j] * kt[i];
        u[j] = bt * (vt[j] - kv);
      }
      for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) H[i * dv + j] += kt[i] * u[j];
      double* ot = o + (t * hv + h) * dv;
      for (int64_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < dk; ++i) acc += H[i * dv + j] * qt[i];
        ot[j] = scale * acc;
      }
    }
    if (ht != NULL)
      memcpy(ht + (n * hv + h) * dk * dv, H, sizeof(double) * (size_t)(dk * dv));
    free(H);
    free(u);
  }
  return bad ? -1 : 0;
}

/* SiLU(y) = y * sigmoid(y) ([xiwon notes] "Qwen3_5MoeGatedDeltaNet": the conv
 * output goes through the SiLU activation). */
static double silu(double y) { return y / (1.0 + exp(-y)); }

/* softplus(x) = log(1 + e^x), written so that it neither overflows nor loses
 * the small tail. */
static double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/*
 * Front end ([MoE report] §3.3 stage 2, §3.5; [xiwon notes]
 * "Qwen3_5MoeGatedDeltaNet"; [intro] "线性注意力"):
 *  1. causal depthwise conv over time per channel, kernel 4, left padding 3,
 *     cross-correlation as nn.Conv1d computes it: tap j (0..3) multiplies the
 *     input 3 - j steps back, so tap 3 is the current token. History before a
 *     sequence's first token is zero; no tap reads another packed sequence.
 *  2. SiLU.
 *  3. split the channels into q (hqk*dk) | k (hqk*dk) | v (hv*dv), heads
 *     contiguous inside each part.
 *  4. q, k head vectors divided by sqrt(sum of squares + l2_eps).
 *  5. beta = sigmoid(b);  g = -exp(A_log) * softplus(a + dt_bias).
 */
int gdn_oracle_prepare(int64_t num_seqs, const int64_t* cu, int64_t hqk, int64_t hv,
                       int64_t dk, int64_t dv, const double* x, const double* w,
                       const double* bias, const double* a, const double* b,
                       const double* A_log, const double* dt_bias, double l2_eps,
                       double* q, double* k, double* v, double* g, double* beta) {
  if (check_cu(num_seqs, cu) != 0) return -1;
  if (hqk <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || hv % hqk != 0) return -1;
  const int64_t qdim = hqk * dk, vdim = hv * dv;
  const int64_t conv_dim = 2 * qdim + vdim;
  int bad = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < num_seqs; ++n) {
    double* y = (double*)malloc(sizeof(double) * (size_t)conv_dim);
    if (y == NULL) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
      for (int64_t c = 0; c < conv_dim; ++c) {
        double acc = bias != NULL ? bias[c] : 0.0;
        for (int64_t j = 0; j < 4; ++j) {
          const int64_t src = t - 3 + j;
          if (src >= cu[n]) acc += w[c * 4 + j] * x[src * conv_dim + c];
        }
        y[c] = silu(acc);
      }
      for (int64_t hh = 0; hh < hqk; ++hh) {
        const double* yq = y + hh * dk;
        const double* yk = y + qdim + hh * dk;
        double sq = 0.0, sk = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
          sq += yq[i] * yq[i];
          sk += yk[i] * yk[i];
        }
        const double nq = sqrt(sq + l2_eps), nk = sqrt(sk + l2_eps);
        for (int64_t i = 0; i < dk; ++i) {
          q[(t * hqk + hh) * dk + i] = yq[i] / nq;
          k[(t * hqk + hh) * dk + i] = yk[i] / nk;
        }
      }
      for (int64_t i = 0; i < vdim; ++i) v[t * vdim + i] = y[2 * qdim + i];
      for (int64_t h = 0; h < hv; ++h) {
        beta[t * hv + h] = 1.0 / (1.0 + exp(-b[t * hv + h]));
        g[t * hv + h] = -exp(A_log[h]) * softplus(a[t * hv + h] + dt_bias[h]);
      }
    }
    free(y);
  }
  return bad ? -1 : 0;
}

/* Output gate ([xiwon notes] "Qwen3_5MoeGatedDeltaNet", output stage: the core output and z are
 * reshaped to head_v_dim rows and normed together; [MoE report] §3.3 stage 4): per row of dv
 * values, RMSNorm then times SiLU(z). The RMSNorm divides by sqrt(mean of squares + eps) and
 * multiplies by a per-channel weight; [MoE report] §7.5 gives the model's RMSNorm weight in
 * the (1 + w) form, the gated norm's form is not stated, so the offset is a parameter:
 * factor_j = w[j] + w_offset, or 1 when w is NULL. */
int gdn_oracle_gated_rmsnorm(int64_t rows, int64_t dv, const double* o, const double* z,
                             const double* w, double w_offset, double eps, double* out) {
  if (rows < 0 || dv <= 0 || o == NULL || z == NULL || out == NULL || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double* x = o + r * dv;
    double ss = 0.0;
    for (int64_t j = 0; j < dv; ++j) ss += x[j] * x[j];
    const double inv = 1.0 / sqrt(ss / (double)dv + eps);
    for (int64_t j = 0; j < dv; ++j) {
      const double factor = w != NULL ? w[j] + w_offset : 1.0;
      out[r * dv + j] = x[j] * inv * factor * silu(z[r * dv + j]);
    }
  }
  return 0;
}

/* Decode-side front end: one new token per sequence with a cached convolution window
 * ([xiwon notes] "Cache": the conv state keeps the last inputs of each channel so that a
 * decode step convolves without the history; [MoE report] §3.3 stage 2). Per channel c of
 * sequence n the window holds the 3 previous mixed_qkv values, oldest first (zeros before the
 * sequence start):
 *   y = bias[c] + w[c][0] win[0] + w[c][1] win[1] + w[c][2] win[2] + w[c][3] x[c],  SiLU(y),
 * then the q | k | v split, q and k head vectors divided by sqrt(sum of squares + eps), and the
 * gates beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias), as in gdn_oracle_prepare for
 * the same token. The window then becomes (win[1], win[2], x[c]).
 *   x : [N][conv_dim]   window : [N][conv_dim][3] (in/out)   a, b : [N][hv]
 *   out q, k : [N][hqk][dk]   v : [N][hv][dv]   g, beta : [N][hv] */
int gdn_oracle_decode_prepare(int64_t num_seqs, int64_t hqk, int64_t hv, int64_t dk, int64_t dv,
                              const double* x, double* window, const double* w,
                              const double* bias, const double* a, const double* b,
                              const double* A_log, const double* dt_bias, double l2_eps,
                              double* q, double* k, double* v, double* g, double* beta) {
  if (num_seqs < 0 || hqk <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || hv % hqk != 0) return -1;
  const int64_t qdim = hqk * dk, vdim = hv * dv;
  const int64_t conv_dim = 2 * qdim + vdim;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < num_seqs; ++n) {
    double* y = (double*)malloc(sizeof(double) * (size_t)conv_dim);
    if (y == NULL) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    for (int64_t c = 0; c < conv_dim; ++c) {
      double* win = window + (n * conv_dim + c) * 3;
      const double xc = x[n * conv_dim + c];
      double acc = bias != NULL ? bias[c] : 0.0;
      acc += w[c * 4 + 0] * win[0] + w[c * 4 + 1] * win[1] + w[c * 4 + 2] * win[2] +
             w[c * 4 + 3] * xc;
      y[c] = silu(acc);
      win[0] = win[1];
      win[1] = win[2];
      win[2] = xc;
    }
    for (int64_t hh = 0; hh < hqk; ++hh) {
      const double* yq = y + hh * dk;
      const double* yk = y + qdim + hh * dk;
      double sq = 0.0, sk = 0.0;
      for (int64_t i = 0; i < dk; ++i) {
        sq += yq[i] * yq[i];
        sk += yk[i] * yk[i];
      }
      const double nq = sqrt(sq + l2_eps), nk = sqrt(sk + l2_eps);
      for (int64_t i = 0; i < dk; ++i) {
        q[(n * hqk + hh) * dk + i] = yq[i] / nq;
        k[(n * hqk + hh) * dk + i] = yk[i] / nk;
      }
    }
    for (int64_t i = 0; i < vdim; ++i) v[n * vdim + i] = y[2 * qdim + i];
    for (int64_t h = 0; h < hv; ++h) {
      beta[n * hv + h] = 1.0 / (1.0 + exp(-b[n * hv + h]));
      g[n * hv + h] = -exp(A_log[h]) * softplus(a[n * hv + h] + dt_bias[h]);
    }
    free(y);
  }
  return bad ? -1 : 0;
}
