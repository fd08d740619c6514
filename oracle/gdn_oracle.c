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
 * WY form at several chunk sizes, the matrix form of the gated delta rule, beta = 0 decay,
 * exact retrieval with orthonormal keys, exact rational arithmetic in the
 * scalar case, numpy.convolve for the conv, and library sigmoid / softplus
 * for the gates; the reverse mode against central finite differences of the
 * forward recurrence. Nothing here is "parity unpinned".
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
 * the matrix-form state S is its transpose). Per token t, following the order of the
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

/* ---- reverse mode of the token recurrence --------------------------------------------
 * Gradients of L = sum(o * dout) + sum(ht * dht) with respect to every input of
 * gdn_oracle_recurrent, by backpropagation through the tokens in reverse order (the
 * recurrence itself is the definition: [MoE report] §3.3 stage 3; the chunked training form
 * of [MoE report] §3.7 and the chunk-wise training the pages mention compute the same
 * gradients). Per token, with Ht~ = alpha H_{t-1}, w = Ht~^T k, u = beta (v - w),
 * H_t = Ht~ + k u^T and o = scale H_t^T q, given dH = dL/dH_t:
 *   dH += scale q do^T;  dq += scale H_t do;
 *   du = dH^T k;  dk += dH u;  dbeta = du . (v - w);  dv = beta du;
 *   dw = -beta du;  dHt~ = dH + k dw^T;  dk += Ht~ dw;
 *   dg = alpha <dHt~, H_{t-1}>;  dL/dH_{t-1} = alpha dHt~.
 * States are recomputed from checkpoints every kSeg tokens (memory stays small). */
enum { kSeg = 64 };

static void step_forward(int64_t dk, int64_t dv, const double* Hp, double* Hn,
                         const double* kt, const double* vt, double alpha, double bt) {
  for (int64_t j = 0; j < dv; ++j) {
    double w = 0.0;
    for (int64_t i = 0; i < dk; ++i) w += alpha * Hp[i * dv + j] * kt[i];
    const double u = bt * (vt[j] - w);
    for (int64_t i = 0; i < dk; ++i) Hn[i * dv + j] = alpha * Hp[i * dv + j] + kt[i] * u;
  }
}

int gdn_oracle_recurrent_backward(int64_t num_seqs, const int64_t* cu, int64_t hqk, int64_t hv,
                                  int64_t dk, int64_t dv, const double* q, const double* k,
                                  const double* v, const double* g, const double* beta,
                                  const double* h0, double scale, const double* dout,
                                  const double* dht, double* dq, double* dkk, double* dvv,
                                  double* dg, double* dbeta, double* dh0) {
  if (check_cu(num_seqs, cu) != 0) return -1;
  if (hqk <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || hv % hqk != 0) return -1;
  const int64_t group = hv / hqk;
  const int64_t T = cu[num_seqs];
  const int64_t S = dk * dv;
  memset(dq, 0, sizeof(double) * (size_t)(T * hqk * dk));
  memset(dkk, 0, sizeof(double) * (size_t)(T * hqk * dk));
  int bad = 0;

  /* One unit = (sequence, QK head): its V heads add into the same dq / dk rows. */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < num_seqs * hqk; ++unit) {
    const int64_t n = unit / hqk, m = unit % hqk;
    const int64_t t0 = cu[n], L = cu[n + 1] - cu[n];
    const int64_t nseg = (L + kSeg - 1) / kSeg;
    double* ckpt = (double*)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * S));
    double* Hs = (double*)malloc(sizeof(double) * (size_t)((kSeg + 1) * S));
    double* dH = (double*)malloc(sizeof(double) * (size_t)S);
    double* dHt = (double*)malloc(sizeof(double) * (size_t)S);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    double* w = (double*)malloc(sizeof(double) * (size_t)dv);
    double* du = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!ckpt || !Hs || !dH || !dHt || !u || !w || !du) {
#pragma omp atomic write
      bad = 1;
    } else {
      for (int64_t h = m * group; h < (m + 1) * group; ++h) {
        const int64_t nh = n * hv + h;
        /* forward: checkpoint the state at the start of every segment */
        double* H = Hs;
        if (h0 != NULL)
          memcpy(H, h0 + nh * S, sizeof(double) * (size_t)S);
        else
          memset(H, 0, sizeof(double) * (size_t)S);
        for (int64_t i = 0; i < L; ++i) {
          const int64_t t = t0 + i;
          if (i % kSeg == 0) memcpy(ckpt + (i / kSeg) * S, H, sizeof(double) * (size_t)S);
          step_forward(dk, dv, H, Hs + S, k + (t * hqk + m) * dk, v + (t * hv + h) * dv,
                       exp(g[t * hv + h]), beta[t * hv + h]);
          memcpy(H, Hs + S, sizeof(double) * (size_t)S);
        }
        if (dht != NULL)
          memcpy(dH, dht + nh * S, sizeof(double) * (size_t)S);
        else
          memset(dH, 0, sizeof(double) * (size_t)S);
        for (int64_t sg = nseg - 1; sg >= 0; --sg) {
          const int64_t i0 = sg * kSeg, len = (L - i0 < kSeg) ? L - i0 : kSeg;
          memcpy(Hs, ckpt + sg * S, sizeof(double) * (size_t)S);
          for (int64_t i = 0; i < len; ++i) {
            const int64_t t = t0 + i0 + i;
            step_forward(dk, dv, Hs + i * S, Hs + (i + 1) * S, k + (t * hqk + m) * dk,
                         v + (t * hv + h) * dv, exp(g[t * hv + h]), beta[t * hv + h]);
          }
          for (int64_t i = len - 1; i >= 0; --i) {
            const int64_t t = t0 + i0 + i;
            const double* Hp = Hs + i * S;       /* H_{t-1} */
            const double* Hn = Hs + (i + 1) * S; /* H_t */
            const double* qt = q + (t * hqk + m) * dk;
            const double* kt = k + (t * hqk + m) * dk;
            const double* vt = v + (t * hv + h) * dv;
            const double* dot = dout + (t * hv + h) * dv;
            double* dqt = dq + (t * hqk + m) * dk;
            double* dkt = dkk + (t * hqk + m) * dk;
            const double alpha = exp(g[t * hv + h]), bt = beta[t * hv + h];
            /* output: o = scale H_t^T q */
            for (int64_t a = 0; a < dk; ++a) {
              double acc = 0.0;
              for (int64_t j = 0; j < dv; ++j) {
                dH[a * dv + j] += scale * qt[a] * dot[j];
                acc += Hn[a * dv + j] * dot[j];
              }
              dqt[a] += scale * acc;
            }
            /* write: H_t = alpha H_{t-1} + k u^T, u = beta (v - w), w = alpha H_{t-1}^T k */
            double dbt = 0.0;
            for (int64_t j = 0; j < dv; ++j) {
              double wj = 0.0, duj = 0.0;
              for (int64_t a = 0; a < dk; ++a) {
                wj += alpha * Hp[a * dv + j] * kt[a];
                duj += dH[a * dv + j] * kt[a];
              }
              w[j] = wj;
              u[j] = bt * (vt[j] - wj);
              du[j] = duj;
              dbt += duj * (vt[j] - wj);
              dvv[(t * hv + h) * dv + j] = bt * duj;
            }
            dbeta[t * hv + h] = dbt;
            double dalpha = 0.0;
            for (int64_t a = 0; a < dk; ++a) {
              double acc_u = 0.0, acc_w = 0.0;
              for (int64_t j = 0; j < dv; ++j) {
                const double dwj = -bt * du[j];
                acc_u += dH[a * dv + j] * u[j];
                acc_w += alpha * Hp[a * dv + j] * dwj;
                const double dtil = dH[a * dv + j] + kt[a] * dwj; /* dL/dHt~ */
                dHt[a * dv + j] = dtil;
                dalpha += dtil * Hp[a * dv + j];
              }
              dkt[a] += acc_u + acc_w;
            }
            dg[t * hv + h] = alpha * dalpha;
            for (int64_t e = 0; e < S; ++e) dH[e] = alpha * dHt[e];
          }
        }
        if (dh0 != NULL) memcpy(dh0 + nh * S, dH, sizeof(double) * (size_t)S);
      }
    }
    free(ckpt);
    free(Hs);
    free(dH);
    free(dHt);
    free(u);
    free(w);
    free(du);
  }
  return bad ? -1 : 0;
}
