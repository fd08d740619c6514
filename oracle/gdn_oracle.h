/*
 * gdn_oracle.h -- float64 CPU oracle for the Gated DeltaNet token mixer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. The GPU library never links it,
 * and it includes nothing from the GPU library.
 *
 * Sources (web pages, cited by title and section):
 *   [MoE report]  "Qwen3.5-MoE-35B-A3B 模型架构深度拆解报告" (pillumina.github.io),
 *                 CH 3: §3.3 operator breakdown, §3.4 K/V head asymmetry,
 *                 §3.5 QK L2 norm, §3.7 chunk_gated_delta_rule seven steps.
 *   [xiwon notes] "Qwen3.5 观测记录" (xiwon.blog): sections "DeltaNet",
 *                 "Gated DeltaNet", "Qwen3_5MoeGatedDeltaNet", "Cache".
 *   [intro]       "Qwen3.5模型介绍" (blog.dijkstra-jhd.cn): section "线性注意力".
 *
 * All arrays are host memory, row-major, float64, caller-owned.
 * cu_seqlens has num_seqs+1 non-decreasing entries starting at 0; sequence n
 * occupies packed rows [cu_seqlens[n], cu_seqlens[n+1]).
 * Return value: 0 on success, -1 on an invalid argument (nothing written).
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Gated delta rule, token by token (the definition; no chunking).
 *   q, k : [T][hqk][dk]      v : [T][hv][dv]      g, beta : [T][hv]
 *   h0   : [N][hv][dk][dv] or NULL (zeros)         o : [T][hv][dv]
 *   ht   : [N][hv][dk][dv] or NULL (not returned)
 * V head h reads QK head h / (hv/hqk). g is the log-decay (alpha = exp(g)). */
int gdn_oracle_recurrent(int64_t num_seqs, const int64_t* cu_seqlens,
                         int64_t hqk, int64_t hv, int64_t dk, int64_t dv,
                         const double* q, const double* k, const double* v,
                         const double* g, const double* beta,
                         const double* h0, double scale,
                         double* o, double* ht);

/* Front end: causal depthwise conv (4 taps) + SiLU over the packed q|k|v
 * channels, split into heads, L2 norm of q and k head vectors, gate math.
 *   x : [T][conv_dim], conv_dim = 2*hqk*dk + hv*dv
 *   w : [conv_dim][4]   bias : [conv_dim] or NULL
 *   a, b : [T][hv]      A_log, dt_bias : [hv]
 *   out q, k : [T][hqk][dk]   v : [T][hv][dv]   g, beta : [T][hv] */
int gdn_oracle_prepare(int64_t num_seqs, const int64_t* cu_seqlens,
                       int64_t hqk, int64_t hv, int64_t dk, int64_t dv,
                       const double* x, const double* w, const double* bias,
                       const double* a, const double* b,
                       const double* A_log, const double* dt_bias, double l2_eps,
                       double* q, double* k, double* v, double* g, double* beta);

/* Output gate: out = RMSNorm(o) * SiLU(z) per row of dv values,
 *   out[r][j] = o[r][j] / sqrt(mean_j o[r][.]^2 + eps) * factor_j * z[r][j] sigmoid(z[r][j]),
 *   factor_j = w[j] + w_offset, or 1 when w is NULL.   o, z, out : [rows][dv]. */
int gdn_oracle_gated_rmsnorm(int64_t rows, int64_t dv, const double* o, const double* z,
                             const double* w, double w_offset, double eps, double* out);

/* Decode-side front end for one token per sequence with a cached conv window.
 *   x : [N][conv_dim]   window : [N][conv_dim][3] previous inputs, oldest first (in/out:
 *   becomes (window[1], window[2], x))   w : [conv_dim][4]   bias : [conv_dim] or NULL
 *   a, b : [N][hv]   A_log, dt_bias : [hv]
 *   out q, k : [N][hqk][dk]   v : [N][hv][dv]   g, beta : [N][hv] */
int gdn_oracle_decode_prepare(int64_t num_seqs, int64_t hqk, int64_t hv, int64_t dk, int64_t dv,
                              const double* x, double* window, const double* w,
                              const double* bias, const double* a, const double* b,
                              const double* A_log, const double* dt_bias, double l2_eps,
                              double* q, double* k, double* v, double* g, double* beta);

/* Reverse mode of gdn_oracle_recurrent: gradients of L = sum(o * dout) + sum(ht * dht)
 * (dht may be NULL: no final-state term) by backpropagation through the tokens.
 *   dout : [T][hv][dv]      dht : [N][hv][dk][dv] or NULL
 *   out dq, dk : [T][hqk][dk] (summed over the V heads that read each QK head)
 *       dv : [T][hv][dv]    dg, dbeta : [T][hv]    dh0 : [N][hv][dk][dv] or NULL
 * The other arguments are those of gdn_oracle_recurrent. */
int gdn_oracle_recurrent_backward(int64_t num_seqs, const int64_t* cu_seqlens,
                                  int64_t hqk, int64_t hv, int64_t dk, int64_t dv,
                                  const double* q, const double* k, const double* v,
                                  const double* g, const double* beta,
                                  const double* h0, double scale,
                                  const double* dout, const double* dht,
                                  double* dq, double* dkk, double* dvv,
                                  double* dg, double* dbeta, double* dh0);

/* Number of OpenMP threads the oracle runs on (for reporting). */
int gdn_oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
