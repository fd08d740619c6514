/*
 * gdn.h -- C ABI of libgdn.so, the Gated DeltaNet token mixer core for MI355X (gfx950).
 *
 * The library computes the gated delta rule with a matrix state per value head,
 *   H_t = a_t H_{t-1} + k_t u_t^T,   u_t = b_t (v_t - a_t H_{t-1}^T k_t),   o_t = scale H_t^T q_t,
 * where a_t = exp(g_t), H is [d_k][d_v] (the matrix-form state S_t is H_t^T), and V head h reads
 * QK head h / (H_v / H_qk). Page citations (by page title and section):
 *   [MoE report]  "Qwen3.5-MoE-35B-A3B 模型架构深度拆解报告" (pillumina.github.io), §3.3-§3.7.
 *   [xiwon notes] "Qwen3.5 观测记录" (xiwon.blog), sections "DeltaNet", "Gated DeltaNet",
 *                 "Qwen3_5MoeGatedDeltaNet", "Cache".
 *   [intro]       "Qwen3.5模型介绍" (blog.dijkstra-jhd.cn), section "线性注意力".
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major memory, owned by the
 *     caller; the library never allocates, frees or keeps them. cu_seqlens is a device int32
 *     array of num_seqs+1 non-decreasing offsets starting at 0, with cu_seqlens[num_seqs] ==
 *     total_tokens (the host copy in the shape). Sequence n occupies packed rows
 *     [cu_seqlens[n], cu_seqlens[n+1]); an empty sequence is allowed.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued on it; no call
 *     synchronises the host, so results are ready after the stream reaches that point.
 *   - Errors: shapes, dtypes and pointers are validated on the host first. An invalid
 *     argument returns GDN_ERR_INVALID_ARGUMENT, a valid but uncompiled shape returns
 *     GDN_ERR_UNSUPPORTED, a short workspace GDN_ERR_WORKSPACE_TOO_SMALL; in all three
 *     cases nothing is launched. GDN_ERR_HIP means a launch failed (hipGetLastError).
 *     No C++ exception crosses this interface. Device contents of cu_seqlens are trusted.
 *   - The library holds no mutable global state apart from the device array of
 *     gdn_chunk_forward_noalloc: concurrent calls on different streams with disjoint outputs and
 *     workspaces are safe (gdn_chunk_forward_noalloc calls on one GPU share that array).
 *   - Supported head dims: d_k == d_v in {32, 64, 128}. num_v_heads % num_qk_heads == 0.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 3
#define GDN_CHUNK 64 /* chunk length of the chunked prefill ([MoE report] §3.7 Step 2) */

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARGUMENT = 1,
  GDN_ERR_UNSUPPORTED = 2,
  GDN_ERR_WORKSPACE_TOO_SMALL = 3,
  GDN_ERR_HIP = 4,
  GDN_ERR_SCRATCH_LIMIT = 5 /* the shape needs more workspace than gdn_chunk_forward_noalloc's
                               library-owned array holds (GDN_NOALLOC_SCRATCH_BYTES) */
} gdn_status_t;

/* GDN_DTYPE_F32_SPLIT names fp32 storage read at a lower operand precision: accepted only as
 * the qkv_dtype of gdn_prepare (which then writes fp32 q/k/v) and of the chunked-prefill calls
 * (gdn_chunk_forward, its _noalloc variant, gdn_chunk_intra, gdn_chunk_scan and the workspace
 * size), GDN_ERR_INVALID_ARGUMENT elsewhere. The prefill then takes its products on bf16 MFMA
 * with fp32 q/k/v and every computed operand as hi + lo bf16 pairs (about 16 significant bits;
 * the inverse (I + A)^-1 stays on fp32 MFMA). It is meant for fp32 q/k/v derived from bf16
 * inputs (the front end's output), whose own bar is the bf16 one; the F32 path keeps every
 * product fp32. */
typedef enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1, GDN_DTYPE_F32_SPLIT = 2 } gdn_dtype_t;

typedef struct gdn_shape {
  int32_t num_seqs;     /* N >= 1                                                         */
  int32_t total_tokens; /* T = cu_seqlens[N] (for gdn_recurrent_step: == num_seqs)        */
  int32_t num_qk_heads; /* H_qk                                                           */
  int32_t num_v_heads;  /* H_v, a multiple of H_qk                                        */
  int32_t head_dim_k;   /* d_k                                                            */
  int32_t head_dim_v;   /* d_v                                                            */
  int32_t qkv_dtype;    /* gdn_dtype_t of q, k, v (core inputs, front-end outputs). BF16   */
                        /* runs the bf16-MFMA path, F32 the fp32-MFMA path, F32_SPLIT      */
                        /* (prefill only) fp32 storage on the split-bf16 MFMA path.        */
  int32_t out_dtype;    /* gdn_dtype_t of o. BF16 output is the round-to-nearest-even cast */
                        /* of the same fp32 result an F32 output would hold.               */
  int32_t in_dtype;     /* gdn_dtype_t of the front-end inputs (mixed_qkv, conv weight and */
                        /* bias, a, b); ignored by the core entry points.                  */
  float scale;          /* multiplies o; 1.0 for the plain rule o_t = S_t q_t              */
  int32_t state_dtype;  /* gdn_dtype_t of every stored recurrent state (initial, final and */
                        /* decode state). Inside a call the state is carried in fp32; a    */
                        /* BF16 state is read exactly and stored as the round-to-nearest-  */
                        /* even cast of the fp32 state, halving its bytes.                 */
} gdn_shape_t;

/*
 * gdn_prepare -- front end of the layer ([MoE report] §3.3 stage 2 and §3.5; [xiwon notes]
 * "Qwen3_5MoeGatedDeltaNet"; [intro] "线性注意力"). Per channel c of mixed_qkv, a causal
 * depthwise conv with 4 taps in the nn.Conv1d cross-correlation order (tap 3 multiplies the
 * current token, tap 0 the token 3 steps back; zero history before each sequence start, so
 * nothing leaks across cu_seqlens boundaries), plus optional bias, then SiLU(y) = y sigmoid(y).
 * The channels split into q (H_qk*d_k) | k (H_qk*d_k) | v (H_v*d_v); each q and k head vector
 * is divided by sqrt(sum of squares + l2norm_eps). Gates: beta = sigmoid(b),
 * g = -exp(A_log) * softplus(a + dt_bias), computed in fp32.
 *   mixed_qkv   [T][2*H_qk*d_k + H_v*d_v]  in_dtype
 *   conv_weight [conv_dim][4]              in_dtype
 *   conv_bias   [conv_dim] in_dtype, or NULL for no bias
 *   a, b        [T][H_v]                   in_dtype
 *   A_log, dt_bias [H_v]                   fp32
 *   q, k (out)  [T][H_qk][d_k]             qkv_dtype
 *   v    (out)  [T][H_v][d_v]              qkv_dtype
 *   g, beta (out) [T][H_v]                 fp32 (g is the log-decay, <= 0)
 * mixed_qkv, conv_bias (when given), a, b, q, k, v, g and beta must be 16-byte aligned
 * (16-byte vector accesses); GDN_ERR_INVALID_ARGUMENT otherwise.
 */
gdn_status_t gdn_prepare(const gdn_shape_t* shape, const int32_t* cu_seqlens,
                         const void* mixed_qkv, const void* conv_weight, const void* conv_bias,
                         const void* a, const void* b, const float* A_log,
                         const float* dt_bias, float l2norm_eps, void* q, void* k, void* v,
                         float* g, float* beta, void* stream);

/* Bytes of device workspace gdn_chunk_forward needs for this shape (0 on a bad shape). The
 * bound uses total_tokens and num_seqs only: (num_seqs + total_tokens / 64) chunk slots times
 * H_v times 20992 bytes. */
size_t gdn_chunk_forward_workspace_size(const gdn_shape_t* shape);

/*
 * gdn_chunk_forward -- chunked prefill, chunk length 64 ([MoE report] §3.7 Steps 2-7, the
 * WY/UT form of the recurrence above). Sequences are cut into chunks of 64 tokens that never
 * straddle a sequence; a short tail chunk behaves as if padded with identity steps
 * (q = k = v = 0, beta = 0, g = 0). The result equals the token recurrence up to rounding.
 *   q, k          [T][H_qk][d_k] qkv_dtype     v [T][H_v][d_v] qkv_dtype
 *   g, beta       [T][H_v] fp32
 *   initial_state [N][H_v][d_k][d_v] state_dtype, or NULL for zeros
 *   o (out)       [T][H_v][d_v] out_dtype
 *   final_state   [N][H_v][d_k][d_v] state_dtype (out), or NULL; it may equal initial_state
 *   workspace     >= gdn_chunk_forward_workspace_size(shape) bytes, 256-byte aligned,
 *                 caller-owned scratch; its contents on entry do not matter.
 * q, k, v and o must be 16-byte aligned (16-byte row accesses); GDN_ERR_INVALID_ARGUMENT
 * otherwise. It runs gdn_chunk_intra then gdn_chunk_scan on `stream`.
 * Precision: the state is carried in fp32 and every product accumulates in fp32. With fp32
 * q/k/v every product is fp32. With bf16 q/k/v the two products with the state (K H and Q H)
 * take fp16 operands: q and k converted (exact for magnitudes in [2^-14, 65504], within 2^-25
 * below that; L2-normalised vectors are in range) and the state rounded to fp16 once per chunk
 * for these products (so its magnitude must stay below 65504). The state update, T diag(beta) Y
 * and P V' take the computed operands as hi + lo bf16 pairs (about 16 significant bits).
 * With qkv_dtype GDN_DTYPE_F32_SPLIT (fp32 q/k/v) every product but the inverse (fp32 MFMA)
 * runs on bf16 MFMA with both operands as hi + lo bf16 pairs, k and q included (about 16
 * significant bits each; the state itself stays fp32).
 */
gdn_status_t gdn_chunk_forward(const gdn_shape_t* shape, const int32_t* cu_seqlens,
                               const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const void* initial_state, void* o,
                               void* final_state, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * gdn_chunk_forward_noalloc -- gdn_chunk_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It takes
 * the same arguments minus the workspace and computes the same result (the same kernels); the
 * workspace is a library-owned device array of GDN_NOALLOC_SCRATCH_BYTES bytes per GPU, held from
 * the library's first use on that GPU until the process ends. It calls no hipMalloc, hipFree or
 * other allocating routine. A shape whose workspace (gdn_chunk_forward_workspace_size) exceeds the
 * array returns GDN_ERR_SCRATCH_LIMIT without launching anything: 64 MiB holds, for example, one
 * 4096-token sequence at 32 V heads ((1 + 64) x 32 records of 20992 bytes). All calls on one GPU
 * share the array, so calls that overlap on one GPU (different streams or host threads) race and
 * must be serialised by the caller. Other errors as gdn_chunk_forward.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
gdn_status_t gdn_chunk_forward_noalloc(const gdn_shape_t* shape, const int32_t* cu_seqlens,
                                       const void* q, const void* k, const void* v,
                                       const float* g, const float* beta,
                                       const void* initial_state, void* o, void* final_state,
                                       void* stream);

/*
 * The two stages of gdn_chunk_forward, exported so that they can be timed or overlapped
 * separately. gdn_chunk_intra computes everything that does not depend on the state
 * ([MoE report] §3.7 Steps 3-4: the in-chunk decay cumsum, the decayed beta*K K^T, the
 * unit-lower-triangular inverse (I + A)^-1 and the masked decayed Q K^T) into the workspace.
 * gdn_chunk_scan then runs the sequential cross-chunk recurrence (Steps 5-7) from it. The
 * workspace contents between the two calls are private to the library; scan must use the same
 * shape (its scale included), cu_seqlens, q, k, g and beta as the intra call that filled it. Alignment as for
 * gdn_chunk_forward (q, k, v, o 16 bytes; workspace 256 bytes).
 */
gdn_status_t gdn_chunk_intra(const gdn_shape_t* shape, const int32_t* cu_seqlens,
                             const void* q, const void* k, const float* g, const float* beta,
                             void* workspace, size_t workspace_bytes, void* stream);
gdn_status_t gdn_chunk_scan(const gdn_shape_t* shape, const int32_t* cu_seqlens,
                            const void* q, const void* k, const void* v,
                            const void* initial_state, void* o, void* final_state,
                            const void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_backward -- gradients of the chunked prefill for training ([MoE report] §3.7: the
 * chunked form trained chunk by chunk; the token recurrence above is the definition it
 * differentiates). For the loss L = sum(o * dout) + sum(final_state * dht), with o and
 * final_state those gdn_chunk_forward returns for the same inputs, it writes
 *   dq, dk [T][H_qk][d_k] qkv_dtype (summed over the V heads that read each QK head),
 *   dv [T][H_v][d_v] qkv_dtype, dg, dbeta [T][H_v] fp32, dh0 [N][H_v][d_k][d_v] state_dtype.
 *   dout [T][H_v][d_v] out_dtype; dht [N][H_v][d_k][d_v] state_dtype, or NULL for no
 *   final-state term; initial_state as in gdn_chunk_forward (NULL for zeros); dh0 may be NULL.
 * Accumulation is fp32; with bf16 q/k/v most products run on bf16 MFMA with the computed
 * operands carried as hi + lo bf16 pairs (about 16 significant bits), the rest on fp32 MFMA; with
 * fp32 inputs every product is fp32. The forward states are recomputed from initial_state
 * (nothing from a forward call is reused). workspace >= gdn_chunk_backward_workspace_size(shape) bytes,
 * 256-byte aligned, caller-owned scratch. q, k, v, dout, dq, dk and dv must be 16-byte aligned
 * (vector row accesses); GDN_ERR_INVALID_ARGUMENT otherwise.
 */
size_t gdn_chunk_backward_workspace_size(const gdn_shape_t* shape);
gdn_status_t gdn_chunk_backward(const gdn_shape_t* shape, const int32_t* cu_seqlens,
                                const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const void* initial_state, const void* dout,
                                const void* dht, void* dq, void* dk, void* dv, float* dg,
                                float* dbeta, void* dh0, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * gdn_recurrent_step -- one decode token per sequence ([MoE report] §3.3 stage 3 decode;
 * [xiwon notes] "Qwen3_5MoeGatedDeltaNet" recurrent branch and "Cache": the state is read,
 * updated once and written back in place). Requires total_tokens == num_seqs.
 *   q, k  [N][H_qk][d_k] qkv_dtype     v [N][H_v][d_v] qkv_dtype
 *   g, beta [N][H_v] fp32
 *   state [N][H_v][d_k][d_v] state_dtype, read and overwritten with the new state (16-byte
 *         aligned)
 *   o (out) [N][H_v][d_v] out_dtype
 */
gdn_status_t gdn_recurrent_step(const gdn_shape_t* shape, const void* q, const void* k,
                                const void* v, const float* g, const float* beta,
                                void* state, void* o, void* stream);

/*
 * gdn_decode_prepare -- front end of one decode token per sequence with a cached convolution
 * window ([xiwon notes] "Cache": the conv state keeps the last inputs of each channel;
 * [MoE report] §3.3 stage 2, decode path). Per channel c of sequence n, with the window
 * win = conv_window[n][c][0..2] holding the three previous mixed_qkv values, oldest first
 * (zeros at a sequence start),
 *   y = bias[c] + w[c][0] win[0] + w[c][1] win[1] + w[c][2] win[2] + w[c][3] x[n][c],
 * then SiLU, the q | k | v split, the q / k L2 norm and the gates exactly as gdn_prepare does
 * for the same token; the window then becomes (win[1], win[2], x[n][c]) in place. Requires
 * total_tokens == num_seqs (one token each).
 *   mixed_qkv   [N][conv_dim]              in_dtype
 *   conv_window [N][conv_dim][3]           in_dtype, read and overwritten
 *   conv_weight [conv_dim][4], conv_bias [conv_dim] or NULL   in_dtype
 *   a, b        [N][H_v] in_dtype           A_log, dt_bias [H_v] fp32
 *   q, k (out)  [N][H_qk][d_k] qkv_dtype   v (out) [N][H_v][d_v] qkv_dtype
 *   g, beta (out) [N][H_v] fp32
 * mixed_qkv, conv_window, conv_weight, conv_bias (when given), q, k and v must be 16-byte
 * aligned (GDN_ERR_INVALID_ARGUMENT otherwise). Followed by gdn_recurrent_step on the same
 * stream this is a whole decode step from projected inputs (gdn_decode_step fuses the two).
 */
gdn_status_t gdn_decode_prepare(const gdn_shape_t* shape, const void* mixed_qkv,
                                void* conv_window, const void* conv_weight,
                                const void* conv_bias, const void* a, const void* b,
                                const float* A_log, const float* dt_bias, float l2norm_eps,
                                void* q, void* k, void* v, float* g, float* beta, void* stream);

/*
 * gdn_decode_step -- one decode token per sequence from projected inputs, fused: the front end
 * of gdn_decode_prepare (conv over the cached window, SiLU, split, q / k L2 norm, gates; the
 * window shifted in place) followed by the gated delta step of gdn_recurrent_step on the state,
 * in one kernel ([xiwon notes] "Cache"; [MoE report] §3.3 stages 2 and 3, decode path). q, k and
 * v stay fp32 between the two (shape->qkv_dtype is ignored), so the result equals the two-call
 * path with fp32 q/k/v up to fp32 rounding. Requires total_tokens == num_seqs; one workgroup
 * holds the q, k and G = H_v / H_qk v rows of a QK head, so (2 + G) * d_v + 2 G floats must fit
 * in 64 KiB (GDN_ERR_UNSUPPORTED otherwise).
 *   mixed_qkv, conv_window, conv_weight, conv_bias, a, b, A_log, dt_bias: as gdn_decode_prepare
 *   state [N][H_v][d_k][d_v] state_dtype, updated in place    o (out) [N][H_v][d_v] out_dtype
 * mixed_qkv, conv_window, conv_weight, conv_bias (when given) and state must be 16-byte aligned
 * (GDN_ERR_INVALID_ARGUMENT otherwise). The window and the state of a sequence must not be
 * shared with another sequence of the same call.
 */
gdn_status_t gdn_decode_step(const gdn_shape_t* shape, const void* mixed_qkv, void* conv_window,
                             const void* conv_weight, const void* conv_bias, const void* a,
                             const void* b, const float* A_log, const float* dt_bias,
                             float l2norm_eps, void* state, void* o, void* stream);

/*
 * gdn_gated_rmsnorm -- output gate of the layer ([xiwon notes] "Qwen3_5MoeGatedDeltaNet",
 * output stage; [MoE report] §3.3 stage 4): per V-head vector of d_v values,
 *   out_j = o_j / sqrt(mean_j o^2 + eps) * factor_j * z_j * sigmoid(z_j),
 *   factor_j = weight[j] + weight_offset, or 1 when weight is NULL
 * ([MoE report] §7.5 gives the model's RMSNorm weight the (1 + w) form, i.e. weight_offset 1;
 * the gated norm's form is not stated, so it is a parameter).
 *   o   [T][H_v][d_v] out_dtype (the core output)    z [T][H_v][d_v] in_dtype
 *   weight [d_v] fp32 or NULL                        out [T][H_v][d_v] out_dtype (may equal o)
 * o, z, out and weight (when given) must be 16-byte aligned; eps >= 0.
 */
gdn_status_t gdn_gated_rmsnorm(const gdn_shape_t* shape, const void* o, const void* z,
                               const float* weight, float weight_offset, float eps, void* out,
                               void* stream);

/*
 * gdn_recurrent_step_gated -- gdn_recurrent_step with the layer's output gate applied in the
 * same kernel ([xiwon notes] "Qwen3_5MoeGatedDeltaNet", output stage; [MoE report] §3.3 stages
 * 3 and 4): the step's fp32 output row o of each (sequence, V head) is never stored; instead
 *   out_j = o_j / sqrt(mean_j o^2 + norm_eps) * factor_j * z_j * sigmoid(z_j),
 *   factor_j = norm_weight[j] + weight_offset, or 1 when norm_weight is NULL,
 * as gdn_gated_rmsnorm computes it from a stored o (here without o's rounding to out_dtype).
 * One workgroup holds a head's whole row, so the mean square needs no second pass.
 *   q, k, v, g, beta, state: as gdn_recurrent_step
 *   z     [N][H_v][d_v] in_dtype (the gate projection), 16-byte aligned
 *   norm_weight [d_v] fp32 or NULL, 16-byte aligned     norm_eps >= 0, weight_offset finite
 *   out   [N][H_v][d_v] out_dtype
 * GDN_ERR_INVALID_ARGUMENT for a NULL z, a bad in_dtype, a misaligned z / weight / state, a
 * negative or NaN norm_eps or a NaN weight_offset, and everything gdn_recurrent_step rejects.
 */
gdn_status_t gdn_recurrent_step_gated(const gdn_shape_t* shape, const void* q, const void* k,
                                      const void* v, const float* g, const float* beta,
                                      void* state, const void* z, const float* norm_weight,
                                      float weight_offset, float norm_eps, void* out,
                                      void* stream);

/*
 * gdn_decode_step_gated -- gdn_decode_step (front end + gated delta step, one kernel) with the
 * output gate of gdn_recurrent_step_gated applied to each V head's row before it is written:
 * one decode token per sequence from projected inputs to the gated mixer output. Arguments as
 * gdn_decode_step, plus z [N][H_v][d_v] in_dtype, norm_weight [d_v] fp32 or NULL,
 * weight_offset and norm_eps as above, and out [N][H_v][d_v] out_dtype. The workgroup of a QK
 * head also holds its G z rows and the d_v factors in LDS: (3 + 2 G) * d_v + 2 G floats must
 * fit in 64 KiB (GDN_ERR_UNSUPPORTED otherwise).
 */
gdn_status_t gdn_decode_step_gated(const gdn_shape_t* shape, const void* mixed_qkv,
                                   void* conv_window, const void* conv_weight,
                                   const void* conv_bias, const void* a, const void* b,
                                   const float* A_log, const float* dt_bias, float l2norm_eps,
                                   void* state, const void* z, const float* norm_weight,
                                   float weight_offset, float norm_eps, void* out, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* gdn_status_string(gdn_status_t status);

/* GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
