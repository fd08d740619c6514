// gdn_abi.cpp -- the extern "C" entry points of libgdn.so: host-side validation, then the
// kernel launchers. Validation never touches the GPU, so every error path can be exercised
// on a machine without one. See include/gdn.h for the contract of each call.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

bool dtype_ok(int32_t d) { return d == GDN_DTYPE_F32 || d == GDN_DTYPE_BF16; }

// Shape checks shared by all entry points. `split_ok`: the call accepts GDN_DTYPE_F32_SPLIT as
// its qkv_dtype (the front end and the chunked prefill).
gdn_status_t check_shape(const gdn_shape_t* s, bool split_ok = false) {
  if (s == nullptr) return GDN_ERR_INVALID_ARGUMENT;
  if (s->num_seqs < 1 || s->total_tokens < 0 || s->num_qk_heads < 1 || s->num_v_heads < 1)
    return GDN_ERR_INVALID_ARGUMENT;
  if (s->num_v_heads % s->num_qk_heads != 0) return GDN_ERR_INVALID_ARGUMENT;
  const bool qkv_ok = dtype_ok(s->qkv_dtype) || (split_ok && s->qkv_dtype == GDN_DTYPE_F32_SPLIT);
  if (!qkv_ok || !dtype_ok(s->out_dtype) || !dtype_ok(s->state_dtype))
    return GDN_ERR_INVALID_ARGUMENT;
  if (s->head_dim_k < 1 || s->head_dim_v < 1) return GDN_ERR_INVALID_ARGUMENT;
  if (!(s->scale == s->scale)) return GDN_ERR_INVALID_ARGUMENT;  // NaN
  if (s->head_dim_k != s->head_dim_v) return GDN_ERR_UNSUPPORTED;
  if (s->head_dim_k != 32 && s->head_dim_k != 64 && s->head_dim_k != 128) return GDN_ERR_UNSUPPORTED;
  // Index arithmetic inside the kernels is 64-bit for element offsets and 32-bit for token
  // and head counts; keep element counts of one tensor and slot counts within range.
  const long long rows = (long long)s->total_tokens * s->num_v_heads;
  if (rows > (1LL << 31) - 1) return GDN_ERR_UNSUPPORTED;
  if ((long long)s->num_seqs * s->num_v_heads > (1LL << 31) - 1) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

gdn_status_t from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Output-gate arguments shared by the gated decode entry points.
gdn_status_t check_gate(const gdn_shape_t* s, const void* z, const float* weight,
                        float weight_offset, float eps) {
  if (!dtype_ok(s->in_dtype)) return GDN_ERR_INVALID_ARGUMENT;
  if (!z || !(eps >= 0.f) || !(weight_offset == weight_offset)) return GDN_ERR_INVALID_ARGUMENT;
  if (!aligned(z, 16) || !aligned(weight, 16)) return GDN_ERR_INVALID_ARGUMENT;
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status_t status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT: bad shape, dtype or pointer";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: shape not compiled into this library";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "GDN_ERR_WORKSPACE_TOO_SMALL";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: a kernel launch failed";
    case GDN_ERR_SCRATCH_LIMIT:
      return "GDN_ERR_SCRATCH_LIMIT: the shape needs more workspace than the no-allocation "
             "entry point's device array holds";
  }
  return "unknown gdn_status_t";
}

size_t gdn_chunk_forward_workspace_size(const gdn_shape_t* s) {
  if (check_shape(s, true) != GDN_OK) return 0;
  return (size_t)gdn::chunk_slots(*s) * (size_t)s->num_v_heads *
         (size_t)gdn::kWorkspaceRecordBytes;
}

gdn_status_t gdn_prepare(const gdn_shape_t* s, const int32_t* cu, const void* x, const void* w,
                         const void* bias, const void* a, const void* b, const float* A_log,
                         const float* dt_bias, float eps, void* q, void* k, void* v, float* g,
                         float* beta, void* stream) {
  gdn_status_t st = check_shape(s, true);
  if (st != GDN_OK) return st;
  if (!dtype_ok(s->in_dtype)) return GDN_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.f)) return GDN_ERR_INVALID_ARGUMENT;
  if (!cu || !A_log || !dt_bias) return GDN_ERR_INVALID_ARGUMENT;
  if (s->total_tokens > 0 && (!x || !w || !a || !b || !q || !k || !v || !g || !beta))
    return GDN_ERR_INVALID_ARGUMENT;
  // 16-byte vector access of mixed_qkv / q / k / v rows, the conv bias and the gate arrays.
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(a, 16) || !aligned(b, 16) || !aligned(g, 16) || !aligned(beta, 16) ||
      !aligned(bias, 16))
    return GDN_ERR_INVALID_ARGUMENT;
  return from_hip(gdn::launch_prepare(*s, cu, x, w, bias, a, b, A_log, dt_bias, eps, q, k, v, g,
                                      beta, static_cast<hipStream_t>(stream)));
}

static gdn_status_t check_chunk_common(const gdn_shape_t* s, const int32_t* cu, const void* q,
                                       const void* k, const void* ws, size_t ws_bytes) {
  gdn_status_t st = check_shape(s, true);
  if (st != GDN_OK) return st;
  if (!cu) return GDN_ERR_INVALID_ARGUMENT;
  if (s->total_tokens > 0 && (!q || !k || !ws)) return GDN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(ws, 256)) return GDN_ERR_INVALID_ARGUMENT;
  if (ws_bytes < gdn_chunk_forward_workspace_size(s)) return GDN_ERR_WORKSPACE_TOO_SMALL;
  return GDN_OK;
}

gdn_status_t gdn_chunk_intra(const gdn_shape_t* s, const int32_t* cu, const void* q,
                             const void* k, const float* g, const float* beta, void* ws,
                             size_t ws_bytes, void* stream) {
  gdn_status_t st = check_chunk_common(s, cu, q, k, ws, ws_bytes);
  if (st != GDN_OK) return st;
  if (s->total_tokens > 0 && (!g || !beta)) return GDN_ERR_INVALID_ARGUMENT;
  return from_hip(gdn::launch_chunk_intra(*s, cu, q, k, g, beta, ws,
                                          static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_chunk_scan(const gdn_shape_t* s, const int32_t* cu, const void* q,
                            const void* k, const void* v, const void* h0, void* o, void* ht,
                            const void* ws, size_t ws_bytes, void* stream) {
  gdn_status_t st = check_chunk_common(s, cu, q, k, ws, ws_bytes);
  if (st != GDN_OK) return st;
  if (s->total_tokens > 0 && (!v || !o)) return GDN_ERR_INVALID_ARGUMENT;
  // v rows are loaded and o rows stored with 16-byte accesses.
  if (!aligned(v, 16) || !aligned(o, 16)) return GDN_ERR_INVALID_ARGUMENT;
  return from_hip(gdn::launch_chunk_scan(*s, cu, q, k, v, h0, o, ht, ws,
                                         static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_chunk_forward(const gdn_shape_t* s, const int32_t* cu, const void* q,
                               const void* k, const void* v, const float* g, const float* beta,
                               const void* h0, void* o, void* ht, void* ws, size_t ws_bytes,
                               void* stream) {
  gdn_status_t st = check_chunk_common(s, cu, q, k, ws, ws_bytes);
  if (st != GDN_OK) return st;
  if (s->total_tokens > 0 && (!v || !o || !g || !beta)) return GDN_ERR_INVALID_ARGUMENT;
  if (!aligned(v, 16) || !aligned(o, 16)) return GDN_ERR_INVALID_ARGUMENT;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = from_hip(gdn::launch_chunk_intra(*s, cu, q, k, g, beta, ws, hs));
  if (st != GDN_OK) return st;
  return from_hip(gdn::launch_chunk_scan(*s, cu, q, k, v, h0, o, ht, ws, hs));
}

gdn_status_t gdn_chunk_forward_noalloc(const gdn_shape_t* s, const int32_t* cu, const void* q,
                                       const void* k, const void* v, const float* g,
                                       const float* beta, const void* h0, void* o, void* ht,
                                       void* stream) {
  // The same checks as gdn_chunk_forward (with the library's array standing in for the
  // workspace), and the size limit, before any HIP call.
  gdn_status_t st = check_shape(s, true);
  if (st != GDN_OK) return st;
  if (gdn_chunk_forward_workspace_size(s) > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
    return GDN_ERR_SCRATCH_LIMIT;
  if (!cu) return GDN_ERR_INVALID_ARGUMENT;
  if (s->total_tokens > 0 && (!q || !k || !v || !o || !g || !beta))
    return GDN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return GDN_ERR_INVALID_ARGUMENT;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (gdn::noalloc_scratch(&ws, &ws_bytes) != hipSuccess) return GDN_ERR_HIP;
  return gdn_chunk_forward(s, cu, q, k, v, g, beta, h0, o, ht, ws, ws_bytes, stream);
}

size_t gdn_chunk_backward_workspace_size(const gdn_shape_t* s) {
  if (check_shape(s) != GDN_OK) return 0;
  return (size_t)gdn::chunk_backward_workspace_floats(*s) * sizeof(float);
}

gdn_status_t gdn_chunk_backward(const gdn_shape_t* s, const int32_t* cu, const void* q,
                                const void* k, const void* v, const float* g, const float* beta,
                                const void* h0, const void* dout, const void* dht, void* dq,
                                void* dk, void* dv, float* dg, float* dbeta, void* dh0,
                                void* ws, size_t ws_bytes, void* stream) {
  gdn_status_t st = check_shape(s);
  if (st != GDN_OK) return st;
  if (!cu || !ws) return GDN_ERR_INVALID_ARGUMENT;
  if (s->total_tokens > 0 &&
      (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta))
    return GDN_ERR_INVALID_ARGUMENT;
  if (!aligned(ws, 256)) return GDN_ERR_INVALID_ARGUMENT;
  // Rows of q, k, v, dout and of the gradients are read and written with 8- and 16-byte
  // vector accesses.
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return GDN_ERR_INVALID_ARGUMENT;
  if (ws_bytes < gdn_chunk_backward_workspace_size(s)) return GDN_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(gdn::launch_chunk_backward(*s, cu, q, k, v, g, beta, h0, dout, dht, dq, dk, dv,
                                             dg, dbeta, dh0, ws,
                                             static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_recurrent_step(const gdn_shape_t* s, const void* q, const void* k,
                                const void* v, const float* g, const float* beta, void* state,
                                void* o, void* stream) {
  gdn_status_t st = check_shape(s);
  if (st != GDN_OK) return st;
  if (s->total_tokens != s->num_seqs) return GDN_ERR_INVALID_ARGUMENT;
  if (!q || !k || !v || !g || !beta || !state || !o) return GDN_ERR_INVALID_ARGUMENT;
  if (!aligned(state, 16)) return GDN_ERR_INVALID_ARGUMENT;
  return from_hip(gdn::launch_recurrent_step(*s, q, k, v, g, beta, state, o,
                                             static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_recurrent_step_gated(const gdn_shape_t* s, const void* q, const void* k,
                                      const void* v, const float* g, const float* beta,
                                      void* state, const void* z, const float* norm_weight,
                                      float weight_offset, float norm_eps, void* out,
                                      void* stream) {
  gdn_status_t st = check_shape(s);
  if (st != GDN_OK) return st;
  if (s->total_tokens != s->num_seqs) return GDN_ERR_INVALID_ARGUMENT;
  if (!q || !k || !v || !g || !beta || !state || !out) return GDN_ERR_INVALID_ARGUMENT;
  if (!aligned(state, 16)) return GDN_ERR_INVALID_ARGUMENT;
  st = check_gate(s, z, norm_weight, weight_offset, norm_eps);
  if (st != GDN_OK) return st;
  return from_hip(gdn::launch_recurrent_step(*s, q, k, v, g, beta, state, out,
                                             static_cast<hipStream_t>(stream), z, norm_weight,
                                             weight_offset, norm_eps));
}

gdn_status_t gdn_decode_prepare(const gdn_shape_t* s, const void* x, void* win, const void* w,
                                const void* bias, const void* a, const void* b,
                                const float* A_log, const float* dt_bias, float eps, void* q,
                                void* k, void* v, float* g, float* beta, void* stream) {
  gdn_status_t st = check_shape(s);
  if (st != GDN_OK) return st;
  if (!dtype_ok(s->in_dtype)) return GDN_ERR_INVALID_ARGUMENT;
  if (s->total_tokens != s->num_seqs) return GDN_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.f)) return GDN_ERR_INVALID_ARGUMENT;
  if (!x || !win || !w || !a || !b || !A_log || !dt_bias || !q || !k || !v || !g || !beta)
    return GDN_ERR_INVALID_ARGUMENT;
  // 16-byte vector access of the input row, the window, the taps, the bias and the q / k / v
  // rows.
  if (!aligned(x, 16) || !aligned(win, 16) || !aligned(w, 16) || !aligned(q, 16) ||
      !aligned(k, 16) || !aligned(v, 16) || !aligned(bias, 16))
    return GDN_ERR_INVALID_ARGUMENT;
  return from_hip(gdn::launch_decode_prepare(*s, x, win, w, bias, a, b, A_log, dt_bias, eps, q, k,
                                             v, g, beta, static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_decode_step(const gdn_shape_t* s, const void* x, void* win, const void* w,
                             const void* bias, const void* a, const void* b, const float* A_log,
                             const float* dt_bias, float eps, void* state, void* o,
                             void* stream) {
  gdn_status_t st = check_shape(s);
  if (st != GDN_OK) return st;
  if (!dtype_ok(s->in_dtype)) return GDN_ERR_INVALID_ARGUMENT;
  if (s->total_tokens != s->num_seqs) return GDN_ERR_INVALID_ARGUMENT;
  // q, k and the G v rows of a workgroup's QK head are held in LDS: at most 64 KiB.
  const long long G = s->num_v_heads / s->num_qk_heads;
  if (((2 + G) * s->head_dim_v + 2 * G) * 4 > 65536) return GDN_ERR_UNSUPPORTED;
  if (!(eps >= 0.f)) return GDN_ERR_INVALID_ARGUMENT;
  if (!x || !win || !w || !a || !b || !A_log || !dt_bias || !state || !o)
    return GDN_ERR_INVALID_ARGUMENT;
  // 16-byte vector access of the input row, the window, the taps, the bias and the state.
  if (!aligned(x, 16) || !aligned(win, 16) || !aligned(w, 16) || !aligned(bias, 16) ||
      !aligned(state, 16))
    return GDN_ERR_INVALID_ARGUMENT;
  return from_hip(gdn::launch_decode_step(*s, x, win, w, bias, a, b, A_log, dt_bias, eps, state,
                                          o, static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_decode_step_gated(const gdn_shape_t* s, const void* x, void* win, const void* w,
                                   const void* bias, const void* a, const void* b,
                                   const float* A_log, const float* dt_bias, float eps,
                                   void* state, const void* z, const float* norm_weight,
                                   float weight_offset, float norm_eps, void* out, void* stream) {
  gdn_status_t st = check_shape(s);
  if (st != GDN_OK) return st;
  if (!dtype_ok(s->in_dtype)) return GDN_ERR_INVALID_ARGUMENT;
  if (s->total_tokens != s->num_seqs) return GDN_ERR_INVALID_ARGUMENT;
  // q, k, the G v rows and z rows of a workgroup's QK head and the factors are held in LDS
  const long long G = s->num_v_heads / s->num_qk_heads;
  if (((3 + 2 * G) * s->head_dim_v + 2 * G) * 4 > 65536) return GDN_ERR_UNSUPPORTED;
  if (!(eps >= 0.f)) return GDN_ERR_INVALID_ARGUMENT;
  if (!x || !win || !w || !a || !b || !A_log || !dt_bias || !state || !out)
    return GDN_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(win, 16) || !aligned(w, 16) || !aligned(bias, 16) ||
      !aligned(state, 16))
    return GDN_ERR_INVALID_ARGUMENT;
  st = check_gate(s, z, norm_weight, weight_offset, norm_eps);
  if (st != GDN_OK) return st;
  return from_hip(gdn::launch_decode_step(*s, x, win, w, bias, a, b, A_log, dt_bias, eps, state,
                                          out, static_cast<hipStream_t>(stream), z, norm_weight,
                                          weight_offset, norm_eps));
}

gdn_status_t gdn_gated_rmsnorm(const gdn_shape_t* s, const void* o, const void* z,
                               const float* weight, float weight_offset, float eps, void* out,
                               void* stream) {
  gdn_status_t st = check_shape(s);
  if (st != GDN_OK) return st;
  if (!dtype_ok(s->in_dtype)) return GDN_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.f) || !(weight_offset == weight_offset)) return GDN_ERR_INVALID_ARGUMENT;
  if (s->total_tokens > 0 && (!o || !z || !out)) return GDN_ERR_INVALID_ARGUMENT;
  if (!aligned(o, 16) || !aligned(z, 16) || !aligned(out, 16) || !aligned(weight, 16))
    return GDN_ERR_INVALID_ARGUMENT;
  return from_hip(gdn::launch_gated_rmsnorm(*s, o, z, weight, weight_offset, eps, out,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
