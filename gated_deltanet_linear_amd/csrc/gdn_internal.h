// gdn_internal.h -- launchers shared between the ABI layer and the kernel sources.
// Host code only; every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/gdn.h"

namespace gdn {

hipError_t launch_chunk_intra(const gdn_shape_t& s, const int32_t* cu, const void* q,
                              const void* k, const float* g, const float* beta, void* ws,
                              hipStream_t stream);

hipError_t launch_chunk_scan(const gdn_shape_t& s, const int32_t* cu, const void* q,
                             const void* k, const void* v, const void* h0, void* o, void* ht,
                             const void* ws, hipStream_t stream);

// The many-chain layout of the scan for bf16 q/k/v (gdn_scan_tiles.hip).
hipError_t launch_chunk_scan_tiles(const gdn_shape_t& s, const int32_t* cu, const void* q,
                                   const void* k, const void* v, const void* h0, void* o,
                                   void* ht, const void* ws, hipStream_t stream);

// gate_z non-null: the output gate out = RMSNorm(o) (gate_w + gate_woff) SiLU(gate_z) is applied
// in the step's epilogue and written to o (z in shape in_dtype, gate_w fp32 or null).
hipError_t launch_recurrent_step(const gdn_shape_t& s, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta, void* state,
                                 void* o, hipStream_t stream, const void* gate_z = nullptr,
                                 const float* gate_w = nullptr, float gate_woff = 0.f,
                                 float gate_eps = 0.f);

hipError_t launch_prepare(const gdn_shape_t& s, const int32_t* cu, const void* x,
                          const void* w, const void* bias, const void* a, const void* b,
                          const float* A_log, const float* dt_bias, float eps, void* q, void* k,
                          void* v, float* g, float* beta, hipStream_t stream);

hipError_t launch_decode_prepare(const gdn_shape_t& s, const void* x, void* window,
                                 const void* w, const void* bias, const void* a, const void* b,
                                 const float* A_log, const float* dt_bias, float eps, void* q,
                                 void* k, void* v, float* g, float* beta, hipStream_t stream);

hipError_t launch_decode_step(const gdn_shape_t& s, const void* x, void* window, const void* w,
                              const void* bias, const void* a, const void* b, const float* A_log,
                              const float* dt_bias, float eps, void* state, void* o,
                              hipStream_t stream, const void* gate_z = nullptr,
                              const float* gate_w = nullptr, float gate_woff = 0.f,
                              float gate_eps = 0.f);

hipError_t launch_gated_rmsnorm(const gdn_shape_t& s, const void* o, const void* z,
                                const float* w, float w_offset, float eps, void* out,
                                hipStream_t stream);

// Backward pass of the chunked form (gdn_backward.hip): workspace size in floats, and launch.
long long chunk_backward_workspace_floats(const gdn_shape_t& s);
hipError_t launch_chunk_backward(const gdn_shape_t& s, const int32_t* cu, const void* q,
                                 const void* k, const void* v, const float* g, const float* beta,
                                 const void* h0, const void* dout, const void* dht, void* dq,
                                 void* dk, void* dv, float* dg, float* dbeta, void* dh0, void* ws,
                                 hipStream_t stream);

// Device address and size of the calling thread's current device's copy of the workspace array
// of gdn_chunk_forward_noalloc (gdn_noalloc.hip); the address is looked up once per device.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Bytes of one workspace record (one chunk slot x one V head); the layout is private to
// gdn_chunk.hip, which checks this value at compile time.
constexpr long long kWorkspaceRecordBytes = 20992;

// Number of chunk slots the workspace holds: num_seqs + total_tokens / 64.
inline long long chunk_slots(const gdn_shape_t& s) {
  return (long long)s.num_seqs + (long long)s.total_tokens / 64;
}

}  // namespace gdn
