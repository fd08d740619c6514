// gdn_decode.hip -- one decode token per sequence: gated delta rule step on the fp32 state,
// updated in place ([MoE report] §3.3 stage 3, decode path; [xiwon notes]
// "Qwen3_5MoeGatedDeltaNet" recurrent branch and "Cache").
//
// Per (sequence n, V head h), with the state H [d_k][d_v] and a = exp(g):
//   kv = H^T k,  qh = H^T q,  qk = q . k           (one pass over the old state)
//   u  = beta (v - a kv)                             (error against the decayed state)
//   H' = a H + k u^T                                 (written back in place)
//   o  = scale (a qh + qk u)  = scale H'^T q          (no second pass over the state)
//
// The step moves 2 * d_k * d_v * 4 bytes of state per head and does ~7 d_k d_v flops, so it is
// bound by HBM. One 256-thread workgroup owns one head: thread (cg, rg) keeps a float4 column
// group cg for rows rg, rg + RG, ... in registers between the read and the write, so every
// state byte crosses HBM exactly once each way. A wave's load instruction covers whole
// contiguous rows (coalesced 16-byte lanes); loads and stores are non-temporal since the state
// is not reused by this step.
#include "gdn_device.hpp"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename InT, typename OutT, int DK, int DV>
__global__ __launch_bounds__(256) void recurrent_step_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    OutT* __restrict__ o, int hqk, int hv, float scale) {
  constexpr int CG = DV / 4;    // float4 column groups per row
  constexpr int RG = 256 / CG;  // row groups
  constexpr int R = DK / RG;    // rows per thread
  static_assert(DV % 4 == 0 && 256 % CG == 0 && DK % RG == 0 && R >= 1, "tile shape");

  __shared__ f32x4 red_k[RG][CG];
  __shared__ f32x4 red_q[RG][CG];
  __shared__ float red_qk[RG];
  __shared__ f32x4 u_sh[CG];

  const int nh = blockIdx.x;  // n * hv + h
  const int n = nh / hv, h = nh - (nh / hv) * hv;
  const int m = h / (hv / hqk);
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;

  f32x4* S = reinterpret_cast<f32x4*>(state + (size_t)nh * DK * DV);
  const InT* qv = q + ((size_t)n * hqk + m) * DK;
  const InT* kv = k + ((size_t)n * hqk + m) * DK;

  f32x4 s[R];
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = __builtin_nontemporal_load(S + (rg + RG * r) * CG + cg);

  float qi[R], ki[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    qi[r] = to_f32(qv[rg + RG * r]);
    ki[r] = to_f32(kv[rg + RG * r]);
  }
  const float alpha = expf(g[nh]);
  const float bt = beta[nh];

  f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
  float pqk = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pk += s[r] * ki[r];
    pq += s[r] * qi[r];
    pqk += qi[r] * ki[r];
  }
  red_k[rg][cg] = pk;
  red_q[rg][cg] = pq;
  if (cg == 0) red_qk[rg] = pqk;
  __syncthreads();

  if (rg == 0) {
    f32x4 sk = red_k[0][cg], sq = red_q[0][cg];
#pragma unroll
    for (int j = 1; j < RG; ++j) {
      sk += red_k[j][cg];
      sq += red_q[j][cg];
    }
    float qk = 0.f;
#pragma unroll
    for (int j = 0; j < RG; ++j) qk += red_qk[j];
    const InT* vv = v + (size_t)nh * DV + 4 * cg;
    f32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = bt * (to_f32(vv[c]) - alpha * sk[c]);
    u_sh[cg] = u;
    OutT* ov = o + (size_t)nh * DV + 4 * cg;
#pragma unroll
    for (int c = 0; c < 4; ++c) ov[c] = from_f32<OutT>(scale * (alpha * sq[c] + qk * u[c]));
  }
  __syncthreads();

  const f32x4 u = u_sh[cg];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    f32x4 nv = s[r] * alpha + u * ki[r];
    __builtin_nontemporal_store(nv, S + (rg + RG * r) * CG + cg);
  }
}

template <typename InT, typename OutT, int D>
hipError_t launch_step_t(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float* state, void* o,
                         hipStream_t stream) {
  const unsigned blocks = (unsigned)s.num_seqs * (unsigned)s.num_v_heads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((recurrent_step_kernel<InT, OutT, D, D>), dim3(blocks), dim3(256), 0, stream,
                     static_cast<const InT*>(q), static_cast<const InT*>(k),
                     static_cast<const InT*>(v), g, beta, state, static_cast<OutT*>(o),
                     s.num_qk_heads, s.num_v_heads, s.scale);
  return hipGetLastError();
}

template <typename InT, typename OutT>
hipError_t launch_step_d(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float* state, void* o,
                         hipStream_t stream) {
  switch (s.head_dim_k) {
    case 32: return launch_step_t<InT, OutT, 32>(s, q, k, v, g, beta, state, o, stream);
    case 64: return launch_step_t<InT, OutT, 64>(s, q, k, v, g, beta, state, o, stream);
    case 128: return launch_step_t<InT, OutT, 128>(s, q, k, v, g, beta, state, o, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_recurrent_step(const gdn_shape_t& s, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta, float* state,
                                 void* o, hipStream_t stream) {
  const bool in_bf16 = s.qkv_dtype == GDN_DTYPE_BF16, out_bf16 = s.out_dtype == GDN_DTYPE_BF16;
  if (in_bf16 && out_bf16) return launch_step_d<bf16, bf16>(s, q, k, v, g, beta, state, o, stream);
  if (in_bf16) return launch_step_d<bf16, float>(s, q, k, v, g, beta, state, o, stream);
  if (out_bf16) return launch_step_d<float, bf16>(s, q, k, v, g, beta, state, o, stream);
  return launch_step_d<float, float>(s, q, k, v, g, beta, state, o, stream);
}

}  // namespace gdn
