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
// bound by HBM. One workgroup owns one head (columns could be split across workgroups, but
// then every load covers 128-byte pieces of rows instead of whole rows, which streams slower):
// thread (cg, rg) keeps a float4 column group cg for rows rg, rg + RG, ... in registers between
// the read and the write, so every state byte crosses HBM exactly once each way. A wave's load
// instruction covers whole contiguous rows (coalesced 16-byte lanes); loads and stores are
// non-temporal since the state is not reused by this step. The row reductions run over lanes
// first (xor shuffles across the row groups of a wave), then over waves through LDS.
// decode_step_kernel below is the same step fused with the decode-side front end.
#include "gdn_device.hpp"
#include "gdn_front.hpp"
#include "gdn_internal.h"

namespace gdn {
namespace {

// Threads per workgroup: 512 for 128 x 128 heads (8 rows per thread: enough loads in flight
// per wave without limiting occupancy), fewer for small heads (at least 2 rows per thread).
template <int DK, int DV>
constexpr int step_threads() {
  return DK * DV / 8 < 512 ? DK * DV / 8 : 512;
}

template <typename InT, typename OutT, int DK, int DV>
__global__ __launch_bounds__((step_threads<DK, DV>())) void recurrent_step_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    OutT* __restrict__ o, int hqk, int hv, float scale) {
  constexpr int NTH = step_threads<DK, DV>();
  constexpr int NW = NTH / 64;  // waves
  constexpr int CG = DV / 4;    // float4 column groups per row
  constexpr int RG = NTH / CG;  // row groups
  constexpr int R = DK / RG;    // rows per thread
  static_assert(DV % 4 == 0 && NTH % 64 == 0 && 64 % CG == 0 && DK % RG == 0 && R >= 1,
                "tile shape");

  __shared__ f32x4 red_k[NW][CG];
  __shared__ f32x4 red_q[NW][CG];
  __shared__ float red_qk[NW];

  const int nh = blockIdx.x;  // n * hv + h
  const int n = nh / hv, h = nh - (nh / hv) * hv;
  const int m = h / (hv / hqk);
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG, lane = tid & 63, wave = tid >> 6;

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
  // Lanes cg, cg + CG, ... of a wave hold the same columns for different rows.
#pragma unroll
  for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pk[c] += __shfl_xor(pk[c], off);
      pq[c] += __shfl_xor(pq[c], off);
    }
    pqk += __shfl_xor(pqk, off);
  }
  if (lane < CG) {
    red_k[wave][lane] = pk;
    red_q[wave][lane] = pq;
    if (lane == 0) red_qk[wave] = pqk;
  }
  __syncthreads();

  f32x4 sk = red_k[0][cg], sq = red_q[0][cg];
  float qk = red_qk[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    sk += red_k[w][cg];
    sq += red_q[w][cg];
    qk += red_qk[w];
  }
  const InT* vv = v + (size_t)nh * DV + 4 * cg;
  f32x4 u;
#pragma unroll
  for (int c = 0; c < 4; ++c) u[c] = bt * (to_f32(vv[c]) - alpha * sk[c]);
  if (rg == 0) {
    OutT* ov = o + (size_t)nh * DV + 4 * cg;
#pragma unroll
    for (int c = 0; c < 4; ++c) ov[c] = from_f32<OutT>(scale * (alpha * sq[c] + qk * u[c]));
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    f32x4 nv = s[r] * alpha + u * ki[r];
    __builtin_nontemporal_store(nv, S + (rg + RG * r) * CG + cg);
  }
}

// ---- fused decode step from projected inputs --------------------------------------------
// One workgroup per (sequence n, QK head m) runs the decode-side front end of the channels that
// group needs -- q and k of head m, v of its G V heads, and their gates -- and then the gated
// delta step of those G V heads in turn. The q/k channels' conv window is read and shifted by
// this workgroup alone, so the in-place window update needs no ordering between workgroups.
// The first head's state loads are issued before the front end (it overlaps with them); each
// next head's rows are loaded into the same registers once the current head's are written back
// (a second register set would halve the workgroups per CU). q, k and v stay fp32 (in LDS)
// between the front end and the step.
struct DecStepParams {
  const void* x;
  void* win;
  const void* w;
  const void* bias;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  float eps;
  float* state;
  void* o;
  int hqk, hv;
  float scale;
};

// At least 4 waves per SIMD (<= 128 VGPRs): two 512-thread workgroups per CU, as for the plain
// step.
template <typename InT, typename OutT, int D>
__global__ __launch_bounds__((step_threads<D, D>())) __attribute__((amdgpu_waves_per_eu(4, 8)))
void decode_step_kernel(DecStepParams p) {
  constexpr int NTH = step_threads<D, D>();
  constexpr int NW = NTH / 64;
  constexpr int CG = D / 4;    // float4 column groups per state row
  constexpr int RG = NTH / CG;  // row groups
  constexpr int R = D / RG;     // state rows per thread
  constexpr int CGN = D / 8;    // front-end threads per channel head (8 channels each)
  static_assert(NTH % 64 == 0 && 64 % CG == 0 && D % RG == 0 && R >= 1 && NTH % CGN == 0,
                "tile shape");

  extern __shared__ float lds[];  // q[D] | k[D] | v[G][D] | alpha[G] | beta[G]
  __shared__ f32x4 red_k[2][NW][CG];
  __shared__ f32x4 red_q[2][NW][CG];
  __shared__ float red_qk[2][NW];

  const int G = p.hv / p.hqk;
  const int nm = blockIdx.x;  // n * hqk + m
  const int n = nm / p.hqk, m = nm - n * p.hqk;
  const int h0 = m * G;
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG, lane = tid & 63, wave = tid >> 6;
  float* sq = lds;
  float* sk = lds + D;
  float* sv = lds + 2 * D;
  float* s_alpha = lds + (2 + G) * D;
  float* s_beta = s_alpha + G;

  auto state_of = [&](int j) {
    return reinterpret_cast<f32x4*>(p.state + ((size_t)n * p.hv + h0 + j) * D * D);
  };
  f32x4 s[R];
  {
    const f32x4* S = state_of(0);
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = __builtin_nontemporal_load(S + (rg + RG * r) * CG + cg);
  }

  // Front end. Channel head hb: 0 = q of head m, 1 = k of head m, 2 + j = v of V head h0 + j.
  const int conv_dim = (2 * p.hqk + p.hv) * D;
  for (int t = tid; t < (2 + G) * CGN; t += NTH) {  // whole CGN-lane groups stay together
    const int hb = t / CGN, ci = t - hb * CGN;
    const int c = (hb == 0 ? m * D : hb == 1 ? (p.hqk + m) * D : (2 * p.hqk + h0 + hb - 2) * D) +
                  8 * ci;
    InT* W3 = static_cast<InT*>(p.win) + ((size_t)n * conv_dim + c) * 3;
    DecodeConv8<InT> cv;
    cv.load(static_cast<const InT*>(p.x) + (size_t)n * conv_dim + c, W3,
            static_cast<const InT*>(p.w) + (size_t)c * 4, static_cast<const InT*>(p.bias), c);
    float y[8];
    float ss = cv.conv_silu(y);
#pragma unroll
    for (int d = 1; d < CGN; d <<= 1) ss += __shfl_xor(ss, d, kWave);  // lanes of one head
    if (hb < 2) {
      const float inv = 1.f / sqrtf(ss + p.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= inv;
    }
    float* dst = lds + hb * D + 8 * ci;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = y[e];
    cv.store_shifted_window(W3);
  }
  for (int j = tid; j < G; j += NTH) {
    const size_t i = (size_t)n * p.hv + h0 + j;
    const float ga = -expf(p.A_log[h0 + j]) *
                     softplus_f32(to_f32(static_cast<const InT*>(p.a)[i]) + p.dt_bias[h0 + j]);
    s_alpha[j] = expf(ga);
    s_beta[j] = sigmoid_f32(to_f32(static_cast<const InT*>(p.b)[i]));
  }
  __syncthreads();

  // q and k of the thread's rows are read from LDS where used (registers go to the state).
  for (int j = 0; j < G; ++j) {
    const int buf = j & 1;  // reductions double-buffered: one barrier per head
    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
    float pqk = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float qr = sq[rg + RG * r], kr = sk[rg + RG * r];
      pk += s[r] * kr;
      pq += s[r] * qr;
      pqk += qr * kr;
    }
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pk[c] += __shfl_xor(pk[c], off);
        pq[c] += __shfl_xor(pq[c], off);
      }
      pqk += __shfl_xor(pqk, off);
    }
    if (lane < CG) {
      red_k[buf][wave][lane] = pk;
      red_q[buf][wave][lane] = pq;
      if (lane == 0) red_qk[buf][wave] = pqk;
    }
    __syncthreads();
    f32x4 skv = red_k[buf][0][cg], sqv = red_q[buf][0][cg];
    float qk = red_qk[buf][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      skv += red_k[buf][w][cg];
      sqv += red_q[buf][w][cg];
      qk += red_qk[buf][w];
    }
    const float alpha = s_alpha[j], bt = s_beta[j];
    f32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = bt * (sv[j * D + 4 * cg + c] - alpha * skv[c]);
    if (rg == 0) {
      OutT* ov = static_cast<OutT*>(p.o) + ((size_t)n * p.hv + h0 + j) * D + 4 * cg;
#pragma unroll
      for (int c = 0; c < 4; ++c) ov[c] = from_f32<OutT>(p.scale * (alpha * sqv[c] + qk * u[c]));
    }
    f32x4* S = state_of(j);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      f32x4 nv = s[r] * alpha + u * sk[rg + RG * r];
      __builtin_nontemporal_store(nv, S + (rg + RG * r) * CG + cg);
    }
    if (j + 1 < G) {  // the next head's rows into the same registers
      const f32x4* Sn = state_of(j + 1);
#pragma unroll
      for (int r = 0; r < R; ++r) s[r] = __builtin_nontemporal_load(Sn + (rg + RG * r) * CG + cg);
    }
  }
}

template <typename InT, typename OutT, int D>
hipError_t launch_decode_step_t(const gdn_shape_t& s, const DecStepParams& p,
                                hipStream_t stream) {
  const unsigned blocks = (unsigned)s.num_seqs * (unsigned)s.num_qk_heads;
  if (blocks == 0) return hipSuccess;
  const int G = s.num_v_heads / s.num_qk_heads;
  const size_t lds = (size_t)((2 + G) * D + 2 * G) * sizeof(float);
  hipLaunchKernelGGL((decode_step_kernel<InT, OutT, D>), dim3(blocks), dim3(step_threads<D, D>()),
                     lds, stream, p);
  return hipGetLastError();
}

template <typename InT, typename OutT>
hipError_t launch_decode_step_d(const gdn_shape_t& s, const DecStepParams& p,
                                hipStream_t stream) {
  switch (s.head_dim_k) {
    case 32: return launch_decode_step_t<InT, OutT, 32>(s, p, stream);
    case 64: return launch_decode_step_t<InT, OutT, 64>(s, p, stream);
    case 128: return launch_decode_step_t<InT, OutT, 128>(s, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename InT, typename OutT, int D>
hipError_t launch_step_t(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float* state, void* o,
                         hipStream_t stream) {
  const unsigned blocks = (unsigned)s.num_seqs * (unsigned)s.num_v_heads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((recurrent_step_kernel<InT, OutT, D, D>), dim3(blocks),
                     dim3(step_threads<D, D>()), 0, stream,
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

hipError_t launch_decode_step(const gdn_shape_t& s, const void* x, void* window, const void* w,
                              const void* bias, const void* a, const void* b, const float* A_log,
                              const float* dt_bias, float eps, float* state, void* o,
                              hipStream_t stream) {
  DecStepParams p{x, window, w, bias, a, b, A_log, dt_bias, eps, state, o,
                  s.num_qk_heads, s.num_v_heads, s.scale};
  const bool in_bf16 = s.in_dtype == GDN_DTYPE_BF16, out_bf16 = s.out_dtype == GDN_DTYPE_BF16;
  if (in_bf16 && out_bf16) return launch_decode_step_d<bf16, bf16>(s, p, stream);
  if (in_bf16) return launch_decode_step_d<bf16, float>(s, p, stream);
  if (out_bf16) return launch_decode_step_d<float, bf16>(s, p, stream);
  return launch_decode_step_d<float, float>(s, p, stream);
}

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
