// gdn_decode.hip -- one decode token per sequence: gated delta rule step on the stored state,
// updated in place ([MoE report] §3.3 stage 3, decode path; [xiwon notes]
// "Qwen3_5MoeGatedDeltaNet" recurrent branch and "Cache").
//
// Per (sequence n, V head h), with the state H [d_k][d_v] and a = exp(g):
//   kv = H^T k,  qh = H^T q,  qk = q . k           (one pass over the old state)
//   u  = beta (v - a kv)                             (error against the decayed state)
//   H' = a H + k u^T                                 (written back in place)
//   o  = scale (a qh + qk u)  = scale H'^T q          (no second pass over the state)
//
// The step moves 2 * d_k * d_v * sizeof(state) bytes of state per head and does ~7 d_k d_v
// flops, so it is bound by HBM. One workgroup owns one head (columns could be split across
// workgroups, but then every load covers 128-byte pieces of rows instead of whole rows, which
// streams slower): thread (cg, rg) keeps one 16-byte column group cg (4 fp32 or 8 bf16 values)
// for rows rg, rg + RG, ... in registers between the read and the write, so every state byte
// crosses HBM exactly once each way. A wave's load instruction covers whole contiguous rows
// (coalesced 16-byte lanes); loads and stores are non-temporal since the state is not reused by
// this step. The row reductions run over lanes first (xor shuffles across the row groups of a
// wave), then over waves through LDS. A bf16 state is read exactly, carried in fp32 through the
// step and stored as the round-to-nearest-even cast of the new fp32 state.
// decode_step_kernel below is the same step fused with the decode-side front end.
#include "gdn_device.hpp"
#include "gdn_front.hpp"
#include "gdn_internal.h"

namespace gdn {
namespace {

// Threads per workgroup. fp32 state: 512 for 128 x 128 heads (8 rows of 16 bytes per thread:
// enough loads in flight per wave without limiting occupancy), fewer for small heads. bf16
// state: also 8 rows of 16 bytes per thread (256 threads for 128 x 128), at least one wave; with
// 512 threads each thread would hold half the bytes and the CU too few loads in flight.
template <typename ST, int D>
constexpr int step_threads() {
  if constexpr (sizeof(ST) == 4) return D * D / 8 < 512 ? D * D / 8 : 512;
  return D * D / 64 > 64 ? D * D / 64 : 64;
}

// 16 bytes of one state row: 4 fp32 or 8 bf16 values.
template <typename ST>
struct StateVec;
template <>
struct StateVec<float> {
  static constexpr int VEC = 4;
  f32x4 r;
  __device__ __forceinline__ void load(const float* p) {
    r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  }
  __device__ __forceinline__ float at(int c) const { return r[c]; }
  __device__ __forceinline__ static void store(float* p, const float (&x)[VEC]) {
    f32x4 v = {x[0], x[1], x[2], x[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
  }
};
template <>
struct StateVec<bf16> {
  static constexpr int VEC = 8;
  bf16x8 r;
  __device__ __forceinline__ void load(const bf16* p) {
    r = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
  }
  __device__ __forceinline__ float at(int c) const { return (float)r[c]; }
  __device__ __forceinline__ static void store(bf16* p, const float (&x)[VEC]) {
    bf16x8 v;
#pragma unroll
    for (int c = 0; c < VEC; ++c) v[c] = (bf16)x[c];  // round to nearest even
    __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
  }
};

// Thread layout of one D x D head over NTH threads.
template <typename ST, int D>
struct StepLayout {
  static constexpr int NTH = step_threads<ST, D>();
  static constexpr int NW = NTH / 64;
  static constexpr int VEC = StateVec<ST>::VEC;
  static constexpr int CG = D / VEC;    // 16-byte column groups per row
  static constexpr int RG = NTH / CG;   // row groups
  static constexpr int R = D / RG;      // rows per thread
  static_assert(D % VEC == 0 && NTH % 64 == 0 && 64 % CG == 0 && D % RG == 0 && R >= 1,
                "tile shape");
};

// LDS for the cross-wave reductions of one head.
template <typename ST, int D>
struct StepRed {
  using L = StepLayout<ST, D>;
  float k[L::NW][L::CG][L::VEC];
  float q[L::NW][L::CG][L::VEC];
  float qk[L::NW];
};

// The step of one head whose rows the thread holds in s[0 .. R) (registers of the caller, which
// loaded them; the call is inlined). qrow / krow give q and k at the thread's rows (index r),
// vcol the v value of column c of its group. Writes o (threads of row group 0) and the new
// state; the barrier inside is workgroup-wide.
// Output gate fused into the step: out_j = o_j / sqrt(mean_j o^2 + eps) * fac_j * SiLU(z_j) over
// the d_v columns of the head ([xiwon notes] "Qwen3_5MoeGatedDeltaNet", output stage). The
// workgroup holds the whole row, so the mean square is a shuffle reduction over the lanes of
// one row group. z is read as in_dtype (bf16 when z_bf16), the weight (or null: factor 1) as
// fp32.
struct OutGate {
  const void* z;  // [N][H_v][d_v], null: no gate (o is written)
  const float* w;
  float woff, eps;
  int z_bf16;
};

// z of one row and the factors into LDS (D values each; threads 0 .. D - 1 of the caller).
template <int D>
__device__ __forceinline__ void gate_to_lds(const OutGate& ga, size_t row, float* zs, float* fs,
                                            int tid) {
  if (tid < D) {
    zs[tid] = ga.z_bf16 ? (float)static_cast<const bf16*>(ga.z)[row + tid]
                        : static_cast<const float*>(ga.z)[row + tid];
    if (fs) fs[tid] = ga.w ? ga.w[tid] + ga.woff : 1.f;
  }
}

template <typename ST, typename OutT, int D, bool GATE, typename QF, typename KF, typename VF>
__device__ __forceinline__ void head_step(const StateVec<ST>* s, StepRed<ST, D>& red, QF qrow,
                                          KF krow, VF vcol,
                                          float alpha, float bt, float scale, ST* S, OutT* ov,
                                          int tid, const float* zs = nullptr,
                                          const float* fs = nullptr, float geps = 0.f) {
  using L = StepLayout<ST, D>;
  constexpr int VEC = L::VEC, CG = L::CG, RG = L::RG, R = L::R, NW = L::NW;
  const int cg = tid % CG, rg = tid / CG, lane = tid & 63, wave = tid >> 6;
  float pk[VEC], pq[VEC], pqk = 0.f;
#pragma unroll
  for (int c = 0; c < VEC; ++c) pk[c] = pq[c] = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float qr = qrow(r), kr = krow(r);
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      pk[c] = fmaf(s[r].at(c), kr, pk[c]);
      pq[c] = fmaf(s[r].at(c), qr, pq[c]);
    }
    pqk = fmaf(qr, kr, pqk);
  }
  // Lanes cg, cg + CG, ... of a wave hold the same columns for different rows.
#pragma unroll
  for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      pk[c] += __shfl_xor(pk[c], off);
      pq[c] += __shfl_xor(pq[c], off);
    }
    pqk += __shfl_xor(pqk, off);
  }
  if (lane < CG) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      red.k[wave][lane][c] = pk[c];
      red.q[wave][lane][c] = pq[c];
    }
    if (lane == 0) red.qk[wave] = pqk;
  }
  __syncthreads();
  float qk = red.qk[0], u[VEC], oc[VEC];
#pragma unroll
  for (int w = 1; w < NW; ++w) qk += red.qk[w];
#pragma unroll
  for (int c = 0; c < VEC; ++c) {
    float skc = red.k[0][cg][c], sqc = red.q[0][cg][c];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      skc += red.k[w][cg][c];
      sqc += red.q[w][cg][c];
    }
    u[c] = bt * (vcol(c) - alpha * skc);
    oc[c] = scale * (alpha * sqc + qk * u[c]);
    if constexpr (!GATE) {
      if (rg == 0) ov[VEC * cg + c] = from_f32<OutT>(oc[c]);
    }
  }
  if constexpr (GATE) {
    // every row group holds the whole row: the CG lanes of one group reduce it (z and the
    // factors were put in LDS before the barrier above)
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < VEC; ++c) ss = fmaf(oc[c], oc[c], ss);
#pragma unroll
    for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off);
    const float inv = 1.f / sqrtf(ss * (1.f / D) + geps);
    if (rg == 0) {
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const float zc = zs[VEC * cg + c];
        ov[VEC * cg + c] = from_f32<OutT>(oc[c] * inv * fs[VEC * cg + c] * (zc / (1.f + expf(-zc))));
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float kr = krow(r);
    float nv[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) nv[c] = fmaf(s[r].at(c), alpha, u[c] * kr);
    StateVec<ST>::store(S + (size_t)(rg + RG * r) * D + VEC * cg, nv);
  }
}

template <typename InT, typename OutT, typename ST, int D, bool GATE>
__global__ __launch_bounds__((step_threads<ST, D>())) void recurrent_step_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, ST* __restrict__ state,
    OutT* __restrict__ o, int hqk, int hv, float scale, OutGate ga) {
  using L = StepLayout<ST, D>;
  __shared__ StepRed<ST, D> red;

  const int nh = blockIdx.x;  // n * hv + h
  const int n = nh / hv, h = nh - (nh / hv) * hv;
  const int m = h / (hv / hqk);
  const int tid = threadIdx.x, cg = tid % L::CG, rg = tid / L::CG;

  ST* S = state + (size_t)nh * D * D;
  StateVec<ST> s[L::R];
#pragma unroll
  for (int r = 0; r < L::R; ++r) s[r].load(S + (size_t)(rg + L::RG * r) * D + L::VEC * cg);

  const InT* qv = q + ((size_t)n * hqk + m) * D;
  const InT* kv = k + ((size_t)n * hqk + m) * D;
  float qi[L::R], ki[L::R];
#pragma unroll
  for (int r = 0; r < L::R; ++r) {
    qi[r] = to_f32(qv[rg + L::RG * r]);
    ki[r] = to_f32(kv[rg + L::RG * r]);
  }
  const InT* vv = v + (size_t)nh * D + L::VEC * cg;
  __shared__ float gzs[GATE ? D : 1], gfs[GATE ? D : 1];
  if constexpr (GATE) gate_to_lds<D>(ga, (size_t)nh * D, gzs, gfs, tid);
  head_step<ST, OutT, D, GATE>(
      s, red, [&](int r) { return qi[r]; }, [&](int r) { return ki[r]; },
      [&](int c) { return to_f32(vv[c]); }, expf(g[nh]), beta[nh], scale, S, o + (size_t)nh * D,
      tid, gzs, gfs, ga.eps);
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
  OutGate gate;  // z null: no output gate
  const void* x;
  void* win;
  const void* w;
  const void* bias;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  float eps;
  void* state;
  void* o;
  int hqk, hv;
  float scale;
};

// fp32 state: at least 4 waves per SIMD (<= 128 VGPRs), two 512-thread workgroups per CU as for
// the plain step. bf16 state (256-thread workgroups): at least 3 (<= 168 VGPRs, no spills).
template <typename InT, typename OutT, typename ST, int D, bool GATE>
__global__ __launch_bounds__((step_threads<ST, D>()))
__attribute__((amdgpu_waves_per_eu(sizeof(ST) == 4 ? 4 : 3, 8))) void decode_step_kernel(
    DecStepParams p) {
  using L = StepLayout<ST, D>;
  constexpr int NTH = L::NTH;
  constexpr int CGN = D / 8;  // front-end threads per channel head (8 channels each)
  static_assert(NTH % CGN == 0, "front-end lane groups");

  // q[D] | k[D] | v[G][D] | alpha[G] | beta[G], then with the output gate z[G][D] | factors[D]
  extern __shared__ float lds[];
  __shared__ StepRed<ST, D> red[2];

  const int G = p.hv / p.hqk;
  const int nm = blockIdx.x;  // n * hqk + m
  const int n = nm / p.hqk, m = nm - n * p.hqk;
  const int h0 = m * G;
  const int tid = threadIdx.x, cg = tid % L::CG, rg = tid / L::CG;
  float* sq = lds;
  float* sk = lds + D;
  float* sv = lds + 2 * D;
  float* s_alpha = lds + (2 + G) * D;
  float* s_beta = s_alpha + G;
  float* s_z = s_beta + G;
  float* s_f = s_z + G * D;

  ST* const state = static_cast<ST*>(p.state);
  auto state_of = [&](int j) { return state + ((size_t)n * p.hv + h0 + j) * D * D; };
  StateVec<ST> s[L::R];
  {
    const ST* S = state_of(0);
#pragma unroll
    for (int r = 0; r < L::R; ++r) s[r].load(S + (size_t)(rg + L::RG * r) * D + L::VEC * cg);
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
  if constexpr (GATE) {
    for (int j = 0; j < G; ++j)
      gate_to_lds<D>(p.gate, ((size_t)n * p.hv + h0 + j) * D, s_z + j * D, j == 0 ? s_f : nullptr,
                     tid);
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
  // The reduction buffers alternate between heads: one barrier per head.
  for (int j = 0; j < G; ++j) {
    ST* S = state_of(j);
    const float* vj = sv + j * D + L::VEC * cg;
    head_step<ST, OutT, D, GATE>(
        s, red[j & 1], [&](int r) { return sq[rg + L::RG * r]; },
        [&](int r) { return sk[rg + L::RG * r]; }, [&](int c) { return vj[c]; }, s_alpha[j],
        s_beta[j], p.scale, S, static_cast<OutT*>(p.o) + ((size_t)n * p.hv + h0 + j) * D, tid,
        s_z + j * D, s_f, p.gate.eps);
    if (j + 1 < G) {  // the next head's rows into the same registers
      const ST* Sn = state_of(j + 1);
#pragma unroll
      for (int r = 0; r < L::R; ++r) s[r].load(Sn + (size_t)(rg + L::RG * r) * D + L::VEC * cg);
    }
  }
}

template <typename InT, typename OutT, typename ST, int D>
hipError_t launch_decode_step_t(const gdn_shape_t& s, const DecStepParams& p,
                                hipStream_t stream) {
  const unsigned blocks = (unsigned)s.num_seqs * (unsigned)s.num_qk_heads;
  if (blocks == 0) return hipSuccess;
  const int G = s.num_v_heads / s.num_qk_heads;
  const size_t lds =
      (size_t)((2 + G) * D + 2 * G + (p.gate.z ? (G + 1) * D : 0)) * sizeof(float);
  if (p.gate.z)
    hipLaunchKernelGGL((decode_step_kernel<InT, OutT, ST, D, true>), dim3(blocks),
                       dim3(step_threads<ST, D>()), lds, stream, p);
  else
    hipLaunchKernelGGL((decode_step_kernel<InT, OutT, ST, D, false>), dim3(blocks),
                       dim3(step_threads<ST, D>()), lds, stream, p);
  return hipGetLastError();
}

template <typename InT, typename OutT, typename ST>
hipError_t launch_decode_step_d(const gdn_shape_t& s, const DecStepParams& p,
                                hipStream_t stream) {
  switch (s.head_dim_k) {
    case 32: return launch_decode_step_t<InT, OutT, ST, 32>(s, p, stream);
    case 64: return launch_decode_step_t<InT, OutT, ST, 64>(s, p, stream);
    case 128: return launch_decode_step_t<InT, OutT, ST, 128>(s, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename InT, typename OutT>
hipError_t launch_decode_step_s(const gdn_shape_t& s, const DecStepParams& p,
                                hipStream_t stream) {
  return s.state_dtype == GDN_DTYPE_BF16 ? launch_decode_step_d<InT, OutT, bf16>(s, p, stream)
                                         : launch_decode_step_d<InT, OutT, float>(s, p, stream);
}

template <typename InT, typename OutT, typename ST, int D>
hipError_t launch_step_t(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, void* state, void* o,
                         const OutGate& ga, hipStream_t stream) {
  const unsigned blocks = (unsigned)s.num_seqs * (unsigned)s.num_v_heads;
  if (blocks == 0) return hipSuccess;
  if (ga.z)
    hipLaunchKernelGGL((recurrent_step_kernel<InT, OutT, ST, D, true>), dim3(blocks),
                       dim3(step_threads<ST, D>()), 0, stream,
                       static_cast<const InT*>(q), static_cast<const InT*>(k),
                       static_cast<const InT*>(v), g, beta, static_cast<ST*>(state),
                       static_cast<OutT*>(o), s.num_qk_heads, s.num_v_heads, s.scale, ga);
  else
    hipLaunchKernelGGL((recurrent_step_kernel<InT, OutT, ST, D, false>), dim3(blocks),
                       dim3(step_threads<ST, D>()), 0, stream,
                       static_cast<const InT*>(q), static_cast<const InT*>(k),
                       static_cast<const InT*>(v), g, beta, static_cast<ST*>(state),
                       static_cast<OutT*>(o), s.num_qk_heads, s.num_v_heads, s.scale, ga);
  return hipGetLastError();
}

template <typename InT, typename OutT, typename ST>
hipError_t launch_step_d(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, void* state, void* o,
                         const OutGate& ga, hipStream_t stream) {
  switch (s.head_dim_k) {
    case 32: return launch_step_t<InT, OutT, ST, 32>(s, q, k, v, g, beta, state, o, ga, stream);
    case 64: return launch_step_t<InT, OutT, ST, 64>(s, q, k, v, g, beta, state, o, ga, stream);
    case 128: return launch_step_t<InT, OutT, ST, 128>(s, q, k, v, g, beta, state, o, ga, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename InT, typename OutT>
hipError_t launch_step_s(const gdn_shape_t& s, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, void* state, void* o,
                         const OutGate& ga, hipStream_t stream) {
  return s.state_dtype == GDN_DTYPE_BF16
             ? launch_step_d<InT, OutT, bf16>(s, q, k, v, g, beta, state, o, ga, stream)
             : launch_step_d<InT, OutT, float>(s, q, k, v, g, beta, state, o, ga, stream);
}

}  // namespace

hipError_t launch_decode_step(const gdn_shape_t& s, const void* x, void* window, const void* w,
                              const void* bias, const void* a, const void* b, const float* A_log,
                              const float* dt_bias, float eps, void* state, void* o,
                              hipStream_t stream, const void* gate_z, const float* gate_w,
                              float gate_woff, float gate_eps) {
  const OutGate ga{gate_z, gate_w, gate_woff, gate_eps, s.in_dtype == GDN_DTYPE_BF16 ? 1 : 0};
  DecStepParams p{ga, x, window, w, bias, a, b, A_log, dt_bias, eps, state, o,
                  s.num_qk_heads, s.num_v_heads, s.scale};
  const bool in_bf16 = s.in_dtype == GDN_DTYPE_BF16, out_bf16 = s.out_dtype == GDN_DTYPE_BF16;
  if (in_bf16 && out_bf16) return launch_decode_step_s<bf16, bf16>(s, p, stream);
  if (in_bf16) return launch_decode_step_s<bf16, float>(s, p, stream);
  if (out_bf16) return launch_decode_step_s<float, bf16>(s, p, stream);
  return launch_decode_step_s<float, float>(s, p, stream);
}

hipError_t launch_recurrent_step(const gdn_shape_t& s, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta, void* state,
                                 void* o, hipStream_t stream, const void* gate_z,
                                 const float* gate_w, float gate_woff, float gate_eps) {
  const OutGate ga{gate_z, gate_w, gate_woff, gate_eps, s.in_dtype == GDN_DTYPE_BF16 ? 1 : 0};
  const bool in_bf16 = s.qkv_dtype == GDN_DTYPE_BF16, out_bf16 = s.out_dtype == GDN_DTYPE_BF16;
  if (in_bf16 && out_bf16) return launch_step_s<bf16, bf16>(s, q, k, v, g, beta, state, o, ga, stream);
  if (in_bf16) return launch_step_s<bf16, float>(s, q, k, v, g, beta, state, o, ga, stream);
  if (out_bf16) return launch_step_s<float, bf16>(s, q, k, v, g, beta, state, o, ga, stream);
  return launch_step_s<float, float>(s, q, k, v, g, beta, state, o, ga, stream);
}

}  // namespace gdn
