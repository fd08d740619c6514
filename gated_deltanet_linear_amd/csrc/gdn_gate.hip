// gdn_gate.hip -- output gate of the layer: RMSNorm of the core output times SiLU of the gate
// projection z, per V-head vector ([xiwon notes] "Qwen3_5MoeGatedDeltaNet", output stage: the
// core output and z are reshaped to rows of head_v_dim and normed together; [MoE report] §3.3
// stage 4; §7.5 for the (1 + w) weight form of the model's RMSNorm):
//   out_j = o_j / sqrt(mean_j o^2 + eps) * factor_j * z_j * sigmoid(z_j),
//   factor_j = w_j + w_offset (1 without a weight).
// One HBM pass over o and z. A thread owns 8 consecutive values of a row (one 16-byte bf16
// access); the D / 8 threads of a row are adjacent lanes and reduce with xor shuffles; each
// thread issues the loads of its two rows before using the first. Two rows per thread keep the
// kernel under 64 VGPRs (8 waves per SIMD); four rows (68 VGPRs, 7 waves) left a short second
// round of workgroups and ran 1.5x slower on the 4096 x 32 x 128 shape. Reads and writes carry
// the nontemporal hint: each byte is touched once.
#include "gdn_device.hpp"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kGateRowsPerThread = 2;

template <typename OT, typename ZT, int D>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const OT* __restrict__ o,
                                                            const ZT* __restrict__ z,
                                                            const float* __restrict__ w,
                                                            float w_offset, float eps,
                                                            OT* __restrict__ out, long long rows) {
  constexpr int TPR = D / 8;    // threads per row
  constexpr int RPP = 256 / TPR;  // rows per pass of the workgroup
  constexpr int RPT = kGateRowsPerThread;
  const int tid = threadIdx.x, cg = tid % TPR, rin = tid / TPR;
  const long long row0 = (long long)blockIdx.x * RPP * RPT + rin;

  // The weight slice first, as two 16-byte loads under one uniform branch (a per-element
  // select would wait for every outstanding load once per element).
  float f[8];
  if (w) {
    Raw8<float> rw;
    rw.load(w + 8 * cg);
    rw.to(f);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] += w_offset;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = 1.f;
  }
  Raw8<OT> ro[RPT];
  Raw8<ZT> rz[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const long long row = min(row0 + (long long)u * RPP, rows - 1);  // in range; not stored
    ro[u].load_nt(o + row * D + 8 * cg);
    rz[u].load_nt(z + row * D + 8 * cg);
  }

#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const long long row = row0 + (long long)u * RPP;
    float x[8], g[8];
    ro[u].to(x);
    rz[u].to(g);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
    for (int d = 1; d < TPR; d <<= 1) ss += __shfl_xor(ss, d, kWave);
    const float inv = 1.f / sqrtf(ss * (1.f / D) + eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[e] * inv * f[e] * (g[e] / (1.f + expf(-g[e])));
    if (row < rows) store8_nt(out + row * D + 8 * cg, y);
  }
}

template <typename OT, typename ZT, int D>
hipError_t launch_gate_t(long long rows, const void* o, const void* z, const float* w,
                         float w_offset, float eps, void* out, hipStream_t stream) {
  constexpr int per_block = 256 / (D / 8) * kGateRowsPerThread;
  const unsigned blocks = (unsigned)((rows + per_block - 1) / per_block);
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL((gated_rmsnorm_kernel<OT, ZT, D>), dim3(blocks), dim3(256), 0, stream,
                     static_cast<const OT*>(o), static_cast<const ZT*>(z), w, w_offset, eps,
                     static_cast<OT*>(out), rows);
  return hipGetLastError();
}

template <typename OT, typename ZT>
hipError_t launch_gate_d(int d, long long rows, const void* o, const void* z, const float* w,
                         float w_offset, float eps, void* out, hipStream_t stream) {
  switch (d) {
    case 32: return launch_gate_t<OT, ZT, 32>(rows, o, z, w, w_offset, eps, out, stream);
    case 64: return launch_gate_t<OT, ZT, 64>(rows, o, z, w, w_offset, eps, out, stream);
    case 128: return launch_gate_t<OT, ZT, 128>(rows, o, z, w, w_offset, eps, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gated_rmsnorm(const gdn_shape_t& s, const void* o, const void* z,
                                const float* w, float w_offset, float eps, void* out,
                                hipStream_t stream) {
  const long long rows = (long long)s.total_tokens * s.num_v_heads;
  const bool o_bf = s.out_dtype == GDN_DTYPE_BF16, z_bf = s.in_dtype == GDN_DTYPE_BF16;
  const int d = s.head_dim_v;
  if (o_bf && z_bf) return launch_gate_d<bf16, bf16>(d, rows, o, z, w, w_offset, eps, out, stream);
  if (o_bf) return launch_gate_d<bf16, float>(d, rows, o, z, w, w_offset, eps, out, stream);
  if (z_bf) return launch_gate_d<float, bf16>(d, rows, o, z, w, w_offset, eps, out, stream);
  return launch_gate_d<float, float>(d, rows, o, z, w, w_offset, eps, out, stream);
}

}  // namespace gdn
