// gdn_front.hpp -- per-thread pieces of the front end ([MoE report] §3.3 stage 2; [xiwon notes]
// "Qwen3_5MoeGatedDeltaNet" and "Cache") shared by the prefill front end, the decode-side front
// end and the fused decode step, so that the three compute the same fp32 arithmetic.
#pragma once

#include "gdn_device.hpp"

namespace gdn {

// softplus(x) = log(1 + e^x) without overflow; sigmoid(x) = 1 / (1 + e^-x); fp32.
__device__ __forceinline__ float softplus_f32(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}
__device__ __forceinline__ float sigmoid_f32(float x) { return 1.f / (1.f + expf(-x)); }

// Conv bias of channels c .. c+7, zeros without a bias. One unconditional 16-byte load (from
// `fallback`, any readable 16-byte-aligned address, when there is no bias) and a select on the
// values: a per-element conditional load compiles to eight dependent loads, and a branch around
// the load makes the compiler wait for every load in flight where the branches join.
template <typename InT>
__device__ __forceinline__ void load_bias8(const InT* bias, const InT* fallback, int c,
                                           float (&out)[8]) {
  Raw8<InT> r;
  r.load(bias ? bias + c : fallback);
  r.to(out);
  const bool has = bias != nullptr;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = has ? out[e] : 0.f;
}

// Decode-side convolution of the 8 channels c .. c+7 of one sequence: the new input (8 values),
// the window (3 previous inputs per channel, oldest first: 24 contiguous values) and the taps
// (4 per channel: 32 contiguous values, tap 3 multiplies the newest input), all as 16-byte loads
// issued before any use.
//   y = SiLU(bias + w0 win0 + w1 win1 + w2 win2 + w3 x)
// The window then becomes (win1, win2, x) per channel.
template <typename InT>
struct DecodeConv8 {
  Raw8<InT> rx, rw[3], rt[4], rb;
  bool has_bias;

  // x, win3 and taps point at channel c of the input row, the window row and the tap table.
  __device__ __forceinline__ void load(const InT* x, const InT* win3, const InT* taps,
                                       const InT* bias_base, int c) {
    rx.load_nt(x);  // the input and the window are touched once
#pragma unroll
    for (int j = 0; j < 3; ++j) rw[j].load_nt(win3 + 8 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) rt[j].load(taps + 8 * j);
    // bias: one unconditional load (from the taps without a bias) and a select on the values
    rb.load(bias_base ? bias_base + c : taps);
    has_bias = bias_base != nullptr;
  }

  // Values by flat index, converted where used (keeps only the raw 16-byte pieces live).
  __device__ __forceinline__ float win(int i) const { return rw[i / 8].at(i % 8); }
  __device__ __forceinline__ float tap(int i) const { return rt[i / 8].at(i % 8); }

  // y = SiLU(conv); returns the sum of squares of the 8 outputs.
  __device__ __forceinline__ float conv_silu(float (&y)[8]) const {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = has_bias ? rb.at(e) : 0.f;
      acc = fmaf(tap(4 * e + 0), win(3 * e + 0), acc);
      acc = fmaf(tap(4 * e + 1), win(3 * e + 1), acc);
      acc = fmaf(tap(4 * e + 2), win(3 * e + 2), acc);
      acc = fmaf(tap(4 * e + 3), rx.at(e), acc);
      y[e] = acc / (1.f + expf(-acc));
      ss = fmaf(y[e], y[e], ss);
    }
    return ss;
  }

  // Writes (win1, win2, x) per channel back to the window row: stored values moved, not
  // recomputed, so the shift is exact.
#define GDN_SHIFTED(f) ((f) % 3 == 2 ? rx.raw((f) / 3) : rw[((f) + 1) / 8].raw(((f) + 1) % 8))
  __device__ __forceinline__ void store_shifted_window(InT* win3) const {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      InT t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = GDN_SHIFTED(8 * j + i);
      store8_raw_nt(win3 + 8 * j, t8);
    }
  }
#undef GDN_SHIFTED
};

}  // namespace gdn
