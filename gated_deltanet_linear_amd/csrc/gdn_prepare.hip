// gdn_prepare.hip -- front end of the Gated DeltaNet layer in one HBM-bound pass
// ([MoE report] §3.3 stage 2 and §3.5; [xiwon notes] "Qwen3_5MoeGatedDeltaNet"; [intro]
// "线性注意力").
//
//   y_t[c] = bias[c] + sum_{j=0..3} w[c][j] x_{t-3+j}[c]   (nn.Conv1d cross-correlation,
//            left padding 3, zero history before the first token of each packed sequence)
//   y      = SiLU(y) = y / (1 + e^-y)
//   q | k | v = split of the channels; q, k head vectors scaled by 1 / sqrt(sum y^2 + eps)
//   beta = sigmoid(b),  g = -exp(A_log) softplus(a + dt_bias)              (fp32)
//
// Grid: x = one channel head (H_qk q heads, H_qk k heads, H_v v heads) plus one extra row
// for the gates, y = blocks of 128 tokens. A thread owns 8 channels (one 16-byte bf16 load)
// and walks 128 * 8 / D consecutive tokens with a 3-row sliding window in registers, so each
// input row is fetched once per thread run (plus 3 rows of history at the run start). The
// D / 8 lanes that share a token are adjacent in the wave; the L2 norm reduces across them
// with lane shuffles.
#include "gdn_device.hpp"
#include "gdn_front.hpp"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kTokBlock = 128;

// Largest n in [0, num_seqs) with cu[n] <= t (the sequence holding token t < cu[num_seqs]).
__device__ __forceinline__ int token_to_seq(const int32_t* cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

struct PrepParams {
  const int32_t* cu;
  const void* x;
  const void* w;
  const void* bias;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  float eps;
  void* q;
  void* k;
  void* v;
  float* g;
  float* beta;
  int num_seqs, T, hqk, hv;
};

template <typename InT, typename QT, int D>
__global__ __launch_bounds__(256) void prepare_kernel(PrepParams p) {
  constexpr int CGN = D / 8;           // threads per token row of one head
  constexpr int TL = 256 / CGN;        // token lanes per workgroup
  constexpr int TPT = kTokBlock / TL;  // consecutive tokens per thread
  static_assert(D % 8 == 0 && 256 % CGN == 0 && kTokBlock % TL == 0, "tile shape");

  // Heads vary fastest over the grid, so that workgroups running together read and write whole
  // token rows (all heads of the same tokens) rather than one head's slice of many rows.
  const int hb = blockIdx.x;
  const int tid = threadIdx.x;
  const int tok0 = blockIdx.y * kTokBlock;
  const int head_blocks = 2 * p.hqk + p.hv;

  if (hb == head_blocks) {  // gates
    // The block's a / b values are one contiguous run of [128 tokens][H_v]: each thread takes
    // 8 consecutive elements per step, all loads issued before the first use.
    const InT* A = static_cast<const InT*>(p.a);
    const InT* B = static_cast<const InT*>(p.b);
    const size_t e0 = (size_t)tok0 * p.hv;
    const int ne = min(kTokBlock, p.T - tok0) * p.hv;  // elements of this block
    constexpr int KMAX = 8;                           // steps per pass (H_v <= 64 in one pass)
    for (int base = 0; base < ne; base += 8 * 256 * KMAX) {
      Raw8<InT> ra[KMAX], rb[KMAX];
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int e = base + 8 * (tid + 256 * k);
        if (e + 8 <= ne) {
          ra[k].load(A + e0 + e);
          rb[k].load(B + e0 + e);
        }
      }
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int e = base + 8 * (tid + 256 * k);
        if (e >= ne) break;
        float av[8], bv[8];
        if (e + 8 <= ne) {
          ra[k].to(av);
          rb[k].to(bv);
        } else {  // ragged end of the run (H_v * tokens not a multiple of 8)
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            av[u] = e + u < ne ? to_f32(A[e0 + e + u]) : 0.f;
            bv[u] = e + u < ne ? to_f32(B[e0 + e + u]) : 0.f;
          }
        }
        float gv[8], betav[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int h = (int)((e0 + e + u) % p.hv);
          betav[u] = sigmoid_f32(bv[u]);
          gv[u] = -expf(p.A_log[h]) * softplus_f32(av[u] + p.dt_bias[h]);
        }
        if (e + 8 <= ne) {
          store8(p.beta + e0 + e, betav);
          store8(p.g + e0 + e, gv);
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (e + u < ne) {
              p.beta[e0 + e + u] = betav[u];
              p.g[e0 + e + u] = gv[u];
            }
        }
      }
    }
    return;
  }

  const int cg = tid % CGN, tl = tid / CGN;
  const int conv_dim = 2 * p.hqk * D + p.hv * D;
  int cbase;
  QT* dst;
  int dst_stride;
  bool is_qk = true;
  if (hb < p.hqk) {
    cbase = hb * D;
    dst = static_cast<QT*>(p.q) + hb * D;
    dst_stride = p.hqk * D;
  } else if (hb < 2 * p.hqk) {
    cbase = p.hqk * D + (hb - p.hqk) * D;
    dst = static_cast<QT*>(p.k) + (hb - p.hqk) * D;
    dst_stride = p.hqk * D;
  } else {
    cbase = 2 * p.hqk * D + (hb - 2 * p.hqk) * D;
    dst = static_cast<QT*>(p.v) + (hb - 2 * p.hqk) * D;
    dst_stride = p.hv * D;
    is_qk = false;
  }
  const int c = cbase + 8 * cg;
  const InT* X = static_cast<const InT*>(p.x) + c;
  dst += 8 * cg;

  const int t_first = tok0 + tl * TPT;
  if (t_first >= p.T) return;  // whole token group idle (its CGN lanes leave together)

  // Every row of this thread's run and the 3 rows of history are loaded before anything else
  // (TPT + 3 loads in flight per thread); the sequence lookup below overlaps with them, and
  // history rows from before the sequence start are dropped where they would be used.
  Raw8<InT> hist[3], rows[TPT];
#pragma unroll
  for (int j = 0; j < 3; ++j) hist[j].load(X + (size_t)max(t_first - 3 + j, 0) * conv_dim);
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    // nontemporal, except the last 3 rows: the next token lane's run reads them as history
    const InT* row = X + (size_t)min(t_first + j, p.T - 1) * conv_dim;
    if (j < TPT - 3)
      rows[j].load_nt(row);
    else
      rows[j].load(row);
  }
  // Taps and bias after the rows, so that waiting for them does not hold back the row loads.
  float w[8][4], bias[8];
  {
    const InT* W = static_cast<const InT*>(p.w) + (size_t)c * 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int j = 0; j < 4; ++j) w[e][j] = to_f32(W[e * 4 + j]);
    }
    load_bias8(static_cast<const InT*>(p.bias), W, c, bias);
  }
  // The lookup is done for the block's first token: a uniform search runs on scalar loads,
  // which are counted apart from the row loads in flight (a per-lane search would wait for all
  // of them before each step). Lanes whose run starts in a later sequence step forward; only
  // blocks that hold a sequence start take that loop.
  int n = token_to_seq(p.cu, p.num_seqs, tok0);
  int seq_start = p.cu[n], seq_end = p.cu[n + 1];
  while (t_first >= seq_end) {
    ++n;
    seq_start = seq_end;
    seq_end = p.cu[n + 1];
  }
  float xm3[8], xm2[8], xm1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) xm3[e] = xm2[e] = xm1[e] = 0.f;
  if (t_first - 3 >= seq_start) hist[0].to(xm3);
  if (t_first - 2 >= seq_start) hist[1].to(xm2);
  if (t_first - 1 >= seq_start) hist[2].to(xm1);

#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const int t = t_first + j;
    if (t >= p.T) break;
    if (t >= seq_end) {  // a new sequence starts at t: no history
      while (t >= p.cu[n + 1]) ++n;
      seq_start = p.cu[n];
      seq_end = p.cu[n + 1];
#pragma unroll
      for (int e = 0; e < 8; ++e) xm3[e] = xm2[e] = xm1[e] = 0.f;
    }
    float x0[8], y[8];
    rows[j].to(x0);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = bias[e];
      acc = fmaf(w[e][0], xm3[e], acc);
      acc = fmaf(w[e][1], xm2[e], acc);
      acc = fmaf(w[e][2], xm1[e], acc);
      acc = fmaf(w[e][3], x0[e], acc);
      y[e] = acc / (1.f + expf(-acc));
      ss = fmaf(y[e], y[e], ss);
    }
    if (is_qk) {
#pragma unroll
      for (int d = 1; d < CGN; d <<= 1) ss += __shfl_xor(ss, d, kWave);
      const float inv = 1.f / sqrtf(ss + p.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= inv;
    }
    store8_nt(dst + (size_t)t * dst_stride, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xm3[e] = xm2[e];
      xm2[e] = xm1[e];
      xm1[e] = x0[e];
    }
  }
}

template <typename InT, typename QT, int D>
hipError_t launch_prepare_t(const PrepParams& p, hipStream_t stream) {
  const unsigned gx = (unsigned)(2 * p.hqk + p.hv + 1);
  const unsigned gy = (unsigned)((p.T + kTokBlock - 1) / kTokBlock);
  if (gy == 0) return hipSuccess;
  hipLaunchKernelGGL((prepare_kernel<InT, QT, D>), dim3(gx, gy), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename InT, typename QT>
hipError_t launch_prepare_d(const PrepParams& p, int d, hipStream_t stream) {
  switch (d) {
    case 32: return launch_prepare_t<InT, QT, 32>(p, stream);
    case 64: return launch_prepare_t<InT, QT, 64>(p, stream);
    case 128: return launch_prepare_t<InT, QT, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---- decode side: one token per sequence with a cached convolution window -----------------
// ([xiwon notes] "Cache": the conv state keeps the last inputs of each channel so that a decode
// step convolves without the history; [MoE report] §3.3 stage 2, decode path.) Per channel:
//   y = bias + w[0] win[0] + w[1] win[1] + w[2] win[2] + w[3] x,  then as above,
// and the window [3] (oldest first) becomes (win[1], win[2], x) in place.
// Grid: x = sequence, y = groups of 256 / (D / 8) channel heads, plus one row for the gates. A
// thread owns 8 channels: one 16-byte input access, three for its 24 window values, four for
// its 32 taps.

struct DecPrepParams {
  const void* x;
  void* win;
  const void* w;
  const void* bias;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  float eps;
  void* q;
  void* k;
  void* v;
  float* g;
  float* beta;
  int hqk, hv;
};

// At most 6 waves per SIMD: the 256-thread launch of 256 sequences fits in one round at that
// occupancy, and the register room lets all nine loads of a thread be issued before the first
// use (a tighter register target makes the compiler issue them one use at a time).
template <typename InT, typename QT, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 6))) void
decode_prepare_kernel(DecPrepParams p) {
  constexpr int CGN = D / 8;      // threads per channel head
  constexpr int HPW = 256 / CGN;  // channel heads per workgroup
  const int n = blockIdx.x, tid = threadIdx.x;
  const int head_blocks = 2 * p.hqk + p.hv;
  const int groups = (head_blocks + HPW - 1) / HPW;

  if ((int)blockIdx.y == groups) {  // gates of sequence n
    const InT* A = static_cast<const InT*>(p.a);
    const InT* B = static_cast<const InT*>(p.b);
    for (int h = tid; h < p.hv; h += 256) {
      const size_t i = (size_t)n * p.hv + h;
      p.beta[i] = sigmoid_f32(to_f32(B[i]));
      p.g[i] = -expf(p.A_log[h]) * softplus_f32(to_f32(A[i]) + p.dt_bias[h]);
    }
    return;
  }

  const int hb_raw = blockIdx.y * HPW + tid / CGN, cg = tid % CGN;
  const bool active = hb_raw < head_blocks;
  const int hb = active ? hb_raw : 0;  // idle lanes read head 0 and store nothing
  const int conv_dim = head_blocks * D;
  const int c = hb * D + 8 * cg;

  InT* W3 = static_cast<InT*>(p.win) + ((size_t)n * conv_dim + c) * 3;
  DecodeConv8<InT> cv;
  cv.load(static_cast<const InT*>(p.x) + (size_t)n * conv_dim + c, W3,
          static_cast<const InT*>(p.w) + (size_t)c * 4, static_cast<const InT*>(p.bias), c);
  float y[8];
  float ss = cv.conv_silu(y);
  const bool is_qk = hb < 2 * p.hqk;
#pragma unroll
  for (int d = 1; d < CGN; d <<= 1) ss += __shfl_xor(ss, d, kWave);  // lanes of one head
  if (is_qk) {
    const float inv = 1.f / sqrtf(ss + p.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] *= inv;
  }
  if (!active) return;
  QT* dst;
  if (hb < p.hqk) dst = static_cast<QT*>(p.q) + ((size_t)n * p.hqk + hb) * D;
  else if (hb < 2 * p.hqk) dst = static_cast<QT*>(p.k) + ((size_t)n * p.hqk + hb - p.hqk) * D;
  else dst = static_cast<QT*>(p.v) + ((size_t)n * p.hv + hb - 2 * p.hqk) * D;
  store8(dst + 8 * cg, y);
  cv.store_shifted_window(W3);
}

template <typename InT, typename QT, int D>
hipError_t launch_decode_prepare_t(const DecPrepParams& p, int num_seqs, hipStream_t stream) {
  constexpr int HPW = 256 / (D / 8);
  const int groups = (2 * p.hqk + p.hv + HPW - 1) / HPW;
  hipLaunchKernelGGL((decode_prepare_kernel<InT, QT, D>), dim3(num_seqs, groups + 1), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename InT, typename QT>
hipError_t launch_decode_prepare_d(const DecPrepParams& p, int d, int num_seqs,
                                   hipStream_t stream) {
  switch (d) {
    case 32: return launch_decode_prepare_t<InT, QT, 32>(p, num_seqs, stream);
    case 64: return launch_decode_prepare_t<InT, QT, 64>(p, num_seqs, stream);
    case 128: return launch_decode_prepare_t<InT, QT, 128>(p, num_seqs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prepare(const gdn_shape_t& s, const int32_t* cu, const void* x,
                          const void* w, const void* bias, const void* a, const void* b,
                          const float* A_log, const float* dt_bias, float eps, void* q, void* k,
                          void* v, float* g, float* beta, hipStream_t stream) {
  PrepParams p{cu, x, w, bias, a, b, A_log, dt_bias, eps, q, k, v, g, beta,
               s.num_seqs, s.total_tokens, s.num_qk_heads, s.num_v_heads};
  const bool in_bf = s.in_dtype == GDN_DTYPE_BF16, out_bf = s.qkv_dtype == GDN_DTYPE_BF16;
  if (in_bf && out_bf) return launch_prepare_d<bf16, bf16>(p, s.head_dim_k, stream);
  if (in_bf) return launch_prepare_d<bf16, float>(p, s.head_dim_k, stream);
  if (out_bf) return launch_prepare_d<float, bf16>(p, s.head_dim_k, stream);
  return launch_prepare_d<float, float>(p, s.head_dim_k, stream);
}

hipError_t launch_decode_prepare(const gdn_shape_t& s, const void* x, void* window,
                                 const void* w, const void* bias, const void* a, const void* b,
                                 const float* A_log, const float* dt_bias, float eps, void* q,
                                 void* k, void* v, float* g, float* beta, hipStream_t stream) {
  DecPrepParams p{x, window, w, bias, a, b, A_log, dt_bias, eps, q, k, v, g, beta,
                  s.num_qk_heads, s.num_v_heads};
  const bool in_bf = s.in_dtype == GDN_DTYPE_BF16, out_bf = s.qkv_dtype == GDN_DTYPE_BF16;
  const int d = s.head_dim_k;
  if (in_bf && out_bf) return launch_decode_prepare_d<bf16, bf16>(p, d, s.num_seqs, stream);
  if (in_bf) return launch_decode_prepare_d<bf16, float>(p, d, s.num_seqs, stream);
  if (out_bf) return launch_decode_prepare_d<float, bf16>(p, d, s.num_seqs, stream);
  return launch_decode_prepare_d<float, float>(p, d, s.num_seqs, stream);
}

}  // namespace gdn
