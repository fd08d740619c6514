// gdn_chunk.hip -- chunked prefill of the gated delta rule, chunk length 64
// ([MoE report] §3.7 "chunk_gated_delta_rule 七步拆解", Steps 2-7).
//
// Notation for one chunk of one V head (local rows t, j = 0..63; rows past the sequence end
// act as identity steps q = k = v = 0, beta = 0, g = 0), H0 = state at the chunk start:
//   b_t = sum_{s<=t} g_s  (in-chunk cumsum, Step 3),  gamma_t = e^{b_t},  G_tj = e^{b_t - b_j}
//   A   = strictly-lower( beta_t G_tj (k_t . k_j) )                        (Step 3)
//   T   = (I + A)^-1 (unit lower triangular)                                (Steps 3-4)
//   V'  = T diag(beta) (V - diag(gamma) K H0)     (the u_t of the token form; Steps 4-5)
//   O   = scale ( diag(gamma) Q H0 + P V' ),  P = (Q K^T) o G o lower-incl  (Step 5)
//   H_C = gamma_C H0 + K^T diag(e^{b_C - b}) V'                              (Step 6)
// V' is the page's v_new written with T diag(beta) applied to V - gamma K H0 instead of
// forming W = T diag(beta gamma) K: the same product, and W is never stored.
//
// This file holds the chunk-parallel half, chunk_intra: one workgroup per (chunk slot, V
// head). It forms K K^T and the masked decayed Q K^T on MFMA (bf16 rows; fp32 rows on fp32
// MFMA, or as hi + lo bf16 pairs under F32SplitMode; the decay and beta applied on the fly to
// the result fragments), inverts the unit-lower-triangular I + A (16x16 diagonal
// blocks by substitution, off-diagonal blocks by two levels of 16x16 fp32 MFMA products) and
// writes T diag(beta), scale P (as ready-made MFMA A fragments; the output scale is applied
// here, where the kernel waits on memory, and to the Q H term by the scan), e^{b_t} and
// e^{b_C - b_t} to the workspace. The sequential half, chunk_scan, is in gdn_scan.hip.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.h"

namespace gdn {
static_assert(kWsRecordBytes == kWorkspaceRecordBytes, "workspace record size");
namespace {

struct IntraParams {
  const int32_t* cu;
  const void* q;
  const void* k;
  const float* g;
  const float* beta;
  char* ws;
  int num_seqs, hqk, hv, num_slots;
  float scale;  // the output scale, folded into P
};

template <typename Mode, int ROWB>
__device__ __forceinline__ typename Mode::frag_t row_frag(const char* buf, int row, int kb, int grp);
template <>
__device__ __forceinline__ bf16x8 row_frag<Bf16Mode, 64>(const char* b, int r, int kb, int g) {
  return afrag<64>(b, r, kb, g);
}
template <>
__device__ __forceinline__ bf16x8 row_frag<Bf16Mode, 128>(const char* b, int r, int kb, int g) {
  return afrag<128>(b, r, kb, g);
}
template <>
__device__ __forceinline__ bf16x8 row_frag<Bf16Mode, 256>(const char* b, int r, int kb, int g) {
  return afrag<256>(b, r, kb, g);
}
template <>
__device__ __forceinline__ f32x8 row_frag<F32Mode, 128>(const char* b, int r, int kb, int g) {
  return afrag_f32<128>(b, r, kb, g);
}
template <>
__device__ __forceinline__ f32x8 row_frag<F32Mode, 256>(const char* b, int r, int kb, int g) {
  return afrag_f32<256>(b, r, kb, g);
}
template <>
__device__ __forceinline__ f32x8 row_frag<F32Mode, 512>(const char* b, int r, int kb, int g) {
  return afrag_f32<512>(b, r, kb, g);
}
// F32SplitMode: the fp32 rows of a matrix (ROWB bytes each) are staged as two bf16 planes, the
// hi halves of all 64 rows and then the lo halves, each laid out like bf16 rows of ROWB / 2
// bytes (the same swizzle), so a fragment is two conflict-free 16-byte reads.
template <int ROWB>
__device__ __forceinline__ Bf16Mode::Op split_row_frag(const char* b, int r, int kb, int g) {
  return {afrag<ROWB / 2>(b, r, kb, g), afrag<ROWB / 2>(b + 64 * (ROWB / 2), r, kb, g)};
}
template <>
__device__ __forceinline__ Bf16Mode::Op row_frag<F32SplitMode, 128>(const char* b, int r, int kb,
                                                                    int g) {
  return split_row_frag<128>(b, r, kb, g);
}
template <>
__device__ __forceinline__ Bf16Mode::Op row_frag<F32SplitMode, 256>(const char* b, int r, int kb,
                                                                    int g) {
  return split_row_frag<256>(b, r, kb, g);
}
template <>
__device__ __forceinline__ Bf16Mode::Op row_frag<F32SplitMode, 512>(const char* b, int r, int kb,
                                                                    int g) {
  return split_row_frag<512>(b, r, kb, g);
}

// One workgroup per (chunk slot, group of NV V heads of one QK head): NV = 2 when the heads per
// QK head come in pairs, else 1. K K^T and Q K^T of the chunk's QK head are formed once and
// serve the NV heads, whose gates, decay masks, inverses and records are worked on side by side
// by 4 waves each. T = (I + A)^-1 overwrites A in place, so that NV heads need the LDS of the
// staged q/k rows, or of one 64x64 fp32 matrix per head, whichever is larger.
template <typename Mode, int DK, int NV>
__global__ __launch_bounds__(256 * NV)
__attribute__((amdgpu_waves_per_eu(sizeof(typename Mode::in_t) == 4 && DK == 128 && NV == 1 ? 2 : 4)))
void chunk_intra_kernel(IntraParams p) {
  using in_t = typename Mode::in_t;
  using frag_t = typename Mode::frag_t;
  // record layout: F32SplitMode's records are F32Mode's (its scan splits them when it reads them)
  using RecM = std::conditional_t<std::is_same<Mode, F32SplitMode>::value, F32Mode, Mode>;
  constexpr int NWV = 4 * NV;  // waves
  constexpr int KB = DK / 32;
  constexpr int ROWB = DK * (int)sizeof(in_t), KBYTES = 64 * ROWB;
  constexpr int TBYTES = 64 * kLd * 4;  // one head's A, then T in place
  constexpr int SBYTES = 2 * KBYTES > NV * TBYTES ? 2 * KBYTES : NV * TBYTES;

  // Staged q/k rows; once the K K^T / Q K^T products are in registers the same bytes hold the
  // heads' A (then T) matrices.
  __shared__ __attribute__((aligned(1024))) char sKQ[SBYTES];
  // In-chunk gate cumsums in fp64: model gates sum to hundreds over a chunk, where an fp32 b
  // carries absolute errors of ~1e-4 into every decay e^{b_t - b_j} and e^{b_C - b_t}.
  __shared__ __attribute__((aligned(16))) double sb[NV][64];
  __shared__ __attribute__((aligned(16))) float sbeta[NV][64];
  auto sA = [&](int v) { return reinterpret_cast<float*>(sKQ + v * TBYTES); };

  // Work assignment: chunk slots are dealt to the 8 XCDs round robin (the hardware deals
  // workgroups b to XCD b % 8) and all H_qk * G / NV workgroups of a slot run back to back on its
  // XCD: the gates of a token (all V heads in one cache line) and the q/k rows of a QK head (read
  // by its G / NV workgroups) come from that XCD's L2.
  const int G = p.hv / p.hqk, NG = G / NV;
  const int j = blockIdx.x >> 3, per_slot = p.hqk * NG, r_ = j % per_slot;
  const int slot = 8 * (j / per_slot) + (blockIdx.x & 7), m = r_ / NG, hb = m * G + (r_ % NG) * NV;
  if (slot >= p.num_slots) return;  // padding workgroup (uniform)
  const int n = slot_to_seq(p.cu, p.num_seqs, slot);
  const int t0 = p.cu[n] + kChunk * (slot - slot_base(p.cu, n));
  const int tend = p.cu[n + 1];
  if (t0 >= tend) return;  // unused slot (uniform over the workgroup)
  const int len = min(kChunk, tend - t0);

  const int tid = threadIdx.x, lane = tid & 63, idx = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const size_t rstride = (size_t)p.hqk * DK;
  auto rec = [&](int v) { return p.ws + ((size_t)slot * p.hv + hb + v) * kWsRecordBytes; };
  float gate_g = 0.f, gate_b = 0.f;  // g and beta of token `lane` of head hb + wave (wave < NV)

  // ---- all memory reads at once: q/k rows into registers (16-byte loads, 1 KiB per wave
  // instruction) and the gates; then the rows go to LDS, row-major with the 16-byte XOR
  // swizzle (F32SplitMode: as hi and lo bf16 planes, the swizzle of bf16 rows). Rows past len
  // are written as zeros (identity steps).
  {
    constexpr bool SPLIT = std::is_same<Mode, F32SplitMode>::value;
    constexpr int NCH = ROWB / 16, RPU = 64 / NCH, KI = KBYTES / 1024;
    constexpr int PER = (2 * KI + NWV - 1) / NWV;  // units per wave (the last ones may idle)
    const in_t* Kg = static_cast<const in_t*>(p.k);
    const in_t* Qg = static_cast<const in_t*>(p.q);
    const char* Kb = reinterpret_cast<const char*>(Kg + (size_t)t0 * rstride + (size_t)m * DK);
    const char* Qb = reinterpret_cast<const char*>(Qg + (size_t)t0 * rstride + (size_t)m * DK);
    const unsigned rs = (unsigned)(rstride * sizeof(in_t));
    f32x4 r[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j2 = wave + NWV * u, jj = j2 < KI ? j2 : j2 - KI;
      const int row = jj * RPU + lane / NCH;
      const unsigned off =
          min(row, len - 1) * rs + 16 * ((lane % NCH) ^ (SPLIT ? 0 : swz<ROWB>(row)));
      if (j2 < 2 * KI) r[u] = *reinterpret_cast<const f32x4*>((j2 < KI ? Kb : Qb) + off);
    }
    if (wave < NV && lane < len) {
      gate_g = p.g[(size_t)(t0 + lane) * p.hv + hb + wave];
      gate_b = p.beta[(size_t)(t0 + lane) * p.hv + hb + wave];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j2 = wave + NWV * u, jj = j2 < KI ? j2 : j2 - KI;
      const int row = jj * RPU + lane / NCH;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      if (j2 < 2 * KI) {
        if constexpr (SPLIT) {
          // 4 fp32 values of a row -> 8 bytes in the hi plane and 8 in the lo plane
          const f32x4 x = row < len ? r[u] : z;
          char* plane = sKQ + (j2 < KI ? 0 : KBYTES);
          const int o2 = swz_off<ROWB / 2, 2>(row, 4 * (lane % NCH));
          bf16x4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hi[e] = (bf16)x[e];
            lo[e] = (bf16)(x[e] - (float)hi[e]);
          }
          *reinterpret_cast<bf16x4*>(plane + o2) = hi;
          *reinterpret_cast<bf16x4*>(plane + 64 * (ROWB / 2) + o2) = lo;
        } else {
          *reinterpret_cast<f32x4*>(sKQ + 1024 * j2 + 16 * lane) = row < len ? r[u] : z;
        }
      }
    }
  }
  lds_barrier();

  // ---- 20 tile products: the 10 A tiles on the first half of the waves (wave w of the half:
  // tiles w, w + NWV / 2, ...), the 10 P tiles on the second half, which owns whole stored P
  // blocks. Both kinds are formed transposed (C = K_ct X_rt^T), so that a lane holds 4
  // consecutive columns of one row of the wanted tile:
  //   A tiles (rt >= ct): A_tj = beta_t e^{b_t - b_j} (k_t . k_j) for j < t, into LDS;
  //   P^T tiles: C = K_ct Q_rt^T, whose C fragment IS half of the stored A fragment of
  //   P = (Q K^T) o Gamma o lower-incl: block (rt, kb) holds tiles ct = 2 kb (slots 0-3) and
  //   2 kb + 1 (slots 4-7; zeros where ct > rt), written as whole 16-byte fragments.
  // The products run first; waves 0 .. NV - 1 form their head's gate cumsum meanwhile. After
  // one barrier the first half writes the A tiles of all NV heads to LDS while the second half
  // writes the P blocks to the workspace.
  constexpr int HW = NWV / 2;                 // waves per half
  constexpr int NJ = (10 + HW - 1) / HW;      // A tiles per wave
  constexpr int NPB = NV == 2 ? 2 : 3;        // P blocks per wave
  const bool pw = wave >= HW;                 // P-tile wave
  const int wj = pw ? wave - HW : wave;       // index inside the half
  const char* sK = sKQ;
  const char* sQ = sKQ + KBYTES;
  auto job_tiles = [](int tt, int& r1, int& r2) {
    r1 = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;  // row tile
    r2 = tt - r1 * (r1 + 1) / 2;                        // column tile (<= r1)
  };
  // P block i of P wave wj (tri_block numbering), -1 for none: whole blocks split as evenly as
  // they allow (NV = 2: 3, 3, 2, 2 tiles; NV = 1: 5 and 5 tiles)
  auto pblock = [](int w, int i) -> int {
    if constexpr (NV == 2) {
      if (i == 0) return w == 0 ? 4 : w == 1 ? 5 : w == 2 ? 2 : 1;
      return w == 0 ? 0 : w == 1 ? 3 : -1;
    } else {
      if (i == 0) return w == 0 ? 4 : 5;
      if (i == 1) return w == 0 ? 0 : 2;
      return w == 0 ? 3 : 1;
    }
  };
  auto block_rt = [](int bl) { return bl < 2 ? bl : 2 + (bl - 2) / 2; };
  auto block_kb = [](int bl) { return bl < 2 ? 0 : (bl - 2) % 2; };
  // C = K_{rows 16 ra_t} X_{rows 16 rb_t}^T over d_k
  auto tile_product = [&](int ra_t, int rb_t, const char* bsrc) {
    frag_t fa[KB], fb[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      fa[kb] = row_frag<Mode, ROWB>(sK, 16 * ra_t + idx, kb, grp);
      fb[kb] = row_frag<Mode, ROWB>(bsrc, 16 * rb_t + idx, kb, grp);
    }
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (std::is_same<Mode, F32SplitMode>::value)
        c = Mode::mma_ss(c, fa[kb], fb[kb]);
      else
        c = mma32(fa[kb], fb[kb], c);
    }
    return c;
  };
  // One product loop for both kinds: job j of an A wave is A tile wj + HW j; job j of a P wave
  // is tile j % 2 of its P block j / 2.
  constexpr int NJM = NJ > 2 * NPB ? NJ : 2 * NPB;
  f32x4 acc[NJM];
#pragma unroll
  for (int i = 0; i < NJM; ++i) {
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    int ra_t = 0, rb_t = 0;
    bool ok;
    if (!pw) {
      const int tt = wj + HW * i;
      ok = i < NJ && tt < 10;
      if (ok) job_tiles(tt, rb_t, ra_t);  // rows ra_t = column tile of K, rb_t = row tile of K
    } else {
      const int bl = i / 2 < NPB ? pblock(wj, i / 2) : -1;
      ra_t = bl >= 0 ? 2 * block_kb(bl) + (i & 1) : 0;  // K rows: column tile ct
      rb_t = bl >= 0 ? block_rt(bl) : 0;                 // Q rows: row tile rt
      ok = bl >= 0 && ra_t <= rb_t;
    }
    if (ok) acc[i] = tile_product(ra_t, rb_t, pw ? sQ : sK);
  }
  if (wave < NV) {
    const double cs = wave_inclusive_scan_f64(gate_g, lane);
    const double cl = __shfl(cs, kChunk - 1, kWave);  // b_C (identity steps keep it at b_{len-1})
    sb[wave][lane] = cs;
    sbeta[wave][lane] = gate_b;
    reinterpret_cast<float*>(rec(wave) + kWsGOff)[lane] = __expf((float)cs);
    reinterpret_cast<float*>(rec(wave) + kWsDOff)[lane] = __expf((float)(cl - cs));
  }
  lds_barrier();  // sb, sbeta ready; every wave is done with the staged rows (sA may overwrite)
  if (!pw) {
#pragma unroll
    for (int i = 0; i < NJ; ++i) {
      const int tt = wj + HW * i;
      if (tt >= 10) continue;
      int r1, r2;
      job_tiles(tt, r1, r2);
      // lane: row t = 16 r1 + idx, columns j = 16 r2 + 4 grp + r (one 16-byte access)
      const int t = 16 * r1 + idx;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const double bt = sb[v][t];
        const float bet = sbeta[v][t];
        const f64x4 bj = ld_f64x4(&sb[v][16 * r2 + 4 * grp]);
        f32x4 av;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jc = 16 * r2 + 4 * grp + r;
          av[r] = jc < t ? bet * __expf((float)(bt - bj[r])) * acc[i][r] : 0.f;
        }
        *reinterpret_cast<f32x4*>(sA(v) + t * kLd + 16 * r2 + 4 * grp) = av;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NPB; ++i) {
      const int bl = pblock(wj, i);
      if (bl < 0) continue;
      const int rt = block_rt(bl), kb = block_kb(bl);
      const int t = 16 * rt + idx;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const double bt = sb[v][t];
        float x[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int ct = 2 * kb + hf;
          const f64x4 bj = ld_f64x4(&sb[v][16 * ct + 4 * grp]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jc = 16 * ct + 4 * grp + r;
            x[4 * hf + r] =
                jc <= t ? __expf((float)(bt - bj[r])) * (p.scale * acc[2 * i + hf][r]) : 0.f;
          }
        }
        ws_store<RecM>(rec(v) + kWsPOff, bl, lane, RecM::make(x));
      }
    }
  }
  lds_barrier();  // A complete

  // ---- T = (I + A)^-1 in place: head v's diagonal blocks on wave v, its off-diagonal blocks on
  // waves 2 v and 2 v + 1.
  invert_unit_lower64(wave < NV ? sA(wave) : nullptr, wave < 2 * NV ? sA(wave >> 1) : nullptr,
                      wave & 1, lane);
  // ---- T diag(beta) of every head as stored A fragments: NV x 6 blocks x 64 lanes.
  for (int it = tid; it < NV * 6 * 64; it += 256 * NV) {
    const int v = it / 384, bi = (it >> 6) % 6, ln = it & 63;
    const int rt = bi < 2 ? bi : 2 + (bi - 2) / 2;
    const int kb = bi < 2 ? 0 : (bi - 2) % 2;
    const int i = ln & 15, gr = ln >> 4;
    const int t = 16 * rt + i;
    const float* Tv = sA(v);
    const f32x4 be0 = row4(&sbeta[v][32 * kb + 4 * gr]), be1 = row4(&sbeta[v][32 * kb + 16 + 4 * gr]);
    const f32x4 ta = row4(Tv + t * kLd + 32 * kb + 4 * gr);
    const f32x4 tb = row4(Tv + t * kLd + 32 * kb + 16 + 4 * gr);
    float x[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int jc = 32 * kb + kslot(gr, s);
      x[s] = jc <= t ? (s < 4 ? ta[s] * be0[s] : tb[s - 4] * be1[s - 4]) : 0.f;
    }
    ws_store<RecM>(rec(v) + kWsTOff, bi, ln, RecM::make(x));
  }
}

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
template <typename Mode, int D>
hipError_t launch_intra_t(const gdn_shape_t& s, const IntraParams& p, hipStream_t stream) {
  const long long slots = chunk_slots(s);
  if (slots <= 0 || s.total_tokens == 0) return hipSuccess;
  const long long G = s.num_v_heads / s.num_qk_heads;
  IntraParams q = p;
  q.num_slots = (int)slots;
  // one workgroup per (unit, pair of V heads) when G is even, else per (unit, V head)
  const unsigned blocks =
      (unsigned)(8 * s.num_qk_heads * ((G % 2 == 0) ? G / 2 : G) * ((slots + 7) / 8));
  if (G % 2 == 0)
    hipLaunchKernelGGL((chunk_intra_kernel<Mode, D, 2>), dim3(blocks), dim3(512), 0, stream, q);
  else
    hipLaunchKernelGGL((chunk_intra_kernel<Mode, D, 1>), dim3(blocks), dim3(256), 0, stream, q);
  return hipGetLastError();
}

template <typename Mode>
hipError_t launch_intra_d(const gdn_shape_t& s, const IntraParams& p, hipStream_t stream) {
  switch (s.head_dim_k) {
    case 32: return launch_intra_t<Mode, 32>(s, p, stream);
    case 64: return launch_intra_t<Mode, 64>(s, p, stream);
    case 128: return launch_intra_t<Mode, 128>(s, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chunk_intra(const gdn_shape_t& s, const int32_t* cu, const void* q,
                              const void* k, const float* g, const float* beta, void* ws,
                              hipStream_t stream) {
  IntraParams p{cu, q, k, g, beta, static_cast<char*>(ws), s.num_seqs, s.num_qk_heads,
                s.num_v_heads, 0, s.scale};
  if (s.qkv_dtype == GDN_DTYPE_BF16) return launch_intra_d<Bf16Mode>(s, p, stream);
  if (s.qkv_dtype == GDN_DTYPE_F32_SPLIT) return launch_intra_d<F32SplitMode>(s, p, stream);
  return launch_intra_d<F32Mode>(s, p, stream);
}

}  // namespace gdn
