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
// head). It forms K K^T and the masked decayed Q K^T on MFMA (the decay and beta applied on
// the fly to the result fragments), inverts the unit-lower-triangular I + A (16x16 diagonal
// blocks by substitution, off-diagonal blocks by two levels of 16x16 fp32 MFMA products) and
// writes T diag(beta), P (as ready-made MFMA A fragments), e^{b_t} and e^{b_C - b_t} to the
// workspace. The sequential half, chunk_scan, is in gdn_scan.hip.
#include "gdn_device.hpp"
#include "gdn_internal.h"

namespace gdn {
static_assert(kWsRecordBytes == kWorkspaceRecordBytes, "workspace record size");
namespace {

// 16x16x16 fp32 product on MFMA with the 16-deep version of the fragment convention:
// A from LDS (row-major, leading dim ld), B either from LDS or from a C fragment in registers.
// Padded row length of the 64x64 fp32 LDS matrices: rows start 16-byte aligned (4 consecutive
// columns are one 16-byte access) and consecutive rows start 4 banks apart.
constexpr int kLd = 68;

__device__ __forceinline__ f32x4 row4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

__device__ __forceinline__ f32x4 mm16_ll(const float* A, const float* B, f32x4 c, int idx,
                                         int grp) {
  // A: 16x16 block at A (row stride kLd), B: 16x16 block at B (row stride kLd).
  const f32x4 a = row4(A + idx * kLd + 4 * grp);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], B[(4 * grp + r) * kLd + idx], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f32x4 mm16_lr(const float* A, const f32x4& Bc, f32x4 c, int idx,
                                         int grp) {
  const f32x4 a = row4(A + idx * kLd + 4 * grp);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], Bc[r], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ void store_c16(float* C, const f32x4& c, int idx, int grp,
                                          float sign) {
#pragma unroll
  for (int r = 0; r < 4; ++r) C[(4 * grp + r) * kLd + idx] = sign * c[r];
}

struct IntraParams {
  const int32_t* cu;
  const void* q;
  const void* k;
  const float* g;
  const float* beta;
  char* ws;
  int num_seqs, hqk, hv, num_slots;
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

// Half fragment (slots 4*half .. +3) of a stored operand block in global memory, split like
// Mode::make.
__device__ __forceinline__ void store_half_global(Bf16Mode, char* blk, int lane, int half,
                                                  const f32x4& x) {
  bf16x4 hi, lo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = (bf16)x[e];
    lo[e] = (bf16)(x[e] - (float)hi[e]);
  }
  *reinterpret_cast<bf16x4*>(blk + lane * 16 + half * 8) = hi;
  *reinterpret_cast<bf16x4*>(blk + 1024 + lane * 16 + half * 8) = lo;
}
__device__ __forceinline__ void store_half_global(F32Mode, char* blk, int lane, int half,
                                                  const f32x4& x) {
  *reinterpret_cast<f32x4*>(blk + lane * 32 + half * 16) = x;
}

// One workgroup per (chunk slot, V head). K K^T and Q K^T of the chunk's QK head are formed
// again for every V head that shares it: ~1 MFLOP per chunk, noise next to the scan, and it
// makes every workgroup independent.
template <typename Mode, int DK>
__global__ __launch_bounds__(256) void chunk_intra_kernel(IntraParams p) {
  using in_t = typename Mode::in_t;
  using frag_t = typename Mode::frag_t;
  constexpr int KB = DK / 32;
  constexpr int ROWB = DK * (int)sizeof(in_t), KBYTES = 64 * ROWB;
  constexpr int TBYTES = 64 * kLd * 4;
  constexpr int SBYTES = 2 * KBYTES > 2 * TBYTES ? 2 * KBYTES : 2 * TBYTES;

  // Staged q/k rows; once the K K^T / Q K^T products are in registers the same bytes hold A
  // and T (small enough for four workgroups per CU).
  __shared__ __attribute__((aligned(1024))) char sKQ[SBYTES];
  __shared__ __attribute__((aligned(16))) float sb[64];
  __shared__ __attribute__((aligned(16))) float sbeta[64];
  float* sA = reinterpret_cast<float*>(sKQ);
  float* sT = reinterpret_cast<float*>(sKQ + TBYTES);

  // Work assignment: units (chunk slot, QK head) are dealt to the 8 XCDs round robin (the
  // hardware deals workgroups b to XCD b % 8); the G workgroups of a unit (its V heads, which
  // read the same q/k rows) are dispatched back to back on one XCD and share its L2.
  const int G = p.hv / p.hqk;
  const int j = blockIdx.x >> 3, unit = 8 * (j / G) + (blockIdx.x & 7);
  const int slot = unit / p.hqk, h = (unit % p.hqk) * G + j % G;
  if (slot >= p.num_slots) return;  // padding workgroup (uniform)
  const int n = slot_to_seq(p.cu, p.num_seqs, slot);
  const int t0 = p.cu[n] + kChunk * (slot - slot_base(p.cu, n));
  const int tend = p.cu[n + 1];
  if (t0 >= tend) return;  // unused slot (uniform over the workgroup)
  const int len = min(kChunk, tend - t0);
  const int m = h / (p.hv / p.hqk);

  const int tid = threadIdx.x, lane = tid & 63, idx = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const size_t rstride = (size_t)p.hqk * DK;
  char* rec = p.ws + ((size_t)slot * p.hv + h) * kWsRecordBytes;
  float gate_g, gate_b;  // g and beta of token `lane` (wave 0)

  // ---- all memory reads at once: q/k rows into registers (16-byte loads, 1 KiB per wave
  // instruction) and this head's gates; then the rows go to LDS, row-major with the 16-byte
  // XOR swizzle. Rows past len are written as zeros (identity steps).
  {
    constexpr int NCH = ROWB / 16, RPU = 64 / NCH, KI = KBYTES / 1024, PER = 2 * KI / 4;
    static_assert(2 * KI % 4 == 0, "units per wave");
    const in_t* Kg = static_cast<const in_t*>(p.k);
    const in_t* Qg = static_cast<const in_t*>(p.q);
    const char* Kb = reinterpret_cast<const char*>(Kg + (size_t)t0 * rstride + (size_t)m * DK);
    const char* Qb = reinterpret_cast<const char*>(Qg + (size_t)t0 * rstride + (size_t)m * DK);
    const unsigned rs = (unsigned)(rstride * sizeof(in_t));
    f32x4 r[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = wave + 4 * u, jj = j < KI ? j : j - KI;
      const int row = jj * RPU + lane / NCH;
      const unsigned off = min(row, len - 1) * rs + 16 * ((lane % NCH) ^ swz<ROWB>(row));
      r[u] = *reinterpret_cast<const f32x4*>((j < KI ? Kb : Qb) + off);
    }
    float gv = 0.f, bv = 0.f;
    if (wave == 0 && lane < len) {
      gv = p.g[(size_t)(t0 + lane) * p.hv + h];
      bv = p.beta[(size_t)(t0 + lane) * p.hv + h];
    }
    gate_g = gv;
    gate_b = bv;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = wave + 4 * u, jj = j < KI ? j : j - KI;
      const int row = jj * RPU + lane / NCH;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(sKQ + 1024 * j + 16 * lane) = row < len ? r[u] : z;
    }
  }
  lds_barrier();

  // ---- 22 tile jobs, round robin over the waves (wave w: jobs w, w+4, ..., w+16 on MFMA,
  // and job w+20 for waves 0, 1). Both kinds are formed transposed (C = K_ct X_rt^T), so that a
  // lane holds 4 consecutive columns of one row of the wanted tile:
  //   0..9   A tiles (tr >= tc): A_tj = beta_t e^{b_t - b_j} (k_t . k_j) for j < t, into LDS;
  //   10..19 P^T tiles: C = K_ct Q_rt^T, whose C fragment IS half of the stored A fragment of
  //          P = (Q K^T) o Gamma o lower-incl (block (rt, ct / 2), slots 4 (ct % 2) + r);
  //   20, 21 the zero halves of the diagonal P blocks (ct = rt + 1 for rt = 0, 2).
  // The products run first; wave 0 forms the gate cumsum meanwhile; the epilogues that need it
  // follow one barrier later.
  const char* sK = sKQ;
  const char* sQ = sKQ + KBYTES;
  auto job_tiles = [](int job, int& r1, int& r2) {
    const int tt = job >= 10 ? job - 10 : job;
    r1 = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;  // row tile
    r2 = tt - r1 * (r1 + 1) / 2;                        // column tile (<= r1)
  };
  f32x4 acc[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int job = wave + 4 * i;
    const bool isp = job >= 10;
    int r1, r2;
    job_tiles(job, r1, r2);
    // Rows r2 of K against rows r1 of K (A^T tiles) or of Q (P^T tiles).
    const int ra = 16 * r2 + idx;
    const int rb = 16 * r1 + idx;
    const char* bsrc = isp ? sQ : sK;
    frag_t fa[KB], fb[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      fa[kb] = row_frag<Mode, ROWB>(sK, ra, kb, grp);
      fb[kb] = row_frag<Mode, ROWB>(bsrc, rb, kb, grp);
    }
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) c = mma32(fa[kb], fb[kb], c);
    acc[i] = c;
  }
  if (wave == 0) {
    const float cs = wave_inclusive_scan(gate_g, lane);
    const float cl = __shfl(cs, kChunk - 1, kWave);  // b_C (identity steps keep it at b_{len-1})
    sb[lane] = cs;
    sbeta[lane] = gate_b;
    reinterpret_cast<float*>(rec + kWsGOff)[lane] = __expf(cs);
    reinterpret_cast<float*>(rec + kWsDOff)[lane] = __expf(cl - cs);
  }
  if (wave < 2) {
    const int rt = wave == 0 ? 0 : 2;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    store_half_global(Mode{}, rec + kWsPOff + tri_block(rt, rt / 2) * kWsBlockBytes, lane, 1, z);
  }
  lds_barrier();  // sb, sbeta ready; every wave is done with the staged rows (sA may overwrite)
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int job = wave + 4 * i;
    int r1, r2;
    job_tiles(job, r1, r2);
    if (job < 10) {
      // lane: row t = 16 r1 + idx, columns j = 16 r2 + 4 grp + r (one 16-byte write)
      const int t = 16 * r1 + idx;
      const float bt = sb[t], bet = sbeta[t];
      const f32x4 bj = *reinterpret_cast<const f32x4*>(sb + 16 * r2 + 4 * grp);
      f32x4 av;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * r2 + 4 * grp + r;
        av[r] = j < t ? bet * __expf(bt - bj[r]) * acc[i][r] : 0.f;
      }
      *reinterpret_cast<f32x4*>(sA + t * kLd + 16 * r2 + 4 * grp) = av;
    } else {
      const int t = 16 * r1 + idx;
      const float bt = sb[t];
      const f32x4 bj = *reinterpret_cast<const f32x4*>(sb + 16 * r2 + 4 * grp);
      f32x4 pv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * r2 + 4 * grp + r;
        pv[r] = j <= t ? __expf(bt - bj[r]) * acc[i][r] : 0.f;
      }
      store_half_global(Mode{}, rec + kWsPOff + tri_block(r1, r2 >> 1) * kWsBlockBytes, lane,
                        r2 & 1, pv);
    }
  }
  lds_barrier();  // sA complete

  // ---- Diagonal 16x16 blocks of T: wave w inverts block w by forward substitution,
  // x_i = delta_ic - sum_{j<i} A_ij x_j with lane c < 16 carrying column c. Lane i holds row i
  // of the block; v_readlane broadcasts A_ij as a scalar operand (no LDS traffic in the loop).
  {
    const float* Ab = sA + (16 * wave) * kLd + 16 * wave;
    float arow[16];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const f32x4 a4 = row4(Ab + (lane & 15) * kLd + 4 * j4);
#pragma unroll
      for (int e = 0; e < 4; ++e) arow[4 * j4 + e] = a4[e];
    }
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == lane) ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      float part[4] = {0.f, 0.f, 0.f, 0.f};  // 4 independent chains
#pragma unroll
      for (int j = 0; j < i; ++j)
        part[j & 3] = fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(
                               __builtin_bit_cast(int, arow[j]), i)),
                           x[j], part[j & 3]);
      x[i] = (i == lane) ? 1.f : -((part[0] + part[1]) + (part[2] + part[3]));
    }
    if (lane < 16) {
      float* Tb = sT + (16 * wave) * kLd + 16 * wave;
#pragma unroll
      for (int i = 0; i < 16; ++i) Tb[i * kLd + lane] = x[i];
    }
  }
  lds_barrier();
  // ---- Level 2: T_10 = -T_11 A_10 T_00, T_32 = -T_33 A_32 T_22.
  if (wave < 2) {
    const int ib = 2 * wave + 1, jb = 2 * wave;
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 M = mm16_ll(sA + 16 * ib * kLd + 16 * jb, sT + 16 * jb * kLd + 16 * jb, z, idx, grp);
    f32x4 R = mm16_lr(sT + 16 * ib * kLd + 16 * ib, M, z, idx, grp);
    store_c16(sT + 16 * ib * kLd + 16 * jb, R, idx, grp, -1.f);
  }
  lds_barrier();
  // ---- Level 3, column block jb in {0, 1} (wave jb):
  //   X_i = sum_{kb=jb..1} A_{i,kb} T_{kb,jb} (i = 2, 3)
  //   T_{2,jb} = -T_22 X_2,  T_{3,jb} = -(T_32 X_2 + T_33 X_3)
  if (wave < 2) {
    const int jb = wave;
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 X2 = z, X3 = z;
    for (int kb = jb; kb < 2; ++kb) {
      const float* Tk = sT + 16 * kb * kLd + 16 * jb;
      X2 = mm16_ll(sA + 32 * kLd + 16 * kb, Tk, X2, idx, grp);
      X3 = mm16_ll(sA + 48 * kLd + 16 * kb, Tk, X3, idx, grp);
    }
    f32x4 T2 = mm16_lr(sT + 32 * kLd + 32, X2, z, idx, grp);
    f32x4 T3 = mm16_lr(sT + 48 * kLd + 32, X2, z, idx, grp);
    T3 = mm16_lr(sT + 48 * kLd + 48, X3, T3, idx, grp);
    store_c16(sT + 32 * kLd + 16 * jb, T2, idx, grp, -1.f);
    store_c16(sT + 48 * kLd + 16 * jb, T3, idx, grp, -1.f);
  }
  lds_barrier();
  // ---- T diag(beta) as stored A fragments: 6 blocks x 64 lanes.
  for (int it = tid; it < 6 * 64; it += 256) {
    const int bi = it >> 6, ln = it & 63;
    const int rt = bi < 2 ? bi : 2 + (bi - 2) / 2;
    const int kb = bi < 2 ? 0 : (bi - 2) % 2;
    const int i = ln & 15, gr = ln >> 4;
    const int t = 16 * rt + i;
    const f32x4 be0 = row4(sbeta + 32 * kb + 4 * gr), be1 = row4(sbeta + 32 * kb + 16 + 4 * gr);
    const f32x4 t0 = row4(sT + t * kLd + 32 * kb + 4 * gr);
    const f32x4 t1 = row4(sT + t * kLd + 32 * kb + 16 + 4 * gr);
    float x[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int j = 32 * kb + kslot(gr, s);
      x[s] = j <= t ? (s < 4 ? t0[s] * be0[s] : t1[s - 4] * be1[s - 4]) : 0.f;
    }
    Mode::store_block(rec + kWsTOff + bi * kWsBlockBytes, ln, Mode::make(x));
  }
}

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
template <typename Mode, int D>
hipError_t launch_intra_t(const gdn_shape_t& s, const IntraParams& p, hipStream_t stream) {
  const long long slots = chunk_slots(s);
  if (slots <= 0 || s.total_tokens == 0) return hipSuccess;
  const long long units = slots * s.num_qk_heads, G = s.num_v_heads / s.num_qk_heads;
  IntraParams q = p;
  q.num_slots = (int)slots;
  hipLaunchKernelGGL((chunk_intra_kernel<Mode, D>), dim3((unsigned)(8 * G * ((units + 7) / 8))),
                     dim3(256), 0, stream, q);
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
                s.num_v_heads, 0};
  if (s.qkv_dtype == GDN_DTYPE_BF16) return launch_intra_d<Bf16Mode>(s, p, stream);
  return launch_intra_d<F32Mode>(s, p, stream);
}

}  // namespace gdn
