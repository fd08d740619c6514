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
// Two kernels:
//   chunk_intra: one workgroup per (chunk slot, QK head), fully chunk-parallel. Forms K K^T and
//     Q K^T once per QK head on MFMA, then for each of its G V heads the cumsum, A, the
//     inverse T (16x16 diagonal blocks by substitution, off-diagonal blocks by two levels of
//     16x16 fp32 MFMA products) and P, and writes T diag(beta), P (as ready-made MFMA A
//     fragments) and b to the workspace.
//   chunk_scan: one workgroup per (sequence, V head, group of 16-column d_v tiles); each wave
//     keeps its [d_k x 16] fp32 slice of the state in registers for the whole sequence and
//     walks the chunks in order. d_v columns of the state evolve independently (column j
//     depends only on column j of v), which is what lets the scan split over d_v.
#include "gdn_device.hpp"
#include "gdn_internal.h"

namespace gdn {
static_assert(kWsRecordBytes == kWorkspaceRecordBytes, "workspace record size");
namespace {

// ---------------------------------------------------------------------------------------
// Operand-fragment loads straight from q/k in global memory (row-major [T][H_qk][DK]).
// Lane (idx, grp) of a 32-deep A fragment of rows r0.. reads K[r0 + idx][32 kb + kslot].
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void load_frag_row(const bf16* row, int kb, int grp, bf16x8& f) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * kb + 4 * grp);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * kb + 16 + 4 * grp);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f[s] = lo[s];
    f[4 + s] = hi[s];
  }
}
__device__ __forceinline__ void load_frag_row(const float* row, int kb, int grp, f32x8& f) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(row + 32 * kb + 4 * grp);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(row + 32 * kb + 16 + 4 * grp);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f[s] = lo[s];
    f[4 + s] = hi[s];
  }
}
template <typename F>
__device__ __forceinline__ void zero_frag(F& f) {
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = 0;
}

// 16x16x16 fp32 product on MFMA with the 16-deep version of the fragment convention:
// A from LDS (row-major, leading dim ld), B either from LDS or from a C fragment in registers.
constexpr int kLd = 65;  // padded row length of the 64x64 fp32 LDS matrices

__device__ __forceinline__ f32x4 mm16_ll(const float* A, const float* B, f32x4 c, int idx,
                                         int grp) {
  // A: 16x16 block at A (row stride kLd), B: 16x16 block at B (row stride kLd).
#pragma unroll
  for (int r = 0; r < 4; ++r)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(A[idx * kLd + 4 * grp + r],
                                             B[(4 * grp + r) * kLd + idx], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f32x4 mm16_lr(const float* A, const f32x4& Bc, f32x4 c, int idx,
                                         int grp) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(A[idx * kLd + 4 * grp + r], Bc[r], c, 0, 0, 0);
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
  int num_seqs, hqk, hv;
};

template <typename Mode, int DK>
__global__ __launch_bounds__(256) void chunk_intra_kernel(IntraParams p) {
  using in_t = typename Mode::in_t;
  using frag_t = typename Mode::frag_t;
  constexpr int KB = DK / 32;

  __shared__ float sKK[64 * kLd];
  __shared__ float sQK[64 * kLd];
  __shared__ float sA[64 * kLd];
  __shared__ float sT[64 * kLd];
  __shared__ float sb[64];
  __shared__ float sbeta[64];

  const int slot = blockIdx.x, m = blockIdx.y;
  const int n = slot_to_seq(p.cu, p.num_seqs, slot);
  const int t0 = p.cu[n] + kChunk * (slot - slot_base(p.cu, n));
  const int tend = p.cu[n + 1];
  if (t0 >= tend) return;  // unused slot (uniform over the workgroup)
  const int len = min(kChunk, tend - t0);
  const int G = p.hv / p.hqk;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, idx = lane & 15,
            grp = lane >> 4;
  const in_t* Q = static_cast<const in_t*>(p.q);
  const in_t* K = static_cast<const in_t*>(p.k);
  const size_t rstride = (size_t)p.hqk * DK;
  const in_t* Qc = Q + (size_t)t0 * rstride + (size_t)m * DK;
  const in_t* Kc = K + (size_t)t0 * rstride + (size_t)m * DK;

  // ---- K K^T and Q K^T, lower 16x16 tiles incl. the diagonal: 10 + 10 tiles, 5 per wave.
  for (int tile = wave; tile < 20; tile += 4) {
    const bool isq = tile >= 10;
    const int tt = isq ? tile - 10 : tile;
    const int tr = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;
    const int tc = tt - tr * (tr + 1) / 2;
    const int ra = 16 * tr + idx, rb = 16 * tc + idx;
    const in_t* rowa = (isq ? Qc : Kc) + (size_t)ra * rstride;
    const in_t* rowb = Kc + (size_t)rb * rstride;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      frag_t a, b;
      if (ra < len) load_frag_row(rowa, kb, grp, a); else zero_frag(a);
      if (rb < len) load_frag_row(rowb, kb, grp, b); else zero_frag(b);
      acc = mma32(a, b, acc);
    }
    float* dst = isq ? sQK : sKK;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(16 * tr + 4 * grp + r) * kLd + 16 * tc + idx] = acc[r];
  }

  for (int gg = 0; gg < G; ++gg) {
    const int h = m * G + gg;
    char* rec = p.ws + ((size_t)slot * p.hv + h) * kWsRecordBytes;
    __syncthreads();  // K K^T / Q K^T ready; previous head done with sA, sT, sb
    if (wave == 0) {
      const float gv = lane < len ? p.g[(size_t)(t0 + lane) * p.hv + h] : 0.f;
      const float bv = lane < len ? p.beta[(size_t)(t0 + lane) * p.hv + h] : 0.f;
      const float cs = wave_inclusive_scan(gv, lane);
      sb[lane] = cs;
      sbeta[lane] = bv;
      reinterpret_cast<float*>(rec + kWsBOff)[lane] = cs;
    }
    __syncthreads();
    // A = strictly-lower(beta_t e^{b_t - b_j} KK_tj); the exponent is <= 0 wherever used.
    for (int e = tid; e < 64 * 64; e += 256) {
      const int t = e >> 6, j = e & 63;
      sA[t * kLd + j] = j < t ? sbeta[t] * expf(sb[t] - sb[j]) * sKK[t * kLd + j] : 0.f;
    }
    __syncthreads();
    // Diagonal 16x16 blocks of T: wave w inverts block w by forward substitution, lane c < 16
    // carrying column c. x_i = delta_ic - sum_{j<i} A_ij x_j.
    if (lane < 16) {
      const float* Ab = sA + (16 * wave) * kLd + 16 * wave;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == lane) ? 1.f : 0.f;
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc = fmaf(Ab[i * kLd + j], x[j], acc);
        x[i] = (i == lane) ? 1.f : -acc;
      }
      float* Tb = sT + (16 * wave) * kLd + 16 * wave;
#pragma unroll
      for (int i = 0; i < 16; ++i) Tb[i * kLd + lane] = x[i];
    }
    __syncthreads();
    // Level 2: T_10 = -T_11 A_10 T_00, T_32 = -T_33 A_32 T_22.
    if (wave < 2) {
      const int ib = 2 * wave + 1, jb = 2 * wave;
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      f32x4 M = mm16_ll(sA + 16 * ib * kLd + 16 * jb, sT + 16 * jb * kLd + 16 * jb, z, idx, grp);
      f32x4 R = mm16_lr(sT + 16 * ib * kLd + 16 * ib, M, z, idx, grp);
      store_c16(sT + 16 * ib * kLd + 16 * jb, R, idx, grp, -1.f);
    }
    __syncthreads();
    // Level 3, column block jb in {0, 1} (wave jb):
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
    __syncthreads();
    // Write T diag(beta) and P as A fragments: 2 matrices x 6 blocks x 64 lanes.
    for (int it = tid; it < 2 * 6 * 64; it += 256) {
      const int mat = it / 384, bi = (it / 64) % 6, ln = it & 63;
      const int rt = bi < 2 ? bi : 2 + (bi - 2) / 2;
      const int kb = bi < 2 ? 0 : (bi - 2) % 2;
      const int i = ln & 15, gr = ln >> 4;
      const int t = 16 * rt + i;
      float x[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int j = 32 * kb + kslot(gr, s);
        float val = 0.f;
        if (j <= t) {
          val = mat == 0 ? sT[t * kLd + j] * sbeta[j]
                         : expf(sb[t] - sb[j]) * sQK[t * kLd + j];
        }
        x[s] = val;
      }
      char* blk = rec + (mat == 0 ? kWsTOff : kWsPOff) + bi * kWsBlockBytes;
      Mode::store_block(blk, ln, Mode::make(x));
    }
  }
}

// ---------------------------------------------------------------------------------------
// Scan kernel.
// ---------------------------------------------------------------------------------------
struct ScanParams {
  const int32_t* cu;
  const void* q;
  const void* k;
  const void* v;
  const float* h0;
  void* o;
  float* ht;
  const char* ws;
  int num_seqs, hqk, hv;
  float scale;
};

// Writes 4 consecutive slots of a fragment in LDS with one 8- or 16-byte store (never a
// read-modify-write of the whole fragment, which would race with the thread that owns the
// other 4 slots).
__device__ __forceinline__ void put4(bf16x8* f, int s0, const float* x) {
  bf16x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (bf16)x[e];
  *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(f) + s0) = v;
}
__device__ __forceinline__ void put4(f32x8* f, int s0, const float* x) {
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = x[e];
  *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(f) + s0) = v;
}
__device__ __forceinline__ void put1(bf16x8* f, int s, float x) {
  reinterpret_cast<bf16*>(f)[s] = (bf16)x;
}
__device__ __forceinline__ void put1(f32x8* f, int s, float x) { reinterpret_cast<float*>(f)[s] = x; }

template <typename Mode, int DK, int DV, int NW, typename OutT>
__global__ __launch_bounds__(NW * 64) void chunk_scan_kernel(ScanParams p) {
  using in_t = typename Mode::in_t;
  using frag_t = typename Mode::frag_t;
  using Op = typename Mode::Op;
  constexpr int KB = DK / 32;   // 32-deep blocks over d_k
  constexpr int IT = DK / 16;   // 16-row tiles over d_k
  constexpr int NB = DV / 16 / NW;
  static_assert(DV % (16 * NW) == 0, "d_v tiles");

  // LDS: per-chunk operand fragments shared by the NW waves.
  __shared__ frag_t sKf[4 * KB * 64];   // A of K H   : [rt][kb][lane]
  __shared__ frag_t sQf[4 * KB * 64];   // A of Q H   : [rt][kb][lane]
  __shared__ frag_t sKTf[IT * 2 * 64];  // A of K^T V : [it][kb'][lane]
  __shared__ __attribute__((aligned(16))) char sTP[12 * kWsBlockBytes];
  __shared__ float sb[64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, idx = lane & 15,
            grp = lane >> 4;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int dvb = lid % NB, nh = lid / NB;
  const int h = nh % p.hv, n = nh / p.hv;
  const int G = p.hv / p.hqk, m = h / G;
  const int col = 16 * (dvb * NW + wave) + idx;  // this lane's d_v column

  const in_t* Qg = static_cast<const in_t*>(p.q);
  const in_t* Kg = static_cast<const in_t*>(p.k);
  const in_t* Vg = static_cast<const in_t*>(p.v);
  OutT* Og = static_cast<OutT*>(p.o);
  const size_t qkstride = (size_t)p.hqk * DK;

  // State slice: Hc[it][r] = H[16 it + 4 grp + r][col].
  f32x4 Hc[IT];
  {
    const float* H0 = p.h0 ? p.h0 + (size_t)nh * DK * DV : nullptr;
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Hc[it][r] = H0 ? H0[(size_t)(16 * it + 4 * grp + r) * DV + col] : 0.f;
  }

  const int start = p.cu[n];
  const int L = p.cu[n + 1] - start;
  const int nchunks = (L + kChunk - 1) / kChunk;
  const int slot0 = slot_base(p.cu, n);

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = start + kChunk * c;
    const int len = min(kChunk, L - kChunk * c);
    __syncthreads();  // previous chunk's LDS reads are done

    // ---- stage q, k operand fragments (rows >= len are zero)
    constexpr int PER_ROW = DK / 8;  // 8-element pieces per row
    for (int pc = tid; pc < 64 * PER_ROW; pc += NW * 64) {
      const int row = pc / PER_ROW, d0 = 8 * (pc % PER_ROW);
      float kx[8], qx[8];
      if (row < len) {
        const in_t* kr = Kg + (size_t)(t0 + row) * qkstride + (size_t)m * DK + d0;
        const in_t* qr = Qg + (size_t)(t0 + row) * qkstride + (size_t)m * DK + d0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kx[e] = to_f32(kr[e]);
          qx[e] = to_f32(qr[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[e] = qx[e] = 0.f;
      }
      const int rt = row >> 4, i = row & 15, kb = d0 >> 5, o = d0 & 31;
      const int g0 = (o & 15) >> 2, s0 = o >= 16 ? 4 : 0;
      // elements 0-3 -> lane (i, g0) slots s0..s0+3; elements 4-7 -> lane (i, g0+1)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int fl = i + 16 * (g0 + half);
        put4(&sKf[(rt * KB + kb) * 64 + fl], s0, kx + 4 * half);
        put4(&sQf[(rt * KB + kb) * 64 + fl], s0, qx + 4 * half);
      }
      // K^T fragments: element d -> tile it = d / 16, lane (d % 16, grp(tok)), slot(tok)
      const int kbp = row >> 5, tt = row & 31;
      const int gp = (tt & 15) >> 2, sp = (tt >> 4) * 4 + (tt & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = d0 + e;
        put1(&sKTf[((d >> 4) * 2 + kbp) * 64 + (d & 15) + 16 * gp], sp, kx[e]);
      }
    }
    // ---- copy T diag(beta) / P fragments and b from the workspace record
    {
      const char* rec = p.ws + ((size_t)(slot0 + c) * p.hv + h) * kWsRecordBytes;
      const f32x4* src = reinterpret_cast<const f32x4*>(rec);
      f32x4* dst = reinterpret_cast<f32x4*>(sTP);
      for (int e = tid; e < 12 * kWsBlockBytes / 16; e += NW * 64) dst[e] = src[e];
      if (tid < 64) sb[tid] = reinterpret_cast<const float*>(rec + kWsBOff)[tid];
    }
    __syncthreads();

    // ---- H as split B fragments over d_k: HB[kb] from tiles 2kb, 2kb+1
    Op HB[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float x[8];
      pack_c_pair(Hc[2 * kb], Hc[2 * kb + 1], x);
      HB[kb] = Mode::make(x);
    }

    // ---- K H and Q H per 16-row tile; Y = V - gamma K H; QH scaled by gamma
    f32x4 QH[4], Y[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 kh = {0.f, 0.f, 0.f, 0.f}, qh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        kh = Mode::mma_xs(kh, sKf[(rt * KB + kb) * 64 + lane], HB[kb]);
        qh = Mode::mma_xs(qh, sQf[(rt * KB + kb) * 64 + lane], HB[kb]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * rt + 4 * grp + r;
        const float gam = expf(sb[t]);
        const float vv = t < len ? to_f32(Vg[((size_t)(t0 + t) * p.hv + h) * DV + col]) : 0.f;
        Y[rt][r] = vv - gam * kh[r];
        QH[rt][r] = gam * qh[r];
      }
    }
    Op YB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float x[8];
      pack_c_pair(Y[2 * kb], Y[2 * kb + 1], x);
      YB[kb] = Mode::make(x);
    }
    // ---- V' = (T diag(beta)) Y   (lower-triangular block structure)
    f32x4 Vp[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= rt / 2; ++kb) {
        const Op a = Mode::load_block(sTP + kWsTOff + tri_block(rt, kb) * kWsBlockBytes, lane);
        acc = Mode::mma_ss(acc, a, YB[kb]);
      }
      Vp[rt] = acc;
    }
    const float bC = sb[63];
    Op VB[2], DB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float x[8], d[8];
      pack_c_pair(Vp[2 * kb], Vp[2 * kb + 1], x);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int t = 32 * kb + kslot(grp, s);
        d[s] = x[s] * expf(bC - sb[t]);
      }
      VB[kb] = Mode::make(x);
      DB[kb] = Mode::make(d);
    }
    // ---- O = gamma Q H + P V'
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 acc = QH[rt];
#pragma unroll
      for (int kb = 0; kb <= rt / 2; ++kb) {
        const Op a = Mode::load_block(sTP + kWsPOff + tri_block(rt, kb) * kWsBlockBytes, lane);
        acc = Mode::mma_ss(acc, a, VB[kb]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * rt + 4 * grp + r;
        if (t < len)
          Og[((size_t)(t0 + t) * p.hv + h) * DV + col] = from_f32<OutT>(p.scale * acc[r]);
      }
    }
    // ---- H <- gamma_C H + K^T diag(e^{b_C - b}) V'
    const float gC = expf(bC);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      f32x4 acc = Hc[it] * gC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) acc = Mode::mma_xs(acc, sKTf[(it * 2 + kb) * 64 + lane], DB[kb]);
      Hc[it] = acc;
    }
  }

  if (p.ht) {
    float* HT = p.ht + (size_t)nh * DK * DV;
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) HT[(size_t)(16 * it + 4 * grp + r) * DV + col] = Hc[it][r];
  }
}

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
template <typename Mode, int D>
hipError_t launch_intra_t(const gdn_shape_t& s, const IntraParams& p, hipStream_t stream) {
  const long long slots = chunk_slots(s);
  if (slots <= 0 || s.total_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_intra_kernel<Mode, D>), dim3((unsigned)slots, (unsigned)s.num_qk_heads),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename Mode, int D, int NW, typename OutT>
hipError_t launch_scan_nw(const ScanParams& p, long long heads, hipStream_t stream) {
  static_assert(D / 16 % NW == 0, "d_v tiles per workgroup");
  const unsigned blocks = (unsigned)(heads * (D / 16 / NW));
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_scan_kernel<Mode, D, D, NW, OutT>), dim3(blocks), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename Mode, int D, typename OutT>
hipError_t launch_scan_t(const gdn_shape_t& s, const ScanParams& p, hipStream_t stream) {
  // Waves per workgroup (each wave owns one 16-column d_v tile): the most (<= 4) that still
  // leaves >= 512 workgroups, else 1.
  const long long heads = (long long)s.num_seqs * s.num_v_heads;
  constexpr int tiles = D / 16;
  if constexpr (tiles % 4 == 0) {
    if (heads * (tiles / 4) >= 512) return launch_scan_nw<Mode, D, 4, OutT>(p, heads, stream);
  }
  if constexpr (tiles % 2 == 0) {
    if (heads * (tiles / 2) >= 512) return launch_scan_nw<Mode, D, 2, OutT>(p, heads, stream);
  }
  return launch_scan_nw<Mode, D, 1, OutT>(p, heads, stream);
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

template <typename Mode, typename OutT>
hipError_t launch_scan_d(const gdn_shape_t& s, const ScanParams& p, hipStream_t stream) {
  switch (s.head_dim_k) {
    case 32: return launch_scan_t<Mode, 32, OutT>(s, p, stream);
    case 64: return launch_scan_t<Mode, 64, OutT>(s, p, stream);
    case 128: return launch_scan_t<Mode, 128, OutT>(s, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chunk_intra(const gdn_shape_t& s, const int32_t* cu, const void* q,
                              const void* k, const float* g, const float* beta, void* ws,
                              hipStream_t stream) {
  IntraParams p{cu, q, k, g, beta, static_cast<char*>(ws), s.num_seqs, s.num_qk_heads,
                s.num_v_heads};
  if (s.qkv_dtype == GDN_DTYPE_BF16) return launch_intra_d<Bf16Mode>(s, p, stream);
  return launch_intra_d<F32Mode>(s, p, stream);
}

hipError_t launch_chunk_scan(const gdn_shape_t& s, const int32_t* cu, const void* q,
                             const void* k, const void* v, const float* h0, void* o, float* ht,
                             const void* ws, hipStream_t stream) {
  ScanParams p{cu, q, k, v, h0, o, ht, static_cast<const char*>(ws), s.num_seqs, s.num_qk_heads,
               s.num_v_heads, s.scale};
  const bool out_bf = s.out_dtype == GDN_DTYPE_BF16;
  if (s.qkv_dtype == GDN_DTYPE_BF16)
    return out_bf ? launch_scan_d<Bf16Mode, bf16>(s, p, stream)
                  : launch_scan_d<Bf16Mode, float>(s, p, stream);
  return out_bf ? launch_scan_d<F32Mode, bf16>(s, p, stream)
                : launch_scan_d<F32Mode, float>(s, p, stream);
}

}  // namespace gdn
