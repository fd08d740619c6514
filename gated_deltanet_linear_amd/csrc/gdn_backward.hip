// gdn_backward.hip -- gradients of the chunked gated delta rule (training backward pass):
// dq, dk, dv, dg, dbeta and the initial-state gradient from the output gradient and, optionally,
// the final-state gradient ([MoE report] §3.7, the chunked form trained chunk by chunk; the token
// recurrence of §3.3 stage 3 is the definition it differentiates).
//
// Chunk form (C = 64 rows, b = in-chunk cumsum of g, gamma = e^b, B = b of the chunk's last
// token, gamma_C = e^B, delta = e^{B - b}, Gamma_tj = e^{b_t - b_j}):
//   Y  = V - diag(gamma) K H              V' = T diag(beta) Y,   T = (I + diag(beta) At)^-1
//   O  = scale (diag(gamma) Q H + P V')   P = lower-incl(Q K^T o Gamma), At = lower(K K^T o Gamma)
//   H' = gamma_C H + K^T diag(delta) V'
// Reverse mode per chunk, with dO^ = scale dO and dH' the gradient of the chunk's end state:
//   dV' = P^T dO^ + diag(delta) K dH'      Z = T^T dV'      dY = dV = diag(beta) Z
//   dH  = gamma_C dH' + Q^T diag(gamma) dO^ - K^T diag(gamma) dY        (the previous chunk's dH')
//   dQ  = diag(gamma) dO^ H^T + (dP o Gamma) K,                         dP = lower-incl(dO^ V'^T)
//   dK  = diag(delta) V' dH'^T - diag(gamma) dY H^T + (dP o Gamma)^T Q + (dS + dS^T) K,
//         dA = -Z V'^T (strictly lower),  dS = dA o diag(beta) Gamma
//   dbeta_t = <Y_t, Z_t> + sum_j dA_tj At_tj
//   dg_s (the reverse in-chunk cumsum of db, written without cancelling terms):
//        sum_{t >= s} gamma_t (<Q_t, (dO^ H^T)_t> - <K_t, (dY H^T)_t>)
//      + sum_{t < s} delta_t <K_t, (V' dH'^T)_t> + gamma_C <H, dH'>
//      + sum_{t >= s, j < s} E_tj,          E = dP o P + dA o diag(beta) At
//   (db_t itself has E's row sum minus its column sum and a -delta_t term balanced by the last
//   token's dB; summed in this form, the parts that cancel are never formed: plain fp32 suffix
//   sums of db lost ~1e-4 of dg's RMS).
//
// Launches (fp32 accumulation throughout; with bf16 inputs the products whose operands allow it
// run on bf16 MFMA, exact operands as they are and computed ones as hi + lo bf16 pairs, the C x C
// products of the gradient kernel on fp32 MFMA; with fp32 inputs every product on fp32 MFMA):
//   bwd_intra  one workgroup per (chunk slot, V head): b, T (forward substitution), P, At.
//   bwd_scan forward pass, per (sequence, V head, 16-column tile): the states H at every chunk
//              start (from the initial state), and Y, V' of every token.
//   bwd_scan reverse pass, same layout, chunks in reverse: dH' of every chunk, Z, dv, dh0. The
//              two passes share no outputs: with bf16 inputs one 8-wave workgroup runs both side
//              by side (bwd_scan2), with fp32 inputs they are two launches.
//   bwd_grads  one 512-thread workgroup per (chunk slot, QK head), its G V heads in turn: dq, dk
//              (summed over the G heads), dg, dbeta.
// The state matrices stay in global memory, read along their contiguous axis.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kC = kChunk;  // 64
constexpr int kRecFloats = 3 * kC * kC + 2 * kC;  // T | P | At (fp32) | b (64 fp64)

// In-chunk cumsum b of the log-decays, in fp64: a fp32 b of a chunk with strong decay (|g| up to
// ~40 per token, |b| up to ~2500) loses ~1e-4 of Gamma_tj = e^{b_t - b_j} where b_t - b_j is
// small, and the gate gradient lost as much; from fp64 values the differences are exact enough.
__device__ __forceinline__ const double* rec_b(const float* rec) {
  return reinterpret_cast<const double*>(rec + 3 * kC * kC);
}

struct BwdParams {
  const int32_t* cu;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const void* h0;    // initial states (state dtype) or null
  const void* dout;  // [T][hv][d] out dtype
  const void* dht;   // final-state gradient (state dtype) or null
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  void* dh0;         // initial-state gradient (state dtype) or null
  float* rec;        // [slots][hv] records of kRecFloats
  float* hs;         // [slots][hv][d][d] state at every chunk start
  float* dhs;        // [slots][hv][d][d] gradient of every chunk's end state
  float* ys;         // [T][hv][d] Y
  float* vp;         // [T][hv][d] V'
  float* zs;         // [T][hv][d] Z
  int num_seqs, T, hqk, hv, num_slots;
  float scale;
  int state_bf16;
};

__device__ __forceinline__ float ld_state(const void* base, size_t i, int bf) {
  return bf ? to_f32(static_cast<const bf16*>(base)[i]) : static_cast<const float*>(base)[i];
}
__device__ __forceinline__ void st_state(void* base, size_t i, float x, int bf) {
  if (bf)
    static_cast<bf16*>(base)[i] = from_f32<bf16>(x);
  else
    static_cast<float*>(base)[i] = x;
}

// acc += A[0..16)[0..K) * B[0..K)[0..16) for the calling wave; a(i, kk) and b(kk, j) return the
// elements (i, j in 0..15, kk the depth index). Result: lane (idx, grp) holds rows 4 grp + r,
// column idx. K is a multiple of 32.
template <typename FA, typename FB>
__device__ __forceinline__ f32x4 tile_mma(FA a, FB b, int K, f32x4 acc) {
  const int lane = threadIdx.x & 63, idx = lane & 15, grp = lane >> 4;
  for (int k0 = 0; k0 < K; k0 += 32) {
    f32x8 av, bv;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int kk = k0 + kslot(grp, s);
      av[s] = a(idx, kk);
      bv[s] = b(kk, idx);
    }
    acc = mma32(av, bv, acc);
  }
  return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 8 fragment values of a row contiguous along the depth: slots 0-3 are depth k0 + 4 grp .. + 3,
// slots 4-7 depth k0 + 16 + 4 grp .. + 3 (kslot), so two 16-byte (fp32) or 8-byte (bf16) loads.
__device__ __forceinline__ void row_frag(const float* row, int k0, int grp, float scale, f32x8& o) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(row + k0 + 4 * grp);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(row + k0 + 16 + 4 * grp);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    o[s] = scale * lo[s];
    o[4 + s] = scale * hi[s];
  }
}
__device__ __forceinline__ void row_frag(const bf16* row, int k0, int grp, float scale, f32x8& o) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + k0 + 4 * grp);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + k0 + 16 + 4 * grp);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    o[s] = scale * (float)lo[s];
    o[4 + s] = scale * (float)hi[s];
  }
}

// acc += A B^T over depth K where this lane's A row (row idx of the tile) and B row (column idx)
// are both contiguous along the depth: the common case of the gradient products, read with
// vector loads. A null A row stands for zeros (rows past the chunk end).
template <typename TA, typename TB>
__device__ __forceinline__ f32x4 tile_mma_rows(const TA* a_row, float a_scale, const TB* b_row,
                                               int K, f32x4 acc) {
  const int grp = (threadIdx.x & 63) >> 4;
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 32) {
    f32x8 av, bv;
    if (a_row) {
      row_frag(a_row, k0, grp, a_scale, av);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) av[s] = 0.f;
    }
    row_frag(b_row, k0, grp, 1.f, bv);
    acc = mma32(av, bv, acc);
  }
  return acc;
}

// acc += A B^T over depth K for bf16 rows (exact operands: one bf16 MFMA per 32-deep step, the
// products exact, fp32 accumulation); an A row with ok == false counts as zeros.
__device__ __forceinline__ f32x4 tile_mma_rows_bf16(const bf16* a_row, bool ok, const bf16* b_row,
                                                    int K, f32x4 acc) {
  const int grp = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    const bf16x4 alo = *reinterpret_cast<const bf16x4*>(a_row + k0 + 4 * grp);
    const bf16x4 ahi = *reinterpret_cast<const bf16x4*>(a_row + k0 + 16 + 4 * grp);
    const bf16x4 blo = *reinterpret_cast<const bf16x4*>(b_row + k0 + 4 * grp);
    const bf16x4 bhi = *reinterpret_cast<const bf16x4*>(b_row + k0 + 16 + 4 * grp);
    const bf16x8 av = ok ? bf16x8{alo[0], alo[1], alo[2], alo[3], ahi[0], ahi[1], ahi[2], ahi[3]}
                         : bf16x8{};
    const bf16x8 bv{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
    acc = mma32(av, bv, acc);
  }
  return acc;
}

// (sequence, first token, valid rows) of chunk slot `slot`; false for an unused slot.
__device__ __forceinline__ bool slot_chunk(const BwdParams& p, int slot, int& n, int& t0, int& L) {
  n = slot_to_seq(p.cu, p.num_seqs, slot);
  t0 = p.cu[n] + kC * (slot - slot_base(p.cu, n));
  const int tend = p.cu[n + 1];
  L = min(kC, tend - t0);
  return t0 < tend;
}

// ---- bwd_intra ------------------------------------------------------------------------------
// One workgroup of 4 waves per (chunk slot, V head); the H_v workgroups of a chunk slot run back
// to back on one XCD (the q/k rows of a QK head and the gate lines come from its L2). The chunk's q/k rows are staged
// in LDS (rows past the end as zeros); the 20 lower 16x16 tiles of K K^T and Q K^T are formed
// transposed (C = K_ct X_rt^T, so a lane holds 4 consecutive columns of one row and writes
// them with one 16-byte store); then T = (I + diag(beta) At)^-1 in place of the staged rows.
template <typename InT, int D>
__global__ __launch_bounds__(256) void bwd_intra_kernel(BwdParams p) {
  constexpr int ROWB = D * (int)sizeof(InT), KBYTES = 64 * ROWB, KB = D / 32;
  constexpr int MBYTES = 64 * kLd * 4;
  constexpr int SBYTES = 2 * KBYTES > MBYTES ? 2 * KBYTES : MBYTES;
  __shared__ __attribute__((aligned(1024))) char sKQ[SBYTES];  // q/k rows, then A / T
  __shared__ double sb[kC];
  __shared__ float sbeta[kC];
  float* const sM = reinterpret_cast<float*>(sKQ);

  const int G = p.hv / p.hqk;
  const int j = blockIdx.x >> 3, per_slot = p.hqk * G;
  const int slot = 8 * (j / per_slot) + (blockIdx.x & 7), h = j % per_slot, m = h / G;
  int n, t0, L;
  if (slot >= p.num_slots || !slot_chunk(p, slot, n, t0, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, idx = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  float* rec = p.rec + ((size_t)slot * p.hv + h) * kRecFloats;

  // ---- q/k rows into registers (16-byte loads; rows past L re-read the last row), then to LDS
  // row-major with the 16-byte XOR swizzle (rows past L as zeros: identity steps)
  {
    constexpr int NCH = ROWB / 16, RPU = 64 / NCH, KI = KBYTES / 1024, PER = 2 * KI / 4;
    static_assert(2 * KI % 4 == 0, "units per wave");
    const size_t rstride = (size_t)p.hqk * D;
    const char* Kb = reinterpret_cast<const char*>(static_cast<const InT*>(p.k) +
                                                   (size_t)t0 * rstride + (size_t)m * D);
    const char* Qb = reinterpret_cast<const char*>(static_cast<const InT*>(p.q) +
                                                   (size_t)t0 * rstride + (size_t)m * D);
    const unsigned rs = (unsigned)(rstride * sizeof(InT));
    f32x4 r[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j2 = wave + 4 * u, jj = j2 < KI ? j2 : j2 - KI;
      const int row = jj * RPU + lane / NCH;
      const unsigned off = min(row, L - 1) * rs + 16 * ((lane % NCH) ^ swz<ROWB>(row));
      r[u] = *reinterpret_cast<const f32x4*>((j2 < KI ? Kb : Qb) + off);
    }
    if (wave == 0) {  // b = inclusive cumsum of g (0 past the end: identity steps)
      const double gi = lane < L ? (double)p.g[(size_t)(t0 + lane) * p.hv + h] : 0.0;
      const double bi = wave_inclusive_scan_f64(gi, lane);
      sb[lane] = bi;
      reinterpret_cast<double*>(rec + 3 * kC * kC)[lane] = bi;
      sbeta[lane] = lane < L ? p.beta[(size_t)(t0 + lane) * p.hv + h] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j2 = wave + 4 * u, jj = j2 < KI ? j2 : j2 - KI;
      const int row = jj * RPU + lane / NCH;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(sKQ + 1024 * j2 + 16 * lane) = row < L ? r[u] : z;
    }
  }
  lds_barrier();

  // ---- 20 tile products, round robin over the waves (wave w: jobs w, w + 4, ...):
  //   0..9   S tiles (rt >= ct) of K K^T,  10..19 the same tiles of Q K^T,
  // each as C = K_ct X_rt^T: lane (idx, grp) gets row t = 16 rt + idx, columns 16 ct + 4 grp + r.
  // Depth order of both operands: column-contiguous over d_k (one 16-byte piece per fragment).
  const char* sK = sKQ;
  const char* sQ = sKQ + KBYTES;
  auto job_tiles = [](int tt, int& r1, int& r2) {
    r1 = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;  // row tile
    r2 = tt - r1 * (r1 + 1) / 2;                        // column tile (<= r1)
  };
  f32x4 acc[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int job = wave + 4 * i, tt = job >= 10 ? job - 10 : job;
    int r1, r2;
    job_tiles(tt, r1, r2);
    const char* bsrc = job >= 10 ? sQ : sK;
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (std::is_same<InT, bf16>::value) {
        c = mma32(afrag<ROWB>(sK, 16 * r2 + idx, kb, grp), afrag<ROWB>(bsrc, 16 * r1 + idx, kb, grp), c);
      } else {
        c = mma32(afrag_f32<ROWB>(sK, 16 * r2 + idx, kb, grp),
                  afrag_f32<ROWB>(bsrc, 16 * r1 + idx, kb, grp), c);
      }
    }
    acc[i] = c;
  }
  lds_barrier();  // the staged rows are read: the matrix may overwrite them

  // ---- records At = lower(S o Gamma), P = lower-incl(Q K^T o Gamma) (row-major, 16-byte
  // stores; the 6 tiles above the diagonal of each as zeros) and A = diag(beta) At into LDS
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int job = wave + 4 * i, tt = job >= 10 ? job - 10 : job;
    int r1, r2;
    job_tiles(tt, r1, r2);
    const int t = 16 * r1 + idx, j0 = 16 * r2 + 4 * grp;
    f32x4 gm;
#pragma unroll
    for (int r = 0; r < 4; ++r) gm[r] = j0 + r <= t ? expf((float)(sb[t] - sb[j0 + r])) : 0.f;
    if (job < 10) {
      f32x4 at;
#pragma unroll
      for (int r = 0; r < 4; ++r) at[r] = j0 + r < t ? acc[i][r] * gm[r] : 0.f;
      *reinterpret_cast<f32x4*>(rec + 2 * kC * kC + t * kC + j0) = at;
      *reinterpret_cast<f32x4*>(sM + t * kLd + j0) = at * sbeta[t];
    } else {
      *reinterpret_cast<f32x4*>(rec + kC * kC + t * kC + j0) = acc[i] * gm;
    }
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {  // tiles above the diagonal: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
    const int zt = wave + 4 * i;   // 0..11: 6 tiles of At, then 6 of P
    const int u = zt % 6, r1 = u < 3 ? 0 : u < 5 ? 1 : 2, r2 = u < 3 ? u + 1 : u < 5 ? u - 1 : 3;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(rec + (zt < 6 ? 2 : 1) * kC * kC + (16 * r1 + idx) * kC + 16 * r2 +
                              4 * grp) = z;
  }
  lds_barrier();  // A complete

  // ---- T = (I + A)^-1 in place: diagonal blocks on wave 0, the others on waves 0 and 1
  invert_unit_lower64(wave == 0 ? sM : nullptr, wave < 2 ? sM : nullptr, wave & 1, lane);

  // ---- T to the record, row-major, zeros above the diagonal
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i, t = e >> 4, j0 = 4 * (e & 15);
    const f32x4 v = *reinterpret_cast<const f32x4*>(sM + t * kLd + j0);
    f32x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = j0 + r <= t ? v[r] : 0.f;
    *reinterpret_cast<f32x4*>(rec + t * kC + j0) = o;
  }
}

// ---- bwd_scan: states forward, state gradients in reverse ---------------------------------
// One pass per (sequence, V head, 16-column tile) on 4 waves; wave w owns token rows
// 16 w .. 16 w + 15 of the chunk products and d_k row tiles w, w + 4 of the carried tile, which
// it holds in registers. Operands are laid out in LDS so that an MFMA fragment (8 values along
// the depth) is two wide reads: the carried tile's copy (hi + lo bf16 pairs for bf16 inputs) and
// the 16-column operands (v or dO^, Y or dV', V' or Z) are stored transposed (a row per column,
// contiguous along the depth), T and P row-major in the forward pass and transposed in the
// reverse pass (whose products take T^T and P^T). K^T and Q^T fragments come from the row-major
// k / q rows: transposing LDS reads for bf16, element reads for fp32. With bf16 inputs both
// passes run side by side in one 8-wave workgroup.
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, const f32x4& x) { *reinterpret_cast<f32x4*>(p) = x; }
// fragment of a row contiguous along the depth, each value scaled by sv[depth]
__device__ __forceinline__ void row_frag_sv(const float* row, const float* sv, int k0, int grp,
                                            f32x8& o) {
  const f32x4 lo = ld4(row + k0 + 4 * grp), hi = ld4(row + k0 + 16 + 4 * grp);
  const f32x4 slo = ld4(sv + k0 + 4 * grp), shi = ld4(sv + k0 + 16 + 4 * grp);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    o[s] = lo[s] * slo[s];
    o[4 + s] = hi[s] * shi[s];
  }
}

// Operand fragments of the scan products in precision mode M (bf16 k / q rows: Bf16Mode, the
// computed fp32 operands carried as hi + lo bf16 pairs; fp32 inputs: F32Mode).
template <typename M>
__device__ __forceinline__ typename M::Op op_frag(const float* row, int k0, int grp) {
  const f32x4 lo = ld4(row + k0 + 4 * grp), hi = ld4(row + k0 + 16 + 4 * grp);
  const float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return M::make(x);
}
template <typename M>
__device__ __forceinline__ typename M::Op op_frag_sv(const float* row, const float* sv, int k0,
                                                     int grp) {
  f32x8 v;
  row_frag_sv(row, sv, k0, grp, v);
  const float x[8] = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
  return M::make(x);
}
// exact fragment of a k / q row (contiguous along the depth)
__device__ __forceinline__ bf16x8 in_frag(const bf16* row, int k0, int grp) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + k0 + 4 * grp);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + k0 + 16 + 4 * grp);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ f32x8 in_frag(const float* row, int k0, int grp) {
  f32x8 o;
  row_frag(row, k0, grp, 1.f, o);
  return o;
}
// exact fragment of a k / q column: lane (idx, grp) gets element (kk, col0 + idx) of rows
// kk = k0 + kslot(grp, s). bf16: two ds_read_b64_tr_b16 over the 16 x 16 blocks of rows k0 and
// k0 + 16 (lane (g, a + 4e) addresses row 4 g + e, columns col0 + 4 a .. + 3 of the block; lane
// (g, i) receives element i of row 4 g + e, for e = 0..3).
template <int KP>
__device__ __forceinline__ bf16x8 in_col_frag(const bf16 (*rows)[KP], int k0, int grp, int col0) {
  const int s = threadIdx.x & 15, a = s & 3, e = s >> 2;
  bf16x8 o;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const bf16* pa = &rows[k0 + 16 * hf + 4 * grp + e][col0 + 4 * a];
    const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(pa));
    const bf16x4 tb = __builtin_bit_cast(bf16x4, t);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[4 * hf + j] = tb[j];
  }
  return o;
}
template <int KP>
__device__ __forceinline__ f32x8 in_col_frag(const float (*rows)[KP], int k0, int grp, int col0) {
  const int idx = threadIdx.x & 15;
  f32x8 o;
#pragma unroll
  for (int s = 0; s < 8; ++s) o[s] = rows[k0 + kslot(grp, s)][col0 + idx];
  return o;
}

// LDS of one scan pass. k / q rows are kept in the input dtype (bf16 exactly), rows padded to
// 16 bytes; the fp32 operands rows padded by 4 floats.
template <typename KT, int D, bool REV>
struct BwdScanLds {
  static constexpr bool kSplit = std::is_same<KT, bf16>::value;  // split-bf16 products
  using XT = std::conditional_t<kSplit, bf16, float>;
  static constexpr int KP = D + 16 / (int)sizeof(KT);  // k / q rows
  static constexpr int XP = D + 16 / (int)sizeof(XT);  // the transposed carried tile
  static constexpr int CP = kC + 4;                    // rows along the tokens
  float sT[kC][CP];            // T (forward), T^T (reverse)
  float sP[REV ? kC : 1][CP];  // P^T (reverse)
  // carried tile (state / gradient)^T as the products read it: hi + lo bf16 pair (split) or fp32
  XT sXh[16][XP];
  XT sXl[kSplit ? 16 : 1][XP];
  float sInT[16][CP];          // (V or dO^ columns)^T
  float sWt[16][CP];           // (Y or dV')^T
  float sZt[16][CP];           // (V' or Z)^T
  float sgam[kC], sdel[kC], sbeta[kC], sgb[kC];
  KT sK[kC][KP];
  KT sQ[REV ? kC : 1][KP];
  float sgc;
};

// Carried-tile copy in LDS: 4 consecutive depth values of column `row` from a C fragment, and
// the B fragment of a product over the depth.
template <typename M, typename L>
__device__ __forceinline__ void store_x(L& S, int row, int col, const f32x4& v) {
  if constexpr (M::kSplit) {
    bf16x4 h, l;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      h[s] = (bf16)v[s];
      l[s] = (bf16)(v[s] - (float)h[s]);
    }
    *reinterpret_cast<bf16x4*>(&S.sXh[row][col]) = h;
    *reinterpret_cast<bf16x4*>(&S.sXl[row][col]) = l;
  } else {
    st4(&S.sXh[row][col], v);
  }
}
template <typename M, typename L>
__device__ __forceinline__ typename M::Op x_frag(const L& S, int row, int k0, int grp) {
  typename M::Op o;
  if constexpr (M::kSplit) {
    o.hi = in_frag(&S.sXh[row][0], k0, grp);
    o.lo = in_frag(&S.sXl[row][0], k0, grp);
  } else {
    row_frag(&S.sXh[row][0], k0, grp, 1.f, o.v);
  }
  return o;
}

// One pass (forward states or reverse state gradients) on 4 waves; `tid` is the thread's index
// among them. Every barrier of a pass is a workgroup barrier: a workgroup that runs both passes
// side by side executes the same number in each.
template <typename InT, typename OT, int D, bool REV>
__device__ __forceinline__ void bwd_scan_pass(const BwdParams& p,
                                              BwdScanLds<InT, D, REV>& S, int tid) {
  constexpr int NB = D / 16;   // column tiles per head
  using M = std::conditional_t<std::is_same<InT, bf16>::value, Bf16Mode, F32Mode>;
  auto& sK = S.sK;
  auto& sQ = S.sQ;
  auto& sT = S.sT;
  auto& sP = S.sP;
  auto& sInT = S.sInT;
  auto& sWt = S.sWt;
  auto& sZt = S.sZt;
  auto& sgam = S.sgam;
  auto& sdel = S.sdel;
  auto& sbeta = S.sbeta;
  auto& sgb = S.sgb;
  float& sgc = S.sgc;

  // The NB column tiles of one (sequence, V head) read the same chunk operands: keep them on one
  // XCD (workgroups are dealt to the 8 XCDs round robin, so blockIdx % 8 picks the XCD).
  const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3;
  const int jt = jj % NB, nh = 8 * (jj / NB) + xcd;
  if (nh >= p.num_seqs * p.hv) return;  // padding workgroup
  const int n = nh / p.hv, h = nh % p.hv;
  const int G = p.hv / p.hqk, m = h / G;
  const int j0 = 16 * jt;
  const int lane = tid & 63, wave = tid >> 6;
  const int idx = lane & 15, grp = lane >> 4;
  const int rw = 16 * wave;
  const int seq0 = p.cu[n], len = p.cu[n + 1] - seq0;
  const int nch = (len + kC - 1) / kC;
  const int sb0 = slot_base(p.cu, n);
  const size_t st_base = (size_t)nh * D * D;

  // carried tile: the initial state (forward) or the final-state gradient (reverse). Wave w
  // holds row tiles w, w + 4, .. of it in registers (lane: rows 4 grp + r, column idx) and keeps
  // the LDS copy the products read.
  constexpr int TPW = (NB + 3) / 4;
  f32x4 xr[TPW];
  const void* init = REV ? p.dht : p.h0;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int rt = wave + 4 * u;
    if (rt < NB) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const size_t e = st_base + (size_t)(16 * rt + 4 * grp + r) * D + j0 + idx;
        xr[u][r] = init ? ld_state(init, e, p.state_bf16) : 0.f;
      }
      store_x<M>(S, idx, 16 * rt + 4 * grp, xr[u]);
    }
  }
  const InT* Q = static_cast<const InT*>(p.q);
  const InT* K = static_cast<const InT*>(p.k);
  const InT* V = static_cast<const InT*>(p.v);
  const OT* dO = static_cast<const OT*>(p.dout);
  __syncthreads();

  // A chunk's global operands (its gates and beta included) are loaded into registers one chunk
  // ahead (16-byte pieces): the next chunk's loads are in flight while this one is computed, and
  // no wait inside a chunk covers them. Rows past the chunk end load row 0 of the chunk and are
  // zeroed when staged.
  constexpr int KV = kC * D / 8 / 256;  // 8-value pieces of the k (q) rows per thread
  static_assert(kC * D % (8 * 256) == 0, "k row pieces");
  using InT2 = std::conditional_t<REV, OT, InT>;  // dO^ (reverse) or v (forward) columns
  Raw8<InT> rk[KV], rq[REV ? KV : 1];
  f32x4 rt[4], rp[REV ? 4 : 1];
  Raw8<InT2> rin;
  double rbb = 0.0, rbl = 0.0;  // b at this lane's row and at the chunk's last row
  float rbt = 0.f;              // beta at this lane's row
  auto load_chunk = [&](int c) {
    const int t0 = seq0 + kC * c, L = min(kC, len - kC * c);
    const float* rec = p.rec + ((size_t)(sb0 + c) * p.hv + h) * kRecFloats;
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int e = tid + 256 * i, row = e / (D / 8), c8 = e % (D / 8);
      const size_t off = ((size_t)(t0 + (row < L ? row : 0)) * p.hqk + m) * D + 8 * c8;
      rk[i].load(K + off);
      if constexpr (REV) rq[i].load(Q + off);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rt[i] = reinterpret_cast<const f32x4*>(rec)[tid + 256 * i];
      if constexpr (REV) rp[i] = reinterpret_cast<const f32x4*>(rec + kC * kC)[tid + 256 * i];
    }
    if (tid < 2 * kC) {
      const int row = tid / 2, half = tid % 2;
      const size_t off = ((size_t)(t0 + (row < L ? row : 0)) * p.hv + h) * D + j0 + 8 * half;
      if constexpr (REV)
        rin.load(dO + off);
      else
        rin.load(V + off);
    }
    if (tid < kC) {
      const double* bb = rec_b(rec);
      rbb = bb[tid];
      rbl = bb[kC - 1];
      rbt = p.beta[(size_t)(t0 + (tid < L ? tid : 0)) * p.hv + h];
    }
  };
  auto stage_chunk = [&](int L) {
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int e = tid + 256 * i, row = e / (D / 8), c8 = e % (D / 8);
      if constexpr (std::is_same<InT, bf16>::value) {  // kept in bf16 (exact), raw 16-byte rows
        *reinterpret_cast<bf16x8*>(&sK[row][8 * c8]) = row < L ? rk[i].r : bf16x8{};
        if constexpr (REV) *reinterpret_cast<bf16x8*>(&sQ[row][8 * c8]) = row < L ? rq[i].r : bf16x8{};
      } else {
        float x[8];
        rk[i].to(x);
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = row < L ? x[u] : 0.f;
        st4(&sK[row][8 * c8], f32x4{x[0], x[1], x[2], x[3]});
        st4(&sK[row][8 * c8 + 4], f32x4{x[4], x[5], x[6], x[7]});
        if constexpr (REV) {
          rq[i].to(x);
#pragma unroll
          for (int u = 0; u < 8; ++u) x[u] = row < L ? x[u] : 0.f;
          st4(&sQ[row][8 * c8], f32x4{x[0], x[1], x[2], x[3]});
          st4(&sQ[row][8 * c8 + 4], f32x4{x[4], x[5], x[6], x[7]});
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * (tid + 256 * i), r = e / kC, cc = e % kC;
      if constexpr (REV) {  // transposed: the reverse products take T^T and P^T
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sT[cc + u][r] = rt[i][u];
          sP[cc + u][r] = rp[i][u];
        }
      } else {
        st4(&sT[r][cc], rt[i]);
      }
    }
    if (tid < 2 * kC) {
      const int row = tid / 2, half = tid % 2;
      float x[8];
      rin.to(x);
      const float sc = REV ? p.scale : 1.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) sInT[8 * half + u][row] = row < L ? sc * x[u] : 0.f;
    }
    if (tid < kC) {
      const float gm = expf((float)rbb), bt = tid < L ? rbt : 0.f;
      sgam[tid] = gm;
      sdel[tid] = expf((float)(rbl - rbb));
      sbeta[tid] = bt;
      sgb[tid] = -gm * bt;
      if (tid == 0) sgc = expf((float)rbl);
    }
  };
  if (nch > 0) load_chunk(REV ? nch - 1 : 0);

  for (int ci = 0; ci < nch; ++ci) {
    const int c = REV ? nch - 1 - ci : ci;
    const int slot = sb0 + c, t0 = seq0 + kC * c, L = min(kC, len - kC * c);
    float* xs = (REV ? p.dhs : p.hs) + ((size_t)slot * p.hv + h) * D * D;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {  // the tile at the chunk boundary
      const int rt = wave + 4 * u;
      if (rt < NB) {
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[(size_t)(16 * rt + 4 * grp + r) * D + j0 + idx] = xr[u][r];
      }
    }
    stage_chunk(L);
    if (ci + 1 < nch) load_chunk(REV ? c - 1 : c + 1);
    __syncthreads();

    // rows rw .. rw + 15 of U = K X
    f32x4 u = zero4();
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 32)
      u = M::mma_xs(u, in_frag(&sK[rw + idx][0], k0, grp), x_frag<M>(S, idx, k0, grp));
    if constexpr (!REV) {  // Y = V - diag(gamma) U
      const f32x4 vv = ld4(&sInT[idx][rw + 4 * grp]), gm = ld4(&sgam[rw + 4 * grp]);
      f32x4 y;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rw + 4 * grp + r;
        y[r] = vv[r] - gm[r] * u[r];
        if (t < L) p.ys[((size_t)(t0 + t) * p.hv + h) * D + j0 + idx] = y[r];
      }
      st4(&sWt[idx][rw + 4 * grp], y);
    } else {  // dV' = P^T dO^ + diag(delta) U
      f32x4 pd = zero4();
#pragma unroll
      for (int k0 = 0; k0 < kC; k0 += 32)
        pd = M::mma_ss(pd, op_frag<M>(&sP[rw + idx][0], k0, grp),
                       op_frag<M>(&sInT[idx][0], k0, grp));
      const f32x4 dl = ld4(&sdel[rw + 4 * grp]);
      f32x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = pd[r] + dl[r] * u[r];
      st4(&sWt[idx][rw + 4 * grp], w);
    }
    __syncthreads();
    if constexpr (!REV) {  // V' = T diag(beta) Y
      f32x4 vpr = zero4();
#pragma unroll
      for (int k0 = 0; k0 < kC; k0 += 32)
        vpr = M::mma_ss(vpr, op_frag<M>(&sT[rw + idx][0], k0, grp),
                        op_frag_sv<M>(&sWt[idx][0], sbeta, k0, grp));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rw + 4 * grp + r;
        if (t < L) p.vp[((size_t)(t0 + t) * p.hv + h) * D + j0 + idx] = vpr[r];
      }
      st4(&sZt[idx][rw + 4 * grp], vpr);
    } else {  // Z = T^T dV';  dv = dY = diag(beta) Z
      f32x4 z = zero4();
#pragma unroll
      for (int k0 = 0; k0 < kC; k0 += 32)
        z = M::mma_ss(z, op_frag<M>(&sT[rw + idx][0], k0, grp), op_frag<M>(&sWt[idx][0], k0, grp));
      InT* dV = static_cast<InT*>(p.dv);
      const f32x4 bt = ld4(&sbeta[rw + 4 * grp]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rw + 4 * grp + r;
        if (t < L) {
          const size_t off = ((size_t)(t0 + t) * p.hv + h) * D + j0 + idx;
          p.zs[off] = z[r];
          dV[off] = from_f32<InT>(bt[r] * z[r]);
        }
      }
      st4(&sZt[idx][rw + 4 * grp], z);
    }
    __syncthreads();
    // carried tile update, its 16-row tiles dealt to the waves (K^T, Q^T fragments by transposing
    // reads of the row-major k / q rows; the right operands, rows of the transposed 16-column
    // tiles, read as fragments once for all of a wave's tiles)
    typename M::Op bz[kC / 32], bi[REV ? kC / 32 : 1];
#pragma unroll
    for (int ks = 0; ks < kC / 32; ++ks) {
      bz[ks] = op_frag_sv<M>(&sZt[idx][0], REV ? sgb : sdel, 32 * ks, grp);
      if constexpr (REV) bi[ks] = op_frag_sv<M>(&sInT[idx][0], sgam, 32 * ks, grp);
    }
#pragma unroll
    for (int uu = 0; uu < TPW; ++uu) {
      const int rt = wave + 4 * uu;
      if (rt >= NB) break;
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sgc * xr[uu][r];
#pragma unroll
      for (int ks = 0; ks < kC / 32; ++ks) {
        // + K^T diag(delta) V' (forward);  - K^T diag(gamma) diag(beta) Z + Q^T diag(gamma) dO^
        acc = M::mma_xs(acc, in_col_frag(sK, 32 * ks, grp, 16 * rt), bz[ks]);
        if constexpr (REV) acc = M::mma_xs(acc, in_col_frag(sQ, 32 * ks, grp, 16 * rt), bi[ks]);
      }
      xr[uu] = acc;
      store_x<M>(S, idx, 16 * rt + 4 * grp, acc);
    }
    __syncthreads();
  }
  if (REV && p.dh0) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int rt = wave + 4 * u;
      if (rt < NB) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st_state(p.dh0, st_base + (size_t)(16 * rt + 4 * grp + r) * D + j0 + idx, xr[u][r],
                   p.state_bf16);
      }
    }
  }
}

template <typename InT, typename OT, int D, bool REV>
__global__ __launch_bounds__(256) void bwd_scan_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) BwdScanLds<InT, D, REV> S;
  bwd_scan_pass<InT, OT, D, REV>(p, S, threadIdx.x);
}

// Both passes side by side (they read the same records and neither needs the other's output):
// waves 0-3 run the forward pass, waves 4-7 the reverse one, so that each hides the other's
// latencies. Used where both LDS sets fit one CU (bf16 k / q rows).
template <typename InT, typename OT, int D>
__global__ __launch_bounds__(512) void bwd_scan2_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) BwdScanLds<InT, D, false> Sf;
  __shared__ __attribute__((aligned(16))) BwdScanLds<InT, D, true> Sr;
  if (threadIdx.x < 256)
    bwd_scan_pass<InT, OT, D, false>(p, Sf, threadIdx.x);
  else
    bwd_scan_pass<InT, OT, D, true>(p, Sr, threadIdx.x - 256);
}

// Fragment of an operand whose values are representable in the fragment type of mode M.
template <typename M>
__device__ __forceinline__ typename M::frag_t exact_frag(const float (&x)[8]) {
  typename M::frag_t o;
#pragma unroll
  for (int s = 0; s < 8; ++s) o[s] = x[s];
  return o;
}
// ---- bwd_grads --------------------------------------------------------------------------------
// 512 threads, two waves per SIMD. For the products with the states (R1..R3) and the dq / dk
// tiles, wave w owns one d_k column tile (w % NB) and NB / 2 of the 4 row tiles: a state-row
// fragment is loaded once and used for all of them. For the C x C tiles (dP, dA) it owns row tile
// w % 4 and half of the columns. Row sums spanning several waves meet in LDS.
template <typename InT, typename OT, int D>
__global__ __launch_bounds__(512) void bwd_grads_kernel(BwdParams p) {
  constexpr int KP = D + 4;
  constexpr int NB = D / 16;
  constexpr int RPW = NB / 2;  // row tiles per wave in the R / dq / dk products
  static_assert(NB % 2 == 0 && 4 * NB == 8 * RPW, "tile split");
  __shared__ __attribute__((aligned(16))) float sK[kC][KP];
  __shared__ __attribute__((aligned(16))) float sQ[kC][KP];
  // One region serves two phases: the R products' operand slab (dO^, Z diag(beta) and V' of
  // SR rows of the chunk over the whole depth, rows padded to SLD floats), then dP o Gamma, dS
  // and E.
  constexpr int SR = 32, SLD = D + 4;
  constexpr int SLAB = 3 * SR * SLD, PGE = 3 * kC * (kC + 1);
  __shared__ __attribute__((aligned(16))) float sU[SLAB > PGE ? SLAB : PGE];
  float (*const sPG)[kC + 1] = reinterpret_cast<float (*)[kC + 1]>(sU);                // dP o Gamma
  float (*const sDS)[kC + 1] = reinterpret_cast<float (*)[kC + 1]>(sU + kC * (kC + 1));  // dS
  float (*const sE)[kC + 1] = reinterpret_cast<float (*)[kC + 1]>(sU + 2 * kC * (kC + 1));  // E
  __shared__ double sb[kC];
  __shared__ float sbeta[kC], sgam[kC], sdel[kC];
  __shared__ float sfe[8][kC];       // per wave: sum over its rows t >= s of sum_{j<s} E_tj
  __shared__ float sga[kC];          // gamma_t (<Q_t, R1_t> - <K_t, R2_t>)
  __shared__ float sdc[kC];          // delta_t <K_t, R3_t>
  __shared__ float sbt[kC];          // sum_j dA_tj At_tj
  __shared__ float sred[8];

  const int slot = blockIdx.x / p.hqk, m = blockIdx.x % p.hqk;
  const int G = p.hv / p.hqk;
  int n, t0, L;
  if (slot >= p.num_slots || !slot_chunk(p, slot, n, t0, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int idx = lane & 15, grp = lane >> 4;
  const int rw = 16 * (wave & 3);  // this wave's rows in the C x C products
  const int ch = wave >> 2;        // this wave's column half of the C x C products
  const int ctw = wave % NB;       // this wave's d_k column tile in the R / dq / dk products
  const int rt0 = (wave / NB) * RPW;  // and its first row tile there
  // bf16 inputs: the products with the states (R1..R3) and the dq / dk products on bf16 MFMA,
  // k / q and a bf16 dO exact, the other operands split hi + lo. The C x C products (dP, dA) stay
  // on fp32 MFMA: dg sums their entries with cancellation, and split operands there double its
  // error.
  using MR = std::conditional_t<std::is_same<InT, bf16>::value, Bf16Mode, F32Mode>;
  constexpr bool kDoXR = MR::kSplit && std::is_same<OT, bf16>::value;  // dO values exact

  const InT* Q = static_cast<const InT*>(p.q);
  const InT* K = static_cast<const InT*>(p.k);
  const OT* dO = static_cast<const OT*>(p.dout);
  {  // k / q rows of the chunk as 8-value pieces, every load of a thread issued at once
    constexpr int NPc = kC * D / 8, PPT = (NPc + 511) / 512;
    Raw8<InT> rk[PPT], rq[PPT];
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int e = tid + 512 * u, i = e / (D / 8), c8 = e % (D / 8);
      if (e < NPc) {
        const size_t off = ((size_t)(t0 + (i < L ? i : 0)) * p.hqk + m) * D + 8 * c8;
        rk[u].load(K + off);
        rq[u].load(Q + off);
      }
    }
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int e = tid + 512 * u, i = e / (D / 8), c8 = e % (D / 8);
      if (e < NPc) {
        float xk[8], xq[8];
        rk[u].to(xk);
        rq[u].to(xq);
        const bool ok = i < L;
        *reinterpret_cast<f32x4*>(&sK[i][8 * c8]) = ok ? f32x4{xk[0], xk[1], xk[2], xk[3]} : zero4();
        *reinterpret_cast<f32x4*>(&sK[i][8 * c8 + 4]) = ok ? f32x4{xk[4], xk[5], xk[6], xk[7]} : zero4();
        *reinterpret_cast<f32x4*>(&sQ[i][8 * c8]) = ok ? f32x4{xq[0], xq[1], xq[2], xq[3]} : zero4();
        *reinterpret_cast<f32x4*>(&sQ[i][8 * c8 + 4]) = ok ? f32x4{xq[4], xq[5], xq[6], xq[7]} : zero4();
      }
    }
  }

  f32x4 dq[RPW], dk[RPW];
#pragma unroll
  for (int u = 0; u < RPW; ++u) dq[u] = dk[u] = zero4();

  for (int jh = 0; jh < G; ++jh) {
    const int h = m * G + jh;
    const float* rec = p.rec + ((size_t)slot * p.hv + h) * kRecFloats;
    const float* Pm = rec + kC * kC;
    const float* At = rec + 2 * kC * kC;
    const float* H = p.hs + ((size_t)slot * p.hv + h) * D * D;
    const float* dH = p.dhs + ((size_t)slot * p.hv + h) * D * D;
    if (tid < kC) {
      const double* bb = rec_b(rec);
      sb[tid] = bb[tid];
      sgam[tid] = expf((float)bb[tid]);
      sdel[tid] = expf((float)(bb[kC - 1] - bb[tid]));
      sbeta[tid] = tid < L ? p.beta[(size_t)(t0 + tid) * p.hv + h] : 0.f;
      sga[tid] = sdc[tid] = sbt[tid] = 0.f;
    }
    __syncthreads();

    auto row_off = [&](int t) { return ((size_t)(t0 + t) * p.hv + h) * D; };
    // this lane's A rows (row rw + idx of the chunk)
    const bool my_ok = rw + idx < L;
    const OT* my_dO = dO + row_off(my_ok ? rw + idx : 0);  // zero scale past the chunk end
    const float* my_Z = p.zs + row_off(my_ok ? rw + idx : 0);
    // R1 = dO^ H^T, R2 = dY H^T, R3 = V' dH'^T (this wave's d_k column tile, RPW row tiles) into
    // dq, dk and the row sums of db. The state rows of the column tile are loaded once per depth
    // step and shared by the row tiles; the waves of the first row-tile group also sum
    // H o dH' over them (each state element once).
    float hdh = 0.f;
    {
      // The A operands are staged in LDS SR = 32 rows (two row tiles) at a time over the whole
      // depth, with one coalesced load of each 16-byte piece (rows past the chunk end: zeros);
      // each wave reads its state fragments from global memory once, for both row groups.
      const int c0 = 16 * ctw;
      const float* hrow = H + (size_t)(c0 + idx) * D;
      const float* dhrow = dH + (size_t)(c0 + idx) * D;
      constexpr int KS = D / 32, PR = D / 4, NPS = 3 * SR * PR, PPS = (NPS + 511) / 512;
      constexpr int UPG = SR / 16;  // row tiles per group
      f32x8 hb[KS], dhb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        row_frag(hrow, 32 * ks, grp, 1.f, hb[ks]);
        row_frag(dhrow, 32 * ks, grp, 1.f, dhb[ks]);
      }
      if (rt0 == 0) {  // <H, dH'>: each state element once over the waves of row-tile group 0
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) hdh = fmaf(hb[ks][e], dhb[ks][e], hdh);
      }
      typename MR::Op ho[KS], dho[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float xh[8] = {hb[ks][0], hb[ks][1], hb[ks][2], hb[ks][3],
                             hb[ks][4], hb[ks][5], hb[ks][6], hb[ks][7]};
        const float xd[8] = {dhb[ks][0], dhb[ks][1], dhb[ks][2], dhb[ks][3],
                             dhb[ks][4], dhb[ks][5], dhb[ks][6], dhb[ks][7]};
        ho[ks] = MR::make(xh);
        dho[ks] = MR::make(xd);
      }
#pragma unroll
      for (int g0 = 0; g0 < kC; g0 += SR) {
        f32x4 pc[PPS];
#pragma unroll
        for (int i = 0; i < PPS; ++i) {
          const int pi = tid + 512 * i, op = pi / (SR * PR), row = g0 + (pi / PR) % SR;
          const size_t off = row_off(row < L ? row : 0) + 4 * (pi % PR);
          if (pi < NPS) {
            if (op == 0) {
              if constexpr (std::is_same<OT, bf16>::value) {
                const bf16x4 b = *reinterpret_cast<const bf16x4*>(dO + off);
                pc[i] = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
              } else {
                pc[i] = *reinterpret_cast<const f32x4*>(dO + off);
              }
            } else {
              pc[i] = *reinterpret_cast<const f32x4*>((op == 1 ? p.zs : p.vp) + off);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < PPS; ++i) {
          const int pi = tid + 512 * i, op = pi / (SR * PR), rl = (pi / PR) % SR, row = g0 + rl;
          if (pi < NPS) {
            const float sc = row >= L ? 0.f : op == 1 ? sbeta[row] : 1.f;  // dO^ = scale dO: later
            *reinterpret_cast<f32x4*>(sU + (op * SR + rl) * SLD + 4 * (pi % PR)) = pc[i] * sc;
          }
        }
        __syncthreads();  // rows g0 .. g0 + SR - 1 staged
        // this wave's row tiles of the group (rt0 .. rt0 + RPW - 1 intersected with the group)
#pragma unroll
        for (int uu = 0; uu < UPG; ++uu) {
          const int rtile = g0 / 16 + uu, u = rtile - rt0;
          if (u < 0 || u >= RPW) continue;  // uniform over the wave
          const int rl = 16 * uu + idx;
          f32x4 r1 = zero4(), r2 = zero4(), r3 = zero4();
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            float ao[8], az[8], av[8];
            {
              f32x8 f;
              row_frag(sU + rl * SLD, 32 * ks, grp, 1.f, f);
#pragma unroll
              for (int e = 0; e < 8; ++e) ao[e] = f[e];
              row_frag(sU + (SR + rl) * SLD, 32 * ks, grp, 1.f, f);
#pragma unroll
              for (int e = 0; e < 8; ++e) az[e] = f[e];
              row_frag(sU + (2 * SR + rl) * SLD, 32 * ks, grp, 1.f, f);
#pragma unroll
              for (int e = 0; e < 8; ++e) av[e] = f[e];
            }
            if constexpr (kDoXR)
              r1 = MR::mma_xs(r1, exact_frag<MR>(ao), ho[ks]);
            else
              r1 = MR::mma_ss(r1, MR::make(ao), ho[ks]);
            r2 = MR::mma_ss(r2, MR::make(az), ho[ks]);
            r3 = MR::mma_ss(r3, MR::make(av), dho[ks]);
          }
          r1 *= p.scale;
          float rs[4], rd[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * rtile + 4 * grp + r, cc = c0 + idx;
            const float dqv = sgam[t] * r1[r];
            const float dkv = sdel[t] * r3[r] - sgam[t] * r2[r];
#pragma unroll
            for (int w = 0; w < RPW; ++w)
              if (w == u) {
                dq[w][r] += dqv;
                dk[w][r] += dkv;
              }
            rs[r] = sgam[t] * (sQ[t][cc] * r1[r] - sK[t][cc] * r2[r]);
            rd[r] = sdel[t] * sK[t][cc] * r3[r];
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
              rs[r] += __shfl_xor(rs[r], off);
              rd[r] += __shfl_xor(rd[r], off);
            }
            if (idx == 0) {
              atomicAdd(&sga[t], rs[r]);
              atomicAdd(&sdc[t], rd[r]);
            }
          }
        }
        __syncthreads();  // group consumed
      }
    }
    // dP = dO^ V'^T (lower-incl), dA = -Z V'^T (strictly lower): this wave's two column tiles
    float rbeta[4] = {0.f, 0.f, 0.f, 0.f};
    float at_v[2][4], pm_v[2][4];  // this lane's At and P entries, loaded ahead of the products
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rw + 4 * grp + r, j = 16 * (2 * ch + u) + idx;
        at_v[u][r] = At[t * kC + j];
        pm_v[u][r] = Pm[t * kC + j];
      }
    // both column tiles in one pass over the depth: this lane's dO and Z fragments are loaded
    // once for the four products (V' rows past the chunk end are read as row 0 of the chunk and
    // masked below)
    f32x4 dpv[2] = {zero4(), zero4()}, zav[2] = {zero4(), zero4()};
    {
      const int j0 = 32 * ch + idx, j1 = 32 * ch + 16 + idx;
      const float* vp0 = p.vp + row_off(j0 < L ? j0 : 0);
      const float* vp1 = p.vp + row_off(j1 < L ? j1 : 0);
      const float am = my_ok ? 1.f : 0.f;
#pragma unroll 2
      for (int k0 = 0; k0 < D; k0 += 32) {
        f32x8 ao, az, b0, b1;
        row_frag(my_dO, k0, grp, am, ao);
        row_frag(my_Z, k0, grp, am, az);
        row_frag(vp0, k0, grp, 1.f, b0);
        row_frag(vp1, k0, grp, 1.f, b1);
        dpv[0] = mma32(ao, b0, dpv[0]);
        zav[0] = mma32(az, b0, zav[0]);
        dpv[1] = mma32(ao, b1, dpv[1]);
        zav[1] = mma32(az, b1, zav[1]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c0 = 16 * (2 * ch + u);
      const f32x4 dp = p.scale * dpv[u];
      const f32x4 za = zav[u];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = rw + 4 * grp + r, j = c0 + idx;
        const float gam = t >= j ? expf((float)(sb[t] - sb[j])) : 0.f;
        const float dPm = t >= j ? dp[r] : 0.f;
        const float dAm = t > j ? -za[r] : 0.f;
        const float at = at_v[u][r];
        sPG[t][j] = dPm * gam;
        sDS[t][j] = dAm * sbeta[t] * gam;
        sE[t][j] = dPm * pm_v[u][r] + dAm * sbeta[t] * at;
        rbeta[r] += dAm * at;
      }
    }
    // row sums of rbeta over the 16 lanes of each row group, then across the waves through LDS
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) rbeta[r] += __shfl_xor(rbeta[r], off);
    }
    if (idx == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) atomicAdd(&sbt[rw + 4 * grp + r], rbeta[r]);
    }
    // <H, dH'> over the whole head: accumulated from the state fragments of the R products
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) hdh += __shfl_xor(hdh, off);
    if (lane == 0) sred[wave] = hdh;
    // <Y_t, Z_t>: wave w takes rows 8 w + 2 grp + r (r = 0, 1), D / 16 consecutive values per
    // lane; rows past the chunk end read row 0 and are dropped at the store
    float yz[2];
    {
      constexpr int CPL = D / 16;  // values per lane
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int t = 8 * wave + 2 * grp + r;
        const float* yr = p.ys + row_off(t < L ? t : 0) + CPL * idx;
        const float* zr = p.zs + row_off(t < L ? t : 0) + CPL * idx;
        float acc = 0.f;
        if constexpr (CPL % 4 == 0) {
#pragma unroll
          for (int c = 0; c < CPL; c += 4) {
            const f32x4 y4 = ld4(yr + c), z4 = ld4(zr + c);
            acc = fmaf(y4[0], z4[0], fmaf(y4[1], z4[1], fmaf(y4[2], z4[2], fmaf(y4[3], z4[3], acc))));
          }
        } else {
#pragma unroll
          for (int c = 0; c < CPL; c += 2) {
            const float2 y2 = *reinterpret_cast<const float2*>(yr + c);
            const float2 z2 = *reinterpret_cast<const float2*>(zr + c);
            acc = fmaf(y2.x, z2.x, fmaf(y2.y, z2.y, acc));
          }
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off);
        yz[r] = acc;
      }
    }
    __syncthreads();  // sPG, sDS, sE, sga, sdc, sbt, sred complete
    if (idx == 0) {  // dbeta_t = <Y_t, Z_t> + sum_j dA_tj At_tj
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int t = 8 * wave + 2 * grp + r;
        if (t < L) p.dbeta[(size_t)(t0 + t) * p.hv + h] = yz[r] + sbt[t];
      }
    }
    {  // sum_{t >= s} sum_{j < s} E_tj: wave w takes rows 8 w .. 8 w + 7, lane = s; each row's
       // exclusive prefix along j by a wave scan
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = 8 * wave + i;
        const float e = sE[t][lane];
        const float pre = wave_inclusive_scan(e, lane) - e;
        if (t >= lane) part += pre;
      }
      sfe[wave][lane] = part;
    }
    __syncthreads();
    if (wave == 0) {
      float fe = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) fe += sfe[w][lane];
      // suffix sum of sga (reverse inclusive scan), prefix sum of sdc (exclusive)
      const float ga_rev = sga[kC - 1 - lane];  // lane l: row 63 - l
      const float suf = __shfl(wave_inclusive_scan(ga_rev, lane), kC - 1 - lane);
      const float dcv = sdc[lane];
      const float pre = wave_inclusive_scan(dcv, lane) - dcv;
      float hs8 = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) hs8 += sred[w];
      const float hdhs = sgam[kC - 1] * hs8;
      if (lane < L) p.dg[(size_t)(t0 + lane) * p.hv + h] = suf + pre + hdhs + fe;
    }
    // dQ += (dP o Gamma) K;  dK += (dP o Gamma)^T Q + (dS + dS^T) K  (this wave's tiles)
    // (the k / q column fragments of a depth step are read once for all of this wave's row tiles;
    // on bf16 MFMA they are exact and the left operands split)
    auto mma_sx = [](f32x4 acc, const float (&xa)[8], const typename MR::frag_t& fb) {
      const typename MR::Op oa = MR::make(xa);
      if constexpr (MR::kSplit) {
        acc = mma32(oa.hi, fb, acc);
        return mma32(oa.lo, fb, acc);
      } else {
        return mma32(oa.v, fb, acc);
      }
    };
#pragma unroll 1
    for (int k0 = 0; k0 < kC; k0 += 32) {
      const int c0 = 16 * ctw;
      float xk[8], xq[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int kk = k0 + kslot(grp, s);
        xk[s] = sK[kk][c0 + idx];
        xq[s] = sQ[kk][c0 + idx];
      }
      const typename MR::frag_t fk = exact_frag<MR>(xk), fq = exact_frag<MR>(xq);
#pragma unroll
      for (int u = 0; u < RPW; ++u) {
        const int ri = 16 * (rt0 + u) + idx;
        float a1[8], a2[8], a3[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int kk = k0 + kslot(grp, s);
          a1[s] = sPG[ri][kk];
          a2[s] = sPG[kk][ri];
          a3[s] = sDS[ri][kk] + sDS[kk][ri];
        }
        dq[u] = mma_sx(dq[u], a1, fk);
        dk[u] = mma_sx(dk[u], a2, fq);
        dk[u] = mma_sx(dk[u], a3, fk);
      }
    }
    __syncthreads();  // LDS reused by the next V head
  }

  InT* dQo = static_cast<InT*>(p.dq);
  InT* dKo = static_cast<InT*>(p.dk);
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * (rt0 + u) + 4 * grp + r;
      if (t < L) {
        const size_t off = ((size_t)(t0 + t) * p.hqk + m) * D + 16 * ctw + idx;
        dQo[off] = from_f32<InT>(dq[u][r]);
        dKo[off] = from_f32<InT>(dk[u][r]);
      }
    }
  }
}

// Workspace sections, each rounded to 256 bytes.
struct BwdLayout {
  size_t rec, hs, dhs, ys, vp, zs, total;  // float offsets, total in floats
};
inline size_t round64(size_t x) { return (x + 63) / 64 * 64; }
inline BwdLayout bwd_layout(const gdn_shape_t& s) {
  const size_t slots = (size_t)chunk_slots(s), hv = (size_t)s.num_v_heads, d = (size_t)s.head_dim_k;
  const size_t rows = (size_t)s.total_tokens * hv * d;
  BwdLayout L{};
  L.rec = 0;
  L.hs = L.rec + round64(slots * hv * kRecFloats);
  L.dhs = L.hs + round64(slots * hv * d * d);
  L.ys = L.dhs + round64(slots * hv * d * d);
  L.vp = L.ys + round64(rows);
  L.zs = L.vp + round64(rows);
  L.total = L.zs + round64(rows);
  return L;
}

template <typename InT, typename OT, int D>
hipError_t launch_bwd_t(const gdn_shape_t& s, BwdParams p, hipStream_t stream) {
  // chunk slots dealt to the 8 XCDs round robin, the H_v workgroups of a slot back to back on
  // its XCD (a token's gates share a cache line; a QK head's G V heads share its q/k rows)
  const unsigned intra_blocks = (unsigned)(8 * p.hv * (((long long)p.num_slots + 7) / 8));
  const unsigned slot_blocks_qk = (unsigned)(p.num_slots * p.hqk);
  const unsigned scan_blocks = (unsigned)(8 * (D / 16) * ((s.num_seqs * s.num_v_heads + 7) / 8));
  if (s.total_tokens > 0) {
    hipLaunchKernelGGL((bwd_intra_kernel<InT, D>), dim3(intra_blocks), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // The reverse pass also runs for empty sequences (dh0 = dht there); the forward pass of an
  // empty sequence writes nothing.
  if constexpr (std::is_same<InT, bf16>::value) {  // both passes in one workgroup
    hipLaunchKernelGGL((bwd_scan2_kernel<InT, OT, D>), dim3(scan_blocks), dim3(512), 0, stream, p);
  } else {
    if (s.total_tokens > 0) {
      hipLaunchKernelGGL((bwd_scan_kernel<InT, OT, D, false>), dim3(scan_blocks), dim3(256), 0,
                         stream, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_scan_kernel<InT, OT, D, true>), dim3(scan_blocks), dim3(256), 0,
                       stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || s.total_tokens == 0) return e;
  hipLaunchKernelGGL((bwd_grads_kernel<InT, OT, D>), dim3(slot_blocks_qk), dim3(512), 0, stream,
                     p);
  return hipGetLastError();
}

template <typename InT, typename OT>
hipError_t launch_bwd_d(const gdn_shape_t& s, const BwdParams& p, hipStream_t stream) {
  switch (s.head_dim_k) {
    case 32: return launch_bwd_t<InT, OT, 32>(s, p, stream);
    case 64: return launch_bwd_t<InT, OT, 64>(s, p, stream);
    case 128: return launch_bwd_t<InT, OT, 128>(s, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

long long chunk_backward_workspace_floats(const gdn_shape_t& s) {
  return (long long)bwd_layout(s).total;
}

hipError_t launch_chunk_backward(const gdn_shape_t& s, const int32_t* cu, const void* q,
                                 const void* k, const void* v, const float* g, const float* beta,
                                 const void* h0, const void* dout, const void* dht, void* dq,
                                 void* dk, void* dv, float* dg, float* dbeta, void* dh0, void* ws,
                                 hipStream_t stream) {
  const BwdLayout L = bwd_layout(s);
  float* w = static_cast<float*>(ws);
  BwdParams p{cu, q, k, v, g, beta, h0, dout, dht, dq, dk, dv, dg, dbeta, dh0,
              w + L.rec, w + L.hs, w + L.dhs, w + L.ys, w + L.vp, w + L.zs,
              s.num_seqs, s.total_tokens, s.num_qk_heads, s.num_v_heads,
              (int)chunk_slots(s), s.scale, s.state_dtype == GDN_DTYPE_BF16 ? 1 : 0};
  const bool in_bf = s.qkv_dtype == GDN_DTYPE_BF16, out_bf = s.out_dtype == GDN_DTYPE_BF16;
  if (in_bf && out_bf) return launch_bwd_d<bf16, bf16>(s, p, stream);
  if (in_bf) return launch_bwd_d<bf16, float>(s, p, stream);
  if (out_bf) return launch_bwd_d<float, bf16>(s, p, stream);
  return launch_bwd_d<float, float>(s, p, stream);
}

}  // namespace gdn
