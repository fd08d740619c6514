// gdn_scan_tiles.hip -- sequential cross-chunk recurrence of the chunked prefill for many
// (sequence, V head) chains, bf16 q/k/v ([MoE report] §3.7 Steps 5-7), from the workspace the
// intra kernel filled.
//
// Per chunk of 64 tokens, with H the [d_k][d_v] state at the chunk start, b the in-chunk cumsum
// of g (gamma_t = e^{b_t}, delta_t = e^{b_C - b_t}), T diag(beta) and P from the workspace:
//   Y   = V - diag(gamma) K H
//   V'  = (T diag(beta)) Y
//   H  <- gamma_C H + K^T diag(delta) V'
//   O^T = scale ( H^T Q^T diag(gamma) + V'^T P^T )     (the output, computed transposed)
// Columns of H evolve independently. A workgroup owns NT tiles of 16 d_v columns of one
// (sequence, V head) chain and has three kinds of waves:
//   * chain wave t (one per tile) runs the recurrence of tile t: its [d_k x 16] fp32 state slice
//     stays in its registers for the whole sequence. Per chunk it forms Y, V' and the new state,
//     and hands the state (as fp16 operand fragments) and V' to the output wave through LDS.
//   * output wave t forms the output rows of tile t from Q, the state and V'. The output
//     is computed transposed, so a lane holds 4 consecutive columns of one token and stores them
//     straight to global memory.
//   * four producer waves stage chunk c+1 (K, Q and v rows, T diag(beta), P, gamma, delta)
//     into LDS while chunk c is computed, from registers loaded one chunk earlier, and build the
//     K^T fragments of the state update from the K rows they staged (transposing LDS reads), so
//     that the chain waves read every operand with plain 16-byte LDS reads.
// On gfx950 a wave's LDS reads, LDS writes, MFMAs and vector ALU instructions hardly overlap with
// one another, while those of different waves on a SIMD do; the chain wave is the serial path,
// so it issues only the recurrence itself, and everything else is done by the other waves.
// Three s_barriers per chunk order the hand-overs (see the schedule below the work assignment).
// Products run on MFMA in the fragment convention of gdn_device.hpp: the two with the state
// (K H, Q H) on fp16 operands (Half); T diag(beta) Y, P V' and the update K^T diag(delta) V' on
// bf16, computed operands as hi + lo pairs.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.h"

namespace gdn {
namespace {

struct TilesParams {
  const int32_t* cu;
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const void* h0;  // initial states, fp32 or bf16 (state_bf16), or null
  void* o;
  void* ht;  // final states, same dtype, or null
  const char* ws;
  int num_seqs, hqk, hv;
  float scale;
  int state_bf16;
};

// d_k index of row m of state tile `it` (16 rows): tiles 2 kb and 2 kb + 1 interleave their
// 4-row groups inside the 32 columns of block kb, so that the C fragments of the two tiles
// stack into a B fragment whose slot s of lane group grp is d_k index 32 kb + 8 grp + s (the
// order of a 16-byte row piece).
__device__ __forceinline__ int st_row(int it, int m) {
  return 32 * (it >> 1) + 8 * (m >> 2) + 4 * (it & 1) + (m & 3);
}

// 4 output values of one token row (4 consecutive columns).
template <typename OutT>
__device__ __forceinline__ void store4(OutT* p, const f32x4& x);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const f32x4& x) {
  bf16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (bf16)x[e];
  *reinterpret_cast<bf16x4*>(p) = r;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const f32x4& x) {
  *reinterpret_cast<f32x4*>(p) = x;
}

template <int D, int NT>
struct TilesCfg {
  static constexpr int KB = D / 32;                    // 32-deep blocks over d_k
  static constexpr int NST = D / 16;                   // 16-row state tiles
  static constexpr int ROWB = 2 * D;                   // bytes of one q / k row
  static constexpr int KBYTES = 64 * ROWB;             // K (or Q) rows of a chunk
  static constexpr int KU = KBYTES / 1024;             // ... in 1 KiB units
  static constexpr int NCH = ROWB / 16, RPU = 64 / NCH;  // 16-byte pieces per row, rows per unit
  static constexpr int KTBYTES = NST * 2 * 1024;       // K^T fragments: (state tile, 32 tokens)
  static constexpr int TBYTES = kWsMatBytes;           // T diag(beta) (or P) blocks of a record
  static constexpr int TU = TBYTES / 1024;             // ... in 1 KiB units
  static constexpr int VROWB = 32;                     // one row of a 16-column bf16 tile
  static constexpr int VSTR = NT * VROWB + 16;         // padded stride: tile reads spread banks
  static constexpr int VPR = NT * VROWB / 16;          // 16-byte pieces per staged v row
  static constexpr int VU = 64 * VPR / 64;             // v units
  static constexpr int HXB = KB * 1024;                // exchanged fp16 state of one tile
  static constexpr int VXB = 4 * 1024;                 // exchanged V' of one tile (4 C fragments)
  // LDS: each piece is staged once per chunk, at a point of the chunk where its previous
  // contents are no longer read; only the K^T fragments (built while the previous ones are in
  // use) are double buffered.
  static constexpr int KOFF = 0, QOFF = KBYTES, VOFF = 2 * KBYTES;
  static constexpr int TOFF = VOFF + 64 * VSTR, POFF = TOFF + TBYTES, GOFF = POFF + TBYTES;
  static constexpr int KTOFF = GOFF + 512;             // two K^T buffers
  static constexpr int XOFF = KTOFF + 2 * KTBYTES;     // per tile: split state, then V'
  static constexpr int XB = HXB + VXB;
  static constexpr int LDS = XOFF + NT * XB;
  static constexpr int NP = 4;                         // producers: 16 rows of K and Q each
  static constexpr int KPER = KU / NP;                 // K (and Q) units per producer
  static constexpr int VPER = (VU + NP - 1) / NP;      // v units per producer (round robin)
  static constexpr int TPER = (TU + NP - 1) / NP;      // T (and P) units per producer (at most)
  static constexpr int NW = 2 * NT + NP;               // chain waves, output waves, producers
  static constexpr int THREADS = 64 * NW;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(KU % NP == 0 && KPER * RPU == 16, "a producer stages 16 whole K rows");
  static_assert(NW <= 16, "waves per workgroup");
};

constexpr int kSortSeqs = 64;  // batches of up to this many sequences run longest first

template <int D, int NT, typename OutT>
__global__ __launch_bounds__((TilesCfg<D, NT>::THREADS)) void chunk_scan_tiles_kernel(TilesParams p) {
  using C = TilesCfg<D, NT>;
  using M = Bf16Mode;
  using Op = M::Op;
  constexpr int KB = C::KB, NST = C::NST;
  constexpr int NB = D / 16 / NT;  // column groups (workgroups) per chain

  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63, idx = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches

  // Work assignment. The hardware deals workgroups round robin over the 8 XCDs (b % 8). A unit
  // (sequence, QK head) has G * NB workgroups (its V heads x column groups) that read the same
  // q/k rows: they stay on one XCD (one L2) and are dispatched back to back. Units go to the
  // XCDs round robin in order of decreasing sequence length (ties by index), so that every XCD
  // gets an equal share of a packed batch of uneven sequences, longest chains first.
  const int G = p.hv / p.hqk;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int u = 8 * (j / (G * NB)) + xcd, w = j % (G * NB), dvb = w % NB;
  if (u >= p.num_seqs * p.hqk) return;  // padding workgroup (whole workgroup, before any barrier)
  const int m = u % p.hqk, h = m * G + w / NB, rank = u / p.hqk;
  int n = rank;
  if (p.num_seqs <= kSortSeqs) {
    // rank -> sequence: sequence t has rank #{s : L_s > L_t or (L_s = L_t and s < t)}. The
    // scratch is the start of the K rows, which nothing else uses yet.
    int* len_s = reinterpret_cast<int*>(smem);
    int* pick = len_s + kSortSeqs;
    for (int t = tid; t < p.num_seqs; t += C::THREADS) len_s[t] = p.cu[t + 1] - p.cu[t];
    lds_barrier();
    for (int t = tid; t < p.num_seqs; t += C::THREADS) {
      const int lt = len_s[t];
      int r = 0;
      for (int s2 = 0; s2 < p.num_seqs; ++s2) {
        const int ls = len_s[s2];
        r += (ls > lt || (ls == lt && s2 < t)) ? 1 : 0;
      }
      if (r == rank) *pick = t;
    }
    lds_barrier();
    n = __builtin_amdgcn_readfirstlane(*pick);
    lds_barrier();  // every wave has read the pick before the first chunk is staged
  }
  const int start = p.cu[n];
  const int L = p.cu[n + 1] - start;
  const int nchunks = (L + kChunk - 1) / kChunk;
  const int slot0 = slot_base(p.cu, n);
  auto ktbuf = [&](int c) -> char* { return smem + C::KTOFF + (c & 1) * C::KTBYTES; };

  // Per chunk c there are three barriers: B(c) (chunk c staged), M(c) (the K, Q and v rows of
  // chunk c are read) and X(c) (V' of chunk c is in LDS). Between them:
  //   chain wave t:  [B] Y = V - diag(gamma) K H            [M] V' = T Y, V' -> LDS
  //                  [X] H <- gamma_C H + K^T diag(delta) V', split state -> LDS
  //   output wave t: [B] Q H^T from the split state in LDS  [M] -  [X] V' P^T, output rows
  //   producers:     [B] P(c)  [M] K, Q, v rows of chunk c + 1
  //                  [X] K^T, T, gamma, delta of chunk c + 1
  // Wave priorities (s_setprio) order the SIMD's instruction arbitration among its waves:
  // producers first (the staging of a window is on every other wave's path), then the chain,
  // then the output waves, whose work has the most slack.
  if (wave >= 2 * NT) {
    // ---------------- producer waves ----------------
    __builtin_amdgcn_s_setprio(3);  // highest: see the schedule above
    // Each producer runs its own copy of this code with its index known at compile time, so the
    // units it moves are fixed in the code: no branch around a load, and the compiler's waits for
    // the loads in flight stay exact.
    if (nchunks == 0) return;
    auto run = [&](auto pw_const) {
      constexpr int PW = decltype(pw_const)::value;
      const int rs = p.hqk * C::ROWB;          // bytes between token rows of q / k
      const int vrs = p.hv * D * 2;            // ... of v
      f32x4 rk[C::KPER], rq[C::KPER], rv[C::VPER], rt_[C::TPER], rp[C::TPER], rg;
      // 1 KiB units of the T (and P) blocks this producer moves, dealt round robin (the index is a
      // compile-time constant in the unrolled loops, so the bound check costs nothing)
      auto tunit = [](int i) { return PW + C::NP * i; };
      auto rec_of = [&](int c) {
        return p.ws + ((size_t)(slot0 + c) * p.hv + h) * kWsRecordBytes;
      };
      auto load_rows = [&](int c) {  // K, Q, v rows of chunk c (rows past the end re-read the last)
        const int t0c = start + kChunk * c, lenc = min(kChunk, L - kChunk * c);
        const char* Kb = reinterpret_cast<const char*>(p.k + ((size_t)t0c * p.hqk + m) * D);
        const char* Qb = reinterpret_cast<const char*>(p.q + ((size_t)t0c * p.hqk + m) * D);
        const char* Vb = reinterpret_cast<const char*>(p.v + ((size_t)t0c * p.hv + h) * D +
                                                       16 * NT * dvb);
#pragma unroll
        for (int i = 0; i < C::KPER; ++i) {
          const int row = (PW * C::KPER + i) * C::RPU + lane / C::NCH;
          const unsigned off = min(row, lenc - 1) * rs + 16 * ((lane % C::NCH) ^ swz<C::ROWB>(row));
          rk[i] = *reinterpret_cast<const f32x4*>(Kb + off);
          rq[i] = *reinterpret_cast<const f32x4*>(Qb + off);
        }
#pragma unroll
        for (int i = 0; i < C::VPER; ++i) {
          const int jj = PW + C::NP * i;
          if (jj < C::VU) {
            const int e = 64 * jj + lane, row = e / C::VPR, cp = e % C::VPR;
            rv[i] = *reinterpret_cast<const f32x4*>(Vb + min(row, lenc - 1) * vrs + 16 * cp);
          }
        }
      };
      auto load_t = [&](int c) {  // T diag(beta) blocks, gamma and delta of chunk c
        const char* rec = rec_of(c);
#pragma unroll
        for (int i = 0; i < C::TPER; ++i)
          if (tunit(i) < C::TU)
            rt_[i] = *reinterpret_cast<const f32x4*>(rec + kWsTOff + 1024 * tunit(i) + 16 * lane);
        if (PW == 0)  // 512 bytes: lanes 32..63 re-read the last 16 bytes
          rg = *reinterpret_cast<const f32x4*>(rec + kWsGOff + 16 * min(lane, 31));
      };
      auto load_p = [&](int c) {  // P blocks of chunk c
        const char* rec = rec_of(c);
#pragma unroll
        for (int i = 0; i < C::TPER; ++i)
          if (tunit(i) < C::TU)
            rp[i] = *reinterpret_cast<const f32x4*>(rec + kWsPOff + 1024 * tunit(i) + 16 * lane);
      };
      auto commit_rows = [&]() {  // K and Q rows staged as fp16 (operands of the state products)
#pragma unroll
        for (int i = 0; i < C::KPER; ++i) {
          *reinterpret_cast<f32x4*>(smem + C::KOFF + 1024 * (PW * C::KPER + i) + 16 * lane) =
              Half::from_bf16(rk[i]);
          *reinterpret_cast<f32x4*>(smem + C::QOFF + 1024 * (PW * C::KPER + i) + 16 * lane) =
              Half::from_bf16(rq[i]);
        }
#pragma unroll
        for (int i = 0; i < C::VPER; ++i) {
          const int jj = PW + C::NP * i;
          if (jj < C::VU) {
            const int e = 64 * jj + lane, row = e / C::VPR, cp = e % C::VPR;
            *reinterpret_cast<f32x4*>(smem + C::VOFF + row * C::VSTR + 16 * cp) = rv[i];
          }
        }
      };
      auto commit_t = [&]() {
#pragma unroll
        for (int i = 0; i < C::TPER; ++i)
          if (tunit(i) < C::TU)
            *reinterpret_cast<f32x4*>(smem + C::TOFF + 1024 * tunit(i) + 16 * lane) = rt_[i];
        if (PW == 0 && lane < 32) *reinterpret_cast<f32x4*>(smem + C::GOFF + 16 * lane) = rg;
      };
      auto commit_p = [&]() {
#pragma unroll
        for (int i = 0; i < C::TPER; ++i)
          if (tunit(i) < C::TU)
            *reinterpret_cast<f32x4*>(smem + C::POFF + 1024 * tunit(i) + 16 * lane) = rp[i];
      };
      // K^T fragments from this producer's own 16 staged K rows (tokens 16 PW .. 16 PW + 15, the
      // half hf = PW & 1 of token block kbp = PW >> 1). ds_read_b64_tr_b16 hands lane (g, 4a + b)
      // element e of the 8 bytes that lane (g, a + 4e) addressed; lane (g, a + 4e) addresses row
      // 16 PW + 4 g + e at the 4 contiguous columns st_row(it, 4a .. 4a + 3), so lane (g, i)
      // receives K[16 PW + 4 g + e][st_row(it, i)] for e = 0..3: slots 4 hf .. 4 hf + 3 of its K^T
      // A fragment.
      auto transpose = [&](char* kt) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's row writes are in LDS
        const int g = lane >> 4, s4 = lane & 15, a = s4 & 3, e = s4 >> 2;
        const int row = 16 * PW + 4 * g + e;
        constexpr int kbp = PW >> 1, hf = PW & 1;
        s16x4 t[NST];
#pragma unroll
        for (int it = 0; it < NST; ++it)
          t[it] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(smem + C::KOFF +
                                                         swz_off<C::ROWB, 2>(row, st_row(it, 4 * a))));
#pragma unroll
        for (int it = 0; it < NST; ++it)  // fp16 back to bf16: exact, the values came from bf16
          *reinterpret_cast<bf16x4*>(kt + ((it * 2 + kbp) * 64 + lane) * 16 + 8 * hf) =
              Half::to_bf16(t[it]);
      };

      // Chunk 0 staged before the first barrier; the next pieces held in registers.
      load_rows(0);
      load_t(0);
      load_p(0);
      commit_rows();
      commit_t();
      commit_p();
      transpose(ktbuf(0));
      if (nchunks > 1) {
        load_rows(1);
        load_t(1);
        load_p(1);
      }
      lds_barrier();  // B(0)
      for (int c = 0; c < nchunks; ++c) {
        if (c > 0) {  // the output waves are done with P of chunk c - 1
          commit_p();
          if (c + 1 < nchunks) load_p(c + 1);
        }
        lds_barrier();  // M(c): the K, Q and v rows of chunk c are read
        if (c + 1 < nchunks) {
          commit_rows();
          if (c + 2 < nchunks) load_rows(c + 2);
        }
        lds_barrier();  // X(c): T, gamma and delta of chunk c are read
        if (c + 1 < nchunks) {
          transpose(ktbuf(c + 1));  // the K^T buffer of chunk c - 1, from this wave's own rows
          commit_t();
          if (c + 2 < nchunks) load_t(c + 2);
          lds_barrier();  // B(c + 1)
        }
      }
    };
    const int pw = wave - 2 * NT;
    if (pw == 0) run(std::integral_constant<int, 0>{});
    if (pw == 1) run(std::integral_constant<int, 1>{});
    if (pw == 2) run(std::integral_constant<int, 2>{});
    if (pw == 3) run(std::integral_constant<int, 3>{});
    return;
  }

  const bool chain = wave < NT;
  const int tile = chain ? wave : wave - NT;
  const int col0 = 16 * (dvb * NT + tile);  // first d_v column of this wave's tile
  const int col = col0 + idx;               // this lane's column in the C fragment layout
  const size_t sbase = (size_t)(n * p.hv + h) * D * D;
  char* const HX = smem + C::XOFF + tile * C::XB;  // this tile's exchanged split state
  char* const VX = HX + C::HXB;                    // ... and V'
  const char* sK = smem + C::KOFF;
  const char* sQ = smem + C::QOFF;
  const char* sV = smem + C::VOFF + tile * C::VROWB;
  const char* sT = smem + C::TOFF;
  const char* sP = smem + C::POFF;
  const float* sgam = reinterpret_cast<const float*>(smem + C::GOFF);
  const float* sdel = sgam + kChunk;
  // A fragment of fp16 K (or Q) rows of the staged chunk
  auto hfrag = [&](const char* rows, int row, int kb) {
    return __builtin_bit_cast(f16x8, afrag<C::ROWB>(rows, row, kb, grp));
  };

  if (chain) {
    // ---------------- chain waves ----------------
    __builtin_amdgcn_s_setprio(2);
    // Hc[it][r] = H[st_row(it, 4 grp + r)][col] (the dtype branch outside the element loops, so
    // that all loads are issued before the first wait)
    f32x4 Hc[NST];
    auto load_state = [&](auto st) {
      using ST = decltype(st);
      const ST* H0 = static_cast<const ST*>(p.h0) + sbase + col;
#pragma unroll
      for (int it = 0; it < NST; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) Hc[it][r] = to_f32(H0[(size_t)st_row(it, 4 * grp + r) * D]);
    };
    if (!p.h0) {
#pragma unroll
      for (int it = 0; it < NST; ++it) Hc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if (p.state_bf16) {
      load_state(bf16{});
    } else {
      load_state(0.f);
    }
    // the state as fp16 B fragments over d_k, kept here and written for the output wave
    f16x8 HB[KB];
    auto split_state = [&]() {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float x[8];
        pack_c_pair(Hc[2 * kb], Hc[2 * kb + 1], x);
        HB[kb] = Half::make(x);
        Half::store_block(HX + kb * 1024, lane, HB[kb]);
      }
    };
    split_state();

    if (nchunks > 0) lds_barrier();  // B(0)
    for (int c = 0; c < nchunks; ++c) {
      const char* sKT = ktbuf(c);
      // Y = V - diag(gamma) K H
      f32x4 Y[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f16x8 kf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kf[kb] = hfrag(sK, 16 * rt + idx, kb);
        f32x4 kh[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kh[kb & 1] = Half::mma(kf[kb], HB[kb], kh[kb & 1]);
        const int vg = lane >> 4, vs = lane & 15, va = vs & 3, ve = vs >> 2;
        const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(sV + (16 * rt + 4 * vg + ve) * C::VSTR + 8 * va));
        const bf16x4 vb = __builtin_bit_cast(bf16x4, vt);
        const f32x4 gam = *reinterpret_cast<const f32x4*>(sgam + 16 * rt + 4 * grp);
        // Rows past the end of the sequence hold the last row again (finite values): the rows
        // and columns of T diag(beta) past the end are zero (identity steps, beta = 0), so these
        // rows add exactly 0 to V' and V' is 0 there.
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[rt][r] = (float)vb[r] - gam[r] * (kh[0][r] + kh[1][r]);
      }
      // Operands of the later phases are read into registers ahead of the barrier that precedes
      // their use, so that their LDS latency overlaps the wait (a read just before its MFMAs
      // would stall every pair of them).
      Op TB[6];
#pragma unroll
      for (int b = 0; b < 6; ++b) TB[b] = ws_load<M>(sT, b, lane);
      lds_barrier();  // M(c)

      Op YB[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8];
        pack_c_pair(Y[2 * kb], Y[2 * kb + 1], x);
        YB[kb] = M::make(x);
      }
      // V' = (T diag(beta)) Y, block lower triangular; V' to the output wave
      f32x4 Vp[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb <= (rt >> 1); ++kb) acc = M::mma_ss(acc, TB[tri_block(rt, kb)], YB[kb]);
        Vp[rt] = acc;
        *reinterpret_cast<f32x4*>(VX + 1024 * rt + 16 * lane) = acc;
      }
      // V'' = diag(delta) V' as split B fragments over tokens; gamma_C (read before X(c), after
      // which the producers restage gamma and delta)
      Op DB[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8], dx[8];
        pack_c_pair(Vp[2 * kb], Vp[2 * kb + 1], x);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(sdel + 32 * kb + 4 * grp);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(sdel + 32 * kb + 16 + 4 * grp);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          dx[s4] = x[s4] * d0[s4];
          dx[4 + s4] = x[4 + s4] * d1[s4];
        }
        DB[kb] = M::make(dx);
      }
      const float gC = sgam[kChunk - 1];
      bf16x8 KT[NST][2];
#pragma unroll
      for (int it = 0; it < NST; ++it)
#pragma unroll
        for (int kbp = 0; kbp < 2; ++kbp)
          KT[it][kbp] = *reinterpret_cast<const bf16x8*>(sKT + ((it * 2 + kbp) * 64 + lane) * 16);
      lds_barrier();  // X(c)

      // H <- gamma_C H + K^T V''
#pragma unroll
      for (int it = 0; it < NST; ++it) {
        f32x4 acc = Hc[it] * gC;
#pragma unroll
        for (int kbp = 0; kbp < 2; ++kbp) acc = M::mma_xs(acc, KT[it][kbp], DB[kbp]);
        Hc[it] = acc;
      }
      split_state();  // the output wave read the previous one before M(c)
      if (c + 1 < nchunks) lds_barrier();  // B(c + 1)
    }

    if (p.ht) {
      auto store_state = [&](auto st) {
        using ST = decltype(st);
        ST* Ht = static_cast<ST*>(p.ht) + sbase + col;
#pragma unroll
        for (int it = 0; it < NST; ++it)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Ht[(size_t)st_row(it, 4 * grp + r) * D] = from_f32<ST>(Hc[it][r]);
      };
      if (p.state_bf16)
        store_state(bf16{});
      else
        store_state(0.f);
    }
    return;
  }

  // ---------------- output waves ----------------
  __builtin_amdgcn_s_setprio(1);
  // O^T = H^T Q^T diag(scale gamma) + V'^T (scale P)^T, computed transposed so that lane
  // (idx = token, grp) holds 4 consecutive columns of its token's output row and stores them
  // directly (the workspace holds P already multiplied by the scale).
  // this lane's output row (token idx of the chunk) advances by whole chunks and row tiles
  const size_t orow = (size_t)p.hv * D;  // elements between token rows
  OutT* Oh = static_cast<OutT*>(p.o) + (size_t)(start + idx) * orow + (size_t)h * D + col0 + 4 * grp;
  if (nchunks > 0) lds_barrier();  // B(0)
  for (int c = 0; c < nchunks; ++c, Oh += kChunk * orow) {
    const int len = min(kChunk, L - kChunk * c);
    f16x8 HB[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) HB[kb] = Half::load_block(HX + kb * 1024, lane);
    f32x4 QH[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f16x8 qf[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) qf[kb] = hfrag(sQ, 16 * rt + idx, kb);
      f32x4 qh[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) qh[kb & 1] = Half::mma(HB[kb], qf[kb], qh[kb & 1]);
      QH[rt] = (qh[0] + qh[1]) * (sgam[16 * rt + idx] * p.scale);
    }
    lds_barrier();  // M(c)
    Op PB[6];  // staged before M(c); read ahead of X(c) so that the wait covers their latency
#pragma unroll
    for (int b = 0; b < 6; ++b) PB[b] = ws_load<M>(sP, b, lane);
    lds_barrier();  // X(c): V' of chunk c from the chain wave
    Op VB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(VX + 1024 * (2 * kb) + 16 * lane);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(VX + 1024 * (2 * kb + 1) + 16 * lane);
      float x[8];
      pack_c_pair(v0, v1, x);
      VB[kb] = M::make(x);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 acc = QH[rt];
#pragma unroll
      for (int kb = 0; kb <= (rt >> 1); ++kb)
        acc = M::mma_ss_t(acc, VB[kb], PB[tri_block(rt, kb)]);
      if (16 * rt + idx < len) store4<OutT>(Oh + 16 * rt * orow, acc);
    }
    if (c + 1 < nchunks) lds_barrier();  // B(c + 1)
  }
}

template <int D, int NT, typename OutT>
hipError_t launch_tiles_cfg(const TilesParams& p, long long heads, int G, hipStream_t stream) {
  static_assert(D / 16 % NT == 0, "d_v tiles per workgroup");
  using C = TilesCfg<D, NT>;
  constexpr int NB = D / 16 / NT;
  const long long units = heads / G;
  const unsigned blocks = (unsigned)(8 * G * NB * ((units + 7) / 8));
  if (heads == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_scan_tiles_kernel<D, NT, OutT>), dim3(blocks), dim3(C::THREADS), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename OutT>
hipError_t launch_tiles_d(const gdn_shape_t& s, const TilesParams& p, hipStream_t stream) {
  const long long heads = (long long)s.num_seqs * s.num_v_heads;
  const int G = s.num_v_heads / s.num_qk_heads;
  switch (s.head_dim_k) {
    case 32: return launch_tiles_cfg<32, 2, OutT>(p, heads, G, stream);
    case 64: return launch_tiles_cfg<64, 4, OutT>(p, heads, G, stream);
    case 128: return launch_tiles_cfg<128, 4, OutT>(p, heads, G, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chunk_scan_tiles(const gdn_shape_t& s, const int32_t* cu, const void* q,
                                   const void* k, const void* v, const void* h0, void* o,
                                   void* ht, const void* ws, hipStream_t stream) {
  TilesParams p{cu, static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                static_cast<const bf16*>(v), h0, o, ht, static_cast<const char*>(ws),
                s.num_seqs, s.num_qk_heads, s.num_v_heads, s.scale,
                s.state_dtype == GDN_DTYPE_BF16 ? 1 : 0};
  if (s.out_dtype == GDN_DTYPE_BF16) return launch_tiles_d<bf16>(s, p, stream);
  return launch_tiles_d<float>(s, p, stream);
}

}  // namespace gdn
