// gdn_scan.hip -- sequential cross-chunk recurrence of the chunked prefill
// ([MoE report] §3.7 Steps 5-7), from the workspace the intra kernel filled.
//
// Per chunk of 64 tokens of one V head, with H the [d_k][d_v] state at the chunk start and
// b the in-chunk cumsum of g (gamma_t = e^{b_t}, b_C = b_63):
//   Y   = V - diag(gamma) K H                  (K H: the state's prediction of v)
//   V'  = (T diag(beta)) Y                     (the delta-rule corrections u_t)
//   O   = scale ( diag(gamma) Q H + P V' )     (P = masked decayed Q K^T)
//   H  <- gamma_C H + K^T diag(e^{b_C - b}) V'
// Columns of H evolve independently, so a workgroup owns NT tiles of 16 d_v columns of one
// (sequence, V head) and walks its chunks in order. Each tile is computed by RW waves:
//   RW = 1: one wave owns all 64 rows of the chunk and its [d_k x 16] fp32 state slice stays
//           in that wave's registers for the whole sequence (fp32 q / k / v with many chains;
//           bf16 q / k / v with many chains run gdn_scan_tiles.hip).
//   RW = 4: wave r owns row tile r (16 tokens) and 32 rows of the state; Y, V' and the new
//           state cross waves through LDS (4x the waves for shapes with few sequences x heads).
// Separate producer waves move the data: while chunk c is computed they write chunk c+1 (held
// in their registers) into the free one of two LDS buffers, load chunk c+2, and store the output
// rows of chunk c-1; the compute waves' only global memory instructions in the chunk loop are
// the row-split layout's loads of their own workspace-record blocks, one chunk ahead. q/k rows
// are staged row-major with a 16-byte XOR swizzle; K^T operand fragments are read from the same
// rows with ds_read_b64_tr_b16. Precision modes: bf16 q / k / v (Bf16Mode, K and Q staged as
// fp16 for the products with the state), fp32 on fp32 MFMA (F32Mode), and fp32 on split-bf16
// MFMA (F32SplitMode: each fp32 K / Q row staged as a hi and a lo bf16 plane, and the record
// blocks split into the bf16 hi / lo layout, by the producers, once per chunk). In the row-split
// layout the waves of a tile exchange Y and V' at two s_barriers per chunk that the producers
// also pass.
// Every product runs on MFMA in the fragment convention of gdn_device.hpp.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.h"

namespace gdn {
namespace {

struct ScanParams {
  const int32_t* cu;
  const void* q;
  const void* k;
  const void* v;
  const void* h0;  // initial states, fp32 or bf16 (state_bf16), or null
  void* o;
  void* ht;  // final states, same dtype, or null
  const char* ws;
  int num_seqs, hqk, hv;
  float scale;
  int state_bf16;
};

// Element i of a stored state (fp32, or bf16 read exactly) and the store of an fp32 value (bf16:
// round to nearest even). The state dtype is uniform over the launch.
__device__ __forceinline__ float state_load(const void* base, size_t i, int bf) {
  return bf ? to_f32(static_cast<const bf16*>(base)[i]) : static_cast<const float*>(base)[i];
}
__device__ __forceinline__ void state_store(void* base, size_t i, float x, int bf) {
  if (bf)
    static_cast<bf16*>(base)[i] = from_f32<bf16>(x);
  else
    static_cast<float*>(base)[i] = x;
}

// d_k index of row m of state tile `it` (16 rows): tiles 2 kb and 2 kb + 1 interleave their
// 4-row groups inside the 32 columns of block kb, so that the C fragments of the two tiles
// stack into a B fragment in the column-contiguous depth order of afrag
// (row 4 g + r of tile 2 kb + hf is column 32 kb + 8 g + 4 hf + r).
__device__ __forceinline__ int state_row(int it, int m) {
  return 32 * (it >> 1) + 8 * (m >> 2) + 4 * (it & 1) + (m & 3);
}

// A fragment of K^T (rows = state tile `it`, depth = tokens of block kbp) from the row-major
// staged K. ds_read_b64_tr_b16 hands lane (g, 4a + b) element e of the 8 bytes that lane
// (g, a + 4e) addressed; lane (g, a + 4e) addresses token row 4g + e at the 4 columns
// state_row(it, 4a .. 4a + 3), so lane (g, i) receives K[tok0 + 4g + e][state_row(it, i)] for
// e = 0..3 (slots 0-3, or 4-7 for the second 16 tokens).
template <int ROWB>
__device__ __forceinline__ bf16x8 ktfrag(const char* sK, int it, int kbp, int lane) {
  const int g = lane >> 4, s = lane & 15, a = s & 3, e = s >> 2;
  bf16x8 f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int row = 32 * kbp + 16 * hf + 4 * g + e;
    const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(sK + swz_off<ROWB, 2>(row, state_row(it, 4 * a))));
    const bf16x4 tb = __builtin_bit_cast(bf16x4, t);
#pragma unroll
    for (int j = 0; j < 4; ++j) f[4 * hf + j] = tb[j];
  }
  return f;
}
template <int ROWB>
__device__ __forceinline__ f32x8 ktfrag_f32(const char* sK, int it, int kbp, int lane) {
  const int idx = lane & 15, g = lane >> 4;
  f32x8 f;
#pragma unroll
  for (int s = 0; s < 8; ++s)
    f[s] = *reinterpret_cast<const float*>(
        sK + swz_off<ROWB, 4>(32 * kbp + kslot(g, s), state_row(it, idx)));
  return f;
}

template <typename Mode, int ROWB>
struct Frags;
template <int ROWB>
struct Frags<Bf16Mode, ROWB> {
  __device__ static bf16x8 a(const char* b, int row, int kb, int grp) {
    return afrag<ROWB>(b, row, kb, grp);
  }
  __device__ static bf16x8 kt(const char* b, int it, int kbp, int lane) {
    return ktfrag<ROWB>(b, it, kbp, lane);
  }
};
template <int ROWB>
struct Frags<F32Mode, ROWB> {
  __device__ static f32x8 a(const char* b, int row, int kb, int grp) {
    return afrag_f32<ROWB>(b, row, kb, grp);
  }
  __device__ static f32x8 kt(const char* b, int it, int kbp, int lane) {
    return ktfrag_f32<ROWB>(b, it, kbp, lane);
  }
};
// F32SplitMode: the fp32 K (or Q) rows of a chunk are staged as two bf16 planes, the hi halves
// of all 64 rows and then the lo halves, each laid out like bf16 rows (ROWB / 2 bytes, the same
// swizzle), so both halves of an operand are read with the bf16 readers.
template <int ROWB>
struct Frags<F32SplitMode, ROWB> {
  static constexpr int HROWB = ROWB / 2, PLANE = 64 * HROWB;
  __device__ static Bf16Mode::Op a(const char* b, int row, int kb, int grp) {
    return {afrag<HROWB>(b, row, kb, grp), afrag<HROWB>(b + PLANE, row, kb, grp)};
  }
  __device__ static Bf16Mode::Op kt(const char* b, int it, int kbp, int lane) {
    return {ktfrag<HROWB>(b, it, kbp, lane), ktfrag<HROWB>(b + PLANE, it, kbp, lane)};
  }
};

// Half of an operand block (slots 4*half .. 4*half+3 of every lane), split like Mode::make.
__device__ __forceinline__ void store_half(Bf16Mode, char* blk, int lane, int half,
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
__device__ __forceinline__ void store_half(F32Mode, char* blk, int lane, int half,
                                           const f32x4& x) {
  *reinterpret_cast<f32x4*>(blk + lane * 32 + half * 16) = x;
}
__device__ __forceinline__ void store_half(F32SplitMode, char* blk, int lane, int half,
                                           const f32x4& x) {
  store_half(F32Mode{}, blk, lane, half, x);  // F32SplitMode::load_block reads this layout
}

// Operand of the two products with the state (K H, Q H): fp16 for bf16 q / k / v (K and Q rows
// then staged as fp16, see Half), the mode's own operand for fp32. kt() turns a K^T fragment read
// from those rows into the operand of the state update (back to bf16 for bf16 q / k / v).
template <typename Mode>
struct StateOp;
template <>
struct StateOp<Bf16Mode> {
  using op = f16x8;
  static constexpr bool kHalfRows = true, kSplitRows = false;
  __device__ static op make(const float (&x)[8]) { return Half::make(x); }
  __device__ static op load(const char* blk, int lane) { return Half::load_block(blk, lane); }
  __device__ static void store(char* blk, int lane, const op& o) { Half::store_block(blk, lane, o); }
  __device__ static f32x4 mma(f32x4 c, const bf16x8& a, const op& b) {
    return Half::mma(__builtin_bit_cast(f16x8, a), b, c);
  }
  __device__ static bf16x8 kt(const bf16x8& raw) {
    return Half::to_bf16(__builtin_bit_cast(f16x8, raw));
  }
};
template <>
struct StateOp<F32Mode> {
  using op = F32Mode::Op;
  static constexpr bool kHalfRows = false, kSplitRows = false;
  __device__ static op make(const float (&x)[8]) { return F32Mode::make(x); }
  __device__ static op load(const char* blk, int lane) { return F32Mode::load_block(blk, lane); }
  __device__ static void store(char* blk, int lane, const op& o) { F32Mode::store_block(blk, lane, o); }
  __device__ static f32x4 mma(f32x4 c, const f32x8& a, const op& b) { return F32Mode::mma_xs(c, a, b); }
  __device__ static f32x8 kt(const f32x8& f) { return f; }
};
template <>
struct StateOp<F32SplitMode> {
  using op = Bf16Mode::Op;
  static constexpr bool kHalfRows = false, kSplitRows = true;
  __device__ static op make(const float (&x)[8]) { return Bf16Mode::make(x); }
  __device__ static op load(const char* blk, int lane) { return Bf16Mode::load_block(blk, lane); }
  __device__ static void store(char* blk, int lane, const op& o) { Bf16Mode::store_block(blk, lane, o); }
  __device__ static f32x4 mma(f32x4 c, const Bf16Mode::Op& a, const op& b) {
    return Bf16Mode::mma_ss(c, a, b);
  }
  __device__ static Bf16Mode::Op kt(const Bf16Mode::Op& f) { return f; }
};

// Layout of the record blocks as staged in LDS: F32SplitMode's producers split the fp32 blocks
// into Bf16Mode's hi / lo layout once per chunk, so the compute waves read them as bf16 pairs.
template <typename Mode>
struct RecLds {
  using type = Mode;
};
template <>
struct RecLds<F32SplitMode> {
  using type = Bf16Mode;
};

// Block of 1 KiB unit um of a record matrix (units 0 .. kWsMatBytes / 1024 - 1; every block
// boundary is a multiple of 1 KiB).
__host__ __device__ constexpr int ws_unit_block(int um) {
  return um == 0 ? 0 : um <= 2 ? 1 : um <= 4 ? 2 : um == 5 ? 3 : um <= 7 ? 4 : 5;
}
static_assert(ws_block_off(ws_unit_block(9)) == 8192 && ws_unit_block(5) == 3 &&
                  ws_block_off(3) == 5120 && kWsMatBytes / 1024 == 10,
              "unit -> block map of the record matrices");

constexpr int kRecUnits = kWsRecordBytes / 16;                   // 16-byte units per record
constexpr int kRecStage = (kWsRecordBytes + 1023) / 1024 * 1024;  // staged record bytes
constexpr int kLdsBytes = 160 * 1024;                             // LDS per workgroup
constexpr int kSortSeqs = 64;  // batches of up to this many sequences run longest first

// C fragment (rows 4 grp + r, column idx) of a 16 x 16 tile stored row-major in LDS with row
// stride `stride` bytes. bf16: one ds_read_b64_tr_b16 (lane (g, a + 4e) addresses row 4g + e,
// columns 4a .. 4a+3; lane (g, 4a + b) receives element b of those, i.e. row 4g + e, column
// 4a + b, for e = 0..3).
template <typename T>
struct VRows;
template <>
struct VRows<bf16> {
  __device__ static f32x4 cfrag(const char* tile, int stride, int lane) {
    const int g = lane >> 4, s = lane & 15, a = s & 3, e = s >> 2;
    const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(tile + (4 * g + e) * stride + 8 * a));
    const bf16x4 tb = __builtin_bit_cast(bf16x4, t);
    f32x4 out;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[r] = (float)tb[r];
    return out;
  }
};
template <>
struct VRows<float> {
  __device__ static f32x4 cfrag(const char* tile, int stride, int lane) {
    const int g = lane >> 4, i = lane & 15;
    f32x4 out;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      out[r] = reinterpret_cast<const float*>(tile + (4 * g + r) * stride)[i];
    return out;
  }
};

// Shapes of one scan workgroup: NT tiles of 16 d_v columns x RW waves per tile compute
// (NC waves), NP producer waves stage the chunks and store the outputs.
//
// A staged chunk (one LDS buffer) holds, in 1 KiB units:
//   [0, KI)              K rows, row-major, 16-byte XOR swizzle (swz)
//   [KI, KQ)             Q rows, same layout
//   [KQ, KQ + RI)        the workspace record of the chunk (T diag(beta), P, gamma, delta)
//   [KQ + RI, TOTAL)     the v rows of the workgroup's NT * 16 columns, row stride VSTR
// RREC (row-split bf16 layout): a compute wave uses only its own row tile's blocks of the
// record, so it loads them from global memory itself, one chunk ahead, into registers, and
// the chunk buffer holds no record (RI = 0). (Loading the wave's own K / Q row fragments the
// same way, instead of staging Q, measured slower.)
// Rows past the end of a sequence re-read its last row (finite values that only ever meet zero
// coefficients); record lanes past its end re-read its last 16 bytes into the padding.
template <typename Mode, int D, int NT, int RW, typename OutT>
struct ScanCfg {
  using in_t = typename Mode::in_t;
  static constexpr bool RREC = RW > 1 && std::is_same<Mode, Bf16Mode>::value;
  static constexpr int ROWB = D * (int)sizeof(in_t), KBYTES = 64 * ROWB;
  static constexpr int NCH = ROWB / 16, RPU = 64 / NCH;  // 16-byte chunks per row, rows per unit
  static constexpr int KI = KBYTES / 1024, RI = RREC ? 0 : kRecStage / 1024;
  static constexpr int KQ = 2 * KI;  // K and Q units
  static constexpr int VROWB = 16 * (int)sizeof(in_t), VPR = VROWB / 16;  // one tile row of v
  static constexpr int VSTR = NT * VROWB + (NT > 1 ? 16 : 0);  // padded: tile reads spread banks
  static constexpr int VI = 64 * NT * VPR / 64;                // v units
  static constexpr int TOTAL = KQ + RI + VI;
  static constexpr int QOFF = KBYTES, ROFF = 1024 * KQ, VOFF = 1024 * (KQ + RI);
  static constexpr int BUFB = VOFF + 64 * VSTR;
  static constexpr int NC = NT * RW;
  // producers hold <= 32 units each in registers; with bf16 q / k / v they also convert the K and
  // Q rows to fp16 on the way (F32SplitMode: split them and the record blocks), and four of
  // them share that work
  static constexpr int NP = std::is_same<Mode, Bf16Mode>::value ? 4 : (TOTAL + 31) / 32;
  static constexpr int PER = (TOTAL + NP - 1) / NP;
  static constexpr int THREADS = 64 * (NC + NP);
  static constexpr int KB = D / 32, R = 4 / RW, OWN = (KB + RW - 1) / RW;
  // Per-tile exchange area (RW > 1): H blocks, then Y, V', V'' (2 blocks each), 2 KiB blocks.
  static constexpr int XH = 0, XY = KB * 2048, XV = XY + 2 * 2048, XD = XV + 2 * 2048;
  static constexpr int XBYTES = RW > 1 ? XD + 2 * 2048 : 0;
  // Output rows of a chunk: 64 rows of NT * 16 columns, row stride OSTR (two buffers).
  static constexpr int OROWB = 16 * (int)sizeof(OutT), OPR = OROWB / 16;
  static constexpr int OSTR = NT * OROWB + (NT > 1 ? 16 : 0);
  static constexpr int OBYTES = 64 * OSTR;
  static constexpr int OPIECES = 64 * NT * OPR, OST = (OPIECES + 64 * NP - 1) / (64 * NP);
  static constexpr int FIXED = NT * XBYTES + 2 * OBYTES;
  static constexpr int NBUF = 2 * BUFB + FIXED <= kLdsBytes ? 2 : 1;
  static constexpr int LDS = NBUF * BUFB + FIXED;
  static_assert(LDS <= kLdsBytes, "LDS budget");
  static_assert(RW == 1 || RW == 4, "row waves");
  static_assert(NC + NP <= 16 && NP <= 4, "waves per workgroup");
};

template <typename Mode, int D, int NT, int RW, typename OutT>
__global__ __launch_bounds__((ScanCfg<Mode, D, NT, RW, OutT>::THREADS)) void chunk_scan_kernel(
    ScanParams p) {
  using C = ScanCfg<Mode, D, NT, RW, OutT>;
  using in_t = typename Mode::in_t;
  using Op = typename Mode::Op;
  using F = Frags<Mode, C::ROWB>;
  using SO = StateOp<Mode>;
  constexpr int KB = C::KB, R = C::R, OWN = C::OWN;

  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  char* const Xbase = smem + C::NBUF * C::BUFB;
  char* const Wo = Xbase + NT * C::XBYTES;  // two output buffers of OBYTES

  const int tid = threadIdx.x, lane = tid & 63, idx = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  constexpr int NB = D / 16 / NT;
  // Work assignment. The hardware deals workgroups round robin over the 8 XCDs (b % 8). A unit
  // (sequence, QK head) has G * NB workgroups (its V heads x column tiles) that read the same
  // q/k rows: they stay on one XCD (one L2) and are dispatched back to back. Units are dealt to
  // the XCDs round robin in order of decreasing sequence length (ties by index), so that every
  // XCD gets an equal share of a packed batch of uneven sequences, longest chains first.
  const int G = p.hv / p.hqk;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int u = 8 * (j / (G * NB)) + xcd, w = j % (G * NB), dvb = w % NB;
  if (u >= p.num_seqs * p.hqk) return;  // padding workgroup (whole workgroup, before any barrier)
  const int m = u % p.hqk, h = m * G + w / NB, rank = u / p.hqk;
  int n = rank;
  if (p.num_seqs <= kSortSeqs) {
    // rank -> sequence: sequence t has rank #{s : L_s > L_t or (L_s = L_t and s < t)}. The
    // scratch is the start of chunk buffer 0, which nothing else uses yet.
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
    lds_barrier();  // every wave has read the pick before buffer 0 is staged
  }
  const int nh = n * p.hv + h;
  const int start = p.cu[n];
  const int L = p.cu[n + 1] - start;
  const int nchunks = (L + kChunk - 1) / kChunk;
  auto chunk_buf = [&](int c) -> char* { return smem + (C::NBUF == 2 ? (c & 1) * C::BUFB : 0); };

  if (wave >= C::NC) {
    // ---------------- producer waves ----------------
    // Each producer runs its own copy of the code with its index known at compile time, so
    // the kind of every staged unit (K, Q, record or v rows) is fixed in the code.
    const in_t* Qg = static_cast<const in_t*>(p.q);
    const in_t* Kg = static_cast<const in_t*>(p.k);
    const in_t* Vg = static_cast<const in_t*>(p.v);
    OutT* Og = static_cast<OutT*>(p.o);
    const int rs = p.hqk * C::ROWB;                    // bytes between token rows of q / k
    const int vrs = p.hv * D * (int)sizeof(in_t);      // ... of v
    const int ors = p.hv * D * (int)sizeof(OutT);      // ... of o
    const int slot0 = slot_base(p.cu, n);
    auto run = [&](auto pw_const) {
      constexpr int PW = decltype(pw_const)::value;
      f32x4 r[C::PER];
      auto load = [&](int c) {
        const int t0c = start + kChunk * c, lenc = min(kChunk, L - kChunk * c);
        const char* Kb = reinterpret_cast<const char*>(Kg + (size_t)t0c * p.hqk * D + (size_t)m * D);
        const char* Qb = reinterpret_cast<const char*>(Qg + (size_t)t0c * p.hqk * D + (size_t)m * D);
        const char* rec = p.ws + ((size_t)(slot0 + c) * p.hv + h) * kWsRecordBytes;
        const char* Vb = reinterpret_cast<const char*>(Vg + (size_t)t0c * p.hv * D + (size_t)h * D +
                                                       16 * dvb * NT);
#pragma unroll
        for (int u = 0; u < C::PER; ++u) {
          const int j = PW + C::NP * u;
          if (j < C::TOTAL) {
            // Uniform base + 32-bit lane offset (one VGPR per address in flight).
            const char* base;
            unsigned off;
            if (j < C::KQ) {
              const int jj = j < C::KI ? j : j - C::KI;
              const int row = jj * C::RPU + lane / C::NCH;
              base = j < C::KI ? Kb : Qb;
              // (split rows take the swizzle of their bf16 planes when they are written)
              off = min(row, lenc - 1) * rs +
                    16 * ((lane % C::NCH) ^ (SO::kSplitRows ? 0 : swz<C::ROWB>(row)));
            } else if (j < C::KQ + C::RI) {
              base = rec;
              off = 16 * min(64 * (j - C::KQ) + lane, kRecUnits - 1);
            } else {
              const int i = 64 * (j - C::KQ - C::RI) + lane;
              const int row = i / (NT * C::VPR), cp = i % (NT * C::VPR);
              base = Vb;
              off = min(row, lenc - 1) * vrs + 16 * cp;
            }
            r[u] = *reinterpret_cast<const f32x4*>(base + off);
          }
        }
      };
      auto commit = [&](char* buf) {
#pragma unroll
        for (int u = 0; u < C::PER; ++u) {
          const int j = PW + C::NP * u;
          if (j < C::TOTAL && SO::kSplitRows && j < C::KQ) {
            // 4 fp32 values of one K (or Q) row -> 8 bytes in the hi plane and 8 in the lo plane
            const int jj = j < C::KI ? j : j - C::KI;
            const int row = jj * C::RPU + lane / C::NCH, cp = lane % C::NCH;
            char* plane = buf + (j < C::KI ? 0 : C::QOFF);
            const int off = swz_off<C::ROWB / 2, 2>(row, 4 * cp);
            bf16x4 hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hi[e] = (bf16)r[u][e];
              lo[e] = (bf16)(r[u][e] - (float)hi[e]);
            }
            *reinterpret_cast<bf16x4*>(plane + off) = hi;
            *reinterpret_cast<bf16x4*>(plane + 64 * (C::ROWB / 2) + off) = lo;
          } else if (j < C::TOTAL && SO::kSplitRows && j >= C::KQ &&
                     j < C::KQ + 2 * (kWsMatBytes / 1024)) {
            // a 1 KiB unit of T diag(beta) or P in F32Mode's layout -> hi / lo halves in
            // Bf16Mode's layout (the same block offsets; within a block, lane l' of the full
            // layout holds 8 floats at 32 l', of the half layout 4 at 16 l')
            constexpr int MU = kWsMatBytes / 1024;
            const int um = (j - C::KQ) % MU;
            const int b = ws_unit_block(um), ob = ws_block_off(b);
            int hoff, lsep;
            if (ws_half_block(b)) {
              hoff = ob + 8 * lane;
              lsep = 512;
            } else {
              hoff = ob + 16 * (32 * (um - ob / 1024) + (lane >> 1)) + 8 * (lane & 1);
              lsep = 1024;
            }
            char* mat = buf + C::ROFF + ((j - C::KQ) / MU) * kWsMatBytes;
            bf16x4 hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hi[e] = (bf16)r[u][e];
              lo[e] = (bf16)(r[u][e] - (float)hi[e]);
            }
            *reinterpret_cast<bf16x4*>(mat + hoff) = hi;
            *reinterpret_cast<bf16x4*>(mat + hoff + lsep) = lo;
          } else if (j < C::TOTAL) {
            int dst;
            if (j < C::KQ + C::RI) {
              dst = 1024 * j + 16 * lane;
            } else {
              const int i = 64 * (j - C::KQ - C::RI) + lane;
              dst = C::VOFF + (i / (NT * C::VPR)) * C::VSTR + 16 * (i % (NT * C::VPR));
            }
            *reinterpret_cast<f32x4*>(buf + dst) =
                (SO::kHalfRows && j < C::KQ) ? Half::from_bf16(r[u]) : r[u];
          }
        }
      };
      auto store_o = [&](int c) {
        const int t0c = start + kChunk * c, lenc = min(kChunk, L - kChunk * c);
        const char* Ws = Wo + (c & 1) * C::OBYTES;
        char* Ob = reinterpret_cast<char*>(Og + (size_t)t0c * p.hv * D + (size_t)h * D + 16 * dvb * NT);
#pragma unroll
        for (int u = 0; u < C::OST; ++u) {
          const int i = 64 * (PW + C::NP * u) + lane;
          const int row = i / (NT * C::OPR), cp = i % (NT * C::OPR);
          if (i < C::OPIECES && row < lenc)
            *reinterpret_cast<f32x4*>(Ob + (unsigned)(row * ors + 16 * cp)) =
                *reinterpret_cast<const f32x4*>(Ws + row * C::OSTR + 16 * cp);
        }
      };

      if (nchunks > 0) load(0);
      if constexpr (C::NBUF == 2) {
        if (nchunks > 0) commit(chunk_buf(0));
        if (nchunks > 1) load(1);
      }
      for (int c = 0; c < nchunks; ++c) {
        lds_barrier();  // chunk c-1 computed: its output rows are in Wo, its buffer is free
        if constexpr (C::NBUF == 2) {
          if (c + 1 < nchunks) commit(chunk_buf(c + 1));
          if (c + 2 < nchunks) load(c + 2);
        } else {
          commit(chunk_buf(c));
          lds_barrier();  // chunk c staged
          if (c + 1 < nchunks) load(c + 1);
        }
        if constexpr (RW > 1) {
          // the compute waves' Y and V' exchanges of chunk c (the producers' LDS writes are
          // waited for at the next chunk's barrier)
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_s_barrier();
        }
        if (c > 0) store_o(c - 1);
      }
      lds_barrier();  // last chunk computed
      if (nchunks > 0) store_o(nchunks - 1);
    };
    const int pw = wave - C::NC;
    if (pw == 0) run(std::integral_constant<int, 0>{});
    if constexpr (C::NP > 1) if (pw == 1) run(std::integral_constant<int, 1>{});
    if constexpr (C::NP > 2) if (pw == 2) run(std::integral_constant<int, 2>{});
    if constexpr (C::NP > 3) if (pw == 3) run(std::integral_constant<int, 3>{});
    return;
  }

  // ---------------- compute waves ----------------
  const int tile = wave / RW, rg = wave % RW;
  const int col = 16 * (dvb * NT + tile) + idx;
  char* const X = Xbase + tile * C::XBYTES;
  // The RW waves of a tile exchange Y and V' twice per chunk, at two s_barriers that the
  // producer waves also pass once their own work of the chunk allows it (an LDS arrival
  // counter among the compute waves alone, with reads issued between arriving and waiting,
  // measured 3% slower).
  auto exchange = [&]() { lds_barrier(); };


  // Owned state blocks: kb = rg + RW * o; Hc[o][hf][r] = H[state_row(2 kb + hf, 4 grp + r)][col].
  f32x4 Hc[OWN][2];
  {
    const size_t h0_base = (size_t)nh * D * D;
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int kb = rg + RW * o;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Hc[o][hf][r] =
              (p.h0 && kb < KB)
                  ? state_load(p.h0, h0_base + (size_t)state_row(2 * kb + hf, 4 * grp + r) * D + col,
                               p.state_bf16)
                  : 0.f;
      if constexpr (RW > 1) {
        if (kb < KB) {
          float x[8];
          pack_c_pair(Hc[o][0], Hc[o][1], x);
          SO::store(X + C::XH + kb * 2048, lane, SO::make(x));
        }
      }
    }
  }

  // RREC: this wave's blocks of the chunk's workspace record (row tile rt = rg): T diag(beta)
  // and P, gamma, delta and gamma_C, loaded one chunk ahead. Every fetch issues the same loads
  // with no branch (row tiles 0 and 1 also load a second, unused block; the last chunk
  // re-loads itself), so that the compiler's wait counts stay exact: after a path with fewer
  // loads in flight it would wait for all of them, the next chunk's included.
  struct Rec {
    Op TB[2], PB[2];
    f32x4 gam, del;
    float gC;
  };
  const int slot0 = slot_base(p.cu, n);
  auto fetch = [&](int c, Rec& f) __attribute__((always_inline)) {
    if constexpr (C::RREC) {
      const int rt = rg;
      const char* rec = p.ws + ((size_t)(slot0 + c) * p.hv + h) * kWsRecordBytes;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f.TB[kb] = ws_load_nb<Mode>(rec + kWsTOff, tri_block(rt, kb), lane);
        f.PB[kb] = ws_load_nb<Mode>(rec + kWsPOff, tri_block(rt, kb), lane);
      }
      f.gam = *reinterpret_cast<const f32x4*>(rec + kWsGOff + 4 * (16 * rt + 4 * grp));
      f.del = *reinterpret_cast<const f32x4*>(rec + kWsDOff + 4 * (16 * rt + 4 * grp));
      f.gC = reinterpret_cast<const float*>(rec + kWsGOff)[kChunk - 1];
    }
  };

  auto body = [&](int c, const Rec& cur, Rec& nxt) __attribute__((always_inline)) {
    const int len = min(kChunk, L - kChunk * c);
    lds_barrier();  // chunk c staged (double buffer); state blocks of chunk c-1 exchanged
    if constexpr (C::NBUF == 1) lds_barrier();  // chunk c staged
    if constexpr (C::RREC) fetch(min(c + 1, nchunks - 1), nxt);
    const char* const S = chunk_buf(c);
    const char* sK = S;
    const char* sQ = S + C::QOFF;
    const char* sR = S + C::ROFF;
    const char* sV = S + C::VOFF + tile * C::VROWB;
    const float* sgam = reinterpret_cast<const float*>(sR + kWsGOff);
    const float* sdel = reinterpret_cast<const float*>(sR + kWsDOff);
    char* const Wc = Wo + (c & 1) * C::OBYTES + tile * C::OROWB;
    // Operand accessors: RREC waves use the fetched registers (rt is always their own).
    using RM = typename RecLds<Mode>::type;  // layout of the staged record blocks
    auto tblock = [&](int rt, int kb) -> Op {
      if constexpr (C::RREC) return cur.TB[kb];
      return ws_load<RM>(sR + kWsTOff, tri_block(rt, kb), lane);
    };
    auto pblock = [&](int rt, int kb) -> Op {
      if constexpr (C::RREC) return cur.PB[kb];
      return ws_load<RM>(sR + kWsPOff, tri_block(rt, kb), lane);
    };
    auto gamma4 = [&](int rt) -> f32x4 {
      if constexpr (C::RREC) return cur.gam;
      return *reinterpret_cast<const f32x4*>(sgam + 16 * rt + 4 * grp);
    };
    auto delta4 = [&](int rt) -> f32x4 {
      if constexpr (C::RREC) return cur.del;
      return *reinterpret_cast<const f32x4*>(sdel + 16 * rt + 4 * grp);
    };

    // (a) state as B fragments over d_k (the operand of the state products)
    typename SO::op HB[KB];
    if constexpr (RW == 1) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float x[8];
        pack_c_pair(Hc[kb][0], Hc[kb][1], x);
        HB[kb] = SO::make(x);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) HB[kb] = SO::load(X + C::XH + kb * 2048, lane);
    }

    // (b) K H, Q H on this wave's row tiles; Y = V - gamma K H, scale gamma Q H.
    // The K / Q fragments of a row tile are read before its products (and, for bf16, those
    // of the next row tile while these run), so LDS latency overlaps the MFMA chains. Two
    // accumulators per product (even / odd depth blocks) halve the dependent chains; the
    // many-chain kernel accumulates in the same order, so the two layouts give the same bits.
    using frag_t = typename Mode::frag_t;
    // fp32 operands over four row tiles leave no registers for reading ahead.
    constexpr bool EARLY = !(std::is_same<Mode, F32Mode>::value && R > 1);
    constexpr int KQB = std::is_same<Mode, Bf16Mode>::value && R > 1 ? 2 : 1;
    frag_t ka[KQB][KB], qa[KQB][KB];
    auto load_kq = [&](int b, int rt) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        ka[b][kb] = F::a(sK, 16 * rt + idx, kb, grp);
        qa[b][kb] = F::a(sQ, 16 * rt + idx, kb, grp);
      }
    };
    f32x4 QH[R], Y[R];
    if constexpr (EARLY) load_kq(0, rg * R);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int rt = rg * R + i, b = KQB > 1 ? (i & 1) : 0;
      if (EARLY && KQB == 1 && i > 0) load_kq(0, rt);
      const f32x4 v4 = VRows<in_t>::cfrag(sV + 16 * rt * C::VSTR, C::VSTR, lane);
      const f32x4 gam = gamma4(rt);
      f32x4 kh[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      f32x4 qh[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const frag_t kf = EARLY ? ka[b][kb] : F::a(sK, 16 * rt + idx, kb, grp);
        const frag_t qf = EARLY ? qa[b][kb] : F::a(sQ, 16 * rt + idx, kb, grp);
        kh[kb & 1] = SO::mma(kh[kb & 1], kf, HB[kb]);
        qh[kb & 1] = SO::mma(qh[kb & 1], qf, HB[kb]);
      }
      if (KQB > 1 && i + 1 < R) load_kq(b ^ 1, rt + 1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float vr = 16 * rt + 4 * grp + r < len ? v4[r] : 0.f;
        Y[i][r] = vr - gam[r] * (kh[0][r] + kh[1][r]);
        QH[i][r] = (qh[0][r] + qh[1][r]) * (gam[r] * p.scale);
      }
    }

    // K^T fragments of the state update (g) for this wave's state rows, over all 64 tokens.
    constexpr bool KT_EARLY = EARLY && RW > 1;
    frag_t kt[OWN][2][2];
    auto load_kt = [&]() {
#pragma unroll
      for (int o = 0; o < OWN; ++o) {
        const int kb = rg + RW * o;
        if (kb < KB)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int kbp = 0; kbp < 2; ++kbp) kt[o][hf][kbp] = F::kt(sK, 2 * kb + hf, kbp, lane);
      }
    };
    // (c) Y as split B fragments over tokens (blocks of 32). Row-split layout: the waves
    // exchange their Y rows; the T diag(beta) blocks of (d) are then in registers (bf16) or
    // read from the staged record, and the K^T fragments of (g) are read while (d) runs.
    Op TB[R][2];
    auto load_t = [&]() {
#pragma unroll
      for (int i = 0; i < (EARLY ? R : 0); ++i) {
        const int rt = rg * R + i;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (kb <= (rt >> 1)) TB[i][kb] = tblock(rt, kb);
      }
    };
    Op YB[2];
    if constexpr (RW == 1) {
      load_t();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8];
        pack_c_pair(Y[2 * kb], Y[2 * kb + 1], x);
        YB[kb] = Mode::make(x);
      }
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int rt = rg * R + i;
        store_half(Mode{}, X + C::XY + (rt >> 1) * 2048, lane, rt & 1, Y[i]);
      }
      exchange();
      load_t();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (2 * kb <= rg * R + R - 1) YB[kb] = Mode::load_block(X + C::XY + kb * 2048, lane);
      load_kt();
    }

    // (d) V' = (T diag(beta)) Y on this wave's row tiles (block lower triangular)
    f32x4 Vp[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int rt = rg * R + i;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb <= (rt >> 1)) acc = Mode::mma_ss(acc, EARLY ? TB[i][kb] : tblock(rt, kb), YB[kb]);
      Vp[i] = acc;
    }

    // (e) V' and V'' = diag(e^{b_C - b}) V' as split B fragments over tokens (row-split
    // layout: exchanged). The P blocks of (f) are taken like the T blocks.
    Op PB[R][2];
    auto load_p = [&]() {
#pragma unroll
      for (int i = 0; i < (EARLY ? R : 0); ++i) {
        const int rt = rg * R + i;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (kb <= (rt >> 1)) PB[i][kb] = pblock(rt, kb);
      }
    };
    Op VB[2], DB[2];
    if constexpr (RW == 1) {
      load_p();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8], d[8];
        pack_c_pair(Vp[2 * kb], Vp[2 * kb + 1], x);
        const f32x4 d0 = delta4(2 * kb), d1 = delta4(2 * kb + 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          d[s] = x[s] * d0[s];
          d[4 + s] = x[4 + s] * d1[s];
        }
        VB[kb] = Mode::make(x);
        DB[kb] = Mode::make(d);
      }
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int rt = rg * R + i;
        store_half(Mode{}, X + C::XV + (rt >> 1) * 2048, lane, rt & 1, Vp[i]);
        store_half(Mode{}, X + C::XD + (rt >> 1) * 2048, lane, rt & 1, Vp[i] * delta4(rt));
      }
      exchange();
      load_p();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (2 * kb <= rg * R + R - 1) VB[kb] = Mode::load_block(X + C::XV + kb * 2048, lane);
        DB[kb] = Mode::load_block(X + C::XD + kb * 2048, lane);
      }
    }

    // (g) owned state blocks first (the next chunk waits on them): H <- gamma_C H + K^T V''
    const float gC = C::RREC ? cur.gC : sgam[kChunk - 1];
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int kb = rg + RW * o;
      if (kb < KB) {
        if constexpr (EARLY && !KT_EARLY) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int kbp = 0; kbp < 2; ++kbp) kt[o][hf][kbp] = F::kt(sK, 2 * kb + hf, kbp, lane);
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          f32x4 acc = Hc[o][hf] * gC;
#pragma unroll
          for (int kbp = 0; kbp < 2; ++kbp)
            acc = Mode::mma_xs(
                acc, SO::kt(EARLY ? kt[o][hf][kbp] : F::kt(sK, 2 * kb + hf, kbp, lane)), DB[kbp]);
          Hc[o][hf] = acc;
        }
        if constexpr (RW > 1) {
          float x[8];
          pack_c_pair(Hc[o][0], Hc[o][1], x);
          SO::store(X + C::XH + kb * 2048, lane, SO::make(x));
        }
      }
    }

    // (f) O = diag(scale gamma) Q H + (scale P) V' on this wave's row tiles, into the output rows
    // (the workspace holds P already multiplied by the scale)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int rt = rg * R + i;
      f32x4 acc = QH[i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb <= (rt >> 1)) acc = Mode::mma_ss(acc, EARLY ? PB[i][kb] : pblock(rt, kb), VB[kb]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        reinterpret_cast<OutT*>(Wc + (16 * rt + 4 * grp + r) * C::OSTR)[idx] = from_f32<OutT>(acc[r]);
    }
  };

  Rec pa, pb;
  if constexpr (C::RREC) {
    // Two register sets, alternating by chunk: the loop is unrolled by two so that no copy
    // of the fetched operands is needed.
    if (nchunks > 0) fetch(0, pa);
    for (int c = 0; c < nchunks; c += 2) {
      body(c, pa, pb);
      if (c + 1 < nchunks) body(c + 1, pb, pa);
    }
  } else {
    for (int c = 0; c < nchunks; ++c) body(c, pa, pb);
  }
  lds_barrier();  // last chunk computed (the producers store its output rows)

  if (p.ht) {
    const size_t ht_base = (size_t)nh * D * D;
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int kb = rg + RW * o;
      if (kb < KB)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            state_store(p.ht, ht_base + (size_t)state_row(2 * kb + hf, 4 * grp + r) * D + col,
                        Hc[o][hf][r], p.state_bf16);
    }
  }
}

template <typename Mode, int D, int NT, int RW, typename OutT>
hipError_t launch_scan_cfg(const ScanParams& p, long long heads, int G, hipStream_t stream) {
  static_assert(D / 16 % NT == 0, "d_v tiles per workgroup");
  using C = ScanCfg<Mode, D, NT, RW, OutT>;
  // Units (sequence, QK head) of G * NB workgroups are dealt to the 8 XCDs round robin;
  // padding workgroups exit.
  constexpr int NB = D / 16 / NT;
  const long long units = heads / G;
  const unsigned blocks = (unsigned)(8 * G * NB * ((units + 7) / 8));
  if (heads == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_scan_kernel<Mode, D, NT, RW, OutT>), dim3(blocks), dim3(C::THREADS), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename Mode, int D, typename OutT>
hipError_t launch_scan_t(const gdn_shape_t& s, const ScanParams& p, hipStream_t stream) {
  const long long heads = (long long)s.num_seqs * s.num_v_heads;
  const int G = s.num_v_heads / s.num_qk_heads;
  constexpr int tiles = D / 16;
  // Few (sequence, head) chains: 4 waves per 16-column tile so that every SIMD gets work.
  // Many chains, fp32 q / k / v (F32Mode or F32SplitMode): 1 wave per tile, 4 (or 2) tiles per
  // workgroup sharing the staged chunk. (Many chains with bf16 operands run
  // chunk_scan_tiles_kernel, gdn_scan_tiles.hip.)
  if (heads * tiles <= 512) return launch_scan_cfg<Mode, D, 1, 4, OutT>(p, heads, G, stream);
  if constexpr (!std::is_same<Mode, Bf16Mode>::value) {
    if constexpr (tiles % 4 == 0) return launch_scan_cfg<Mode, D, 4, 1, OutT>(p, heads, G, stream);
    else return launch_scan_cfg<Mode, D, 2, 1, OutT>(p, heads, G, stream);
  }
  return hipErrorInvalidValue;  // not reached: the caller dispatches bf16 many-chain shapes
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

hipError_t launch_chunk_scan(const gdn_shape_t& s, const int32_t* cu, const void* q,
                             const void* k, const void* v, const void* h0, void* o, void* ht,
                             const void* ws, hipStream_t stream) {
  ScanParams p{cu, q, k, v, h0, o, ht, static_cast<const char*>(ws), s.num_seqs, s.num_qk_heads,
               s.num_v_heads, s.scale, s.state_dtype == GDN_DTYPE_BF16 ? 1 : 0};
  const bool out_bf = s.out_dtype == GDN_DTYPE_BF16;
  if (s.qkv_dtype == GDN_DTYPE_BF16 &&
      (long long)s.num_seqs * s.num_v_heads * (s.head_dim_v / 16) > 512)
    return launch_chunk_scan_tiles(s, cu, q, k, v, h0, o, ht, ws, stream);
  if (s.qkv_dtype == GDN_DTYPE_BF16)
    return out_bf ? launch_scan_d<Bf16Mode, bf16>(s, p, stream)
                  : launch_scan_d<Bf16Mode, float>(s, p, stream);
  if (s.qkv_dtype == GDN_DTYPE_F32_SPLIT)
    return out_bf ? launch_scan_d<F32SplitMode, bf16>(s, p, stream)
                  : launch_scan_d<F32SplitMode, float>(s, p, stream);
  return out_bf ? launch_scan_d<F32Mode, bf16>(s, p, stream)
                : launch_scan_d<F32Mode, float>(s, p, stream);
}

}  // namespace gdn
