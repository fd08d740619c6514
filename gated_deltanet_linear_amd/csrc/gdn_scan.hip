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
// (sequence, V head) and walks its chunks in order. Each tile is handled by RW waves:
//   RW = 1: one wave owns all 64 rows of the chunk and its [d_k x 16] fp32 state slice stays
//           in that wave's registers for the whole sequence (most work per wave, least LDS).
//   RW = 4: wave r owns row tile r (16 tokens) and 32 rows of the state; Y, V' and the new
//           state cross waves through LDS (4x the waves for shapes with few sequences x heads).
// q/k rows and the workspace record of chunk c+1 are loaded into registers while chunk c
// computes and written to LDS when chunk c+1 starts. q/k rows are stored row-major with a
// 16-byte XOR swizzle; K^T operand fragments are read from the same rows with
// ds_read_b64_tr_b16.
// Every product runs on MFMA in the fragment convention of gdn_device.hpp.
#include <cstdlib>
#include <cstring>
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
  const float* h0;
  void* o;
  float* ht;
  const char* ws;
  int num_seqs, hqk, hv;
  float scale;
};

// A fragment of K^T (rows = d_k tile `it`, depth = tokens of block kbp) from the row-major
// staged K. ds_read_b64_tr_b16 hands lane (g, 4a + b) element e of the 8 bytes that lane
// (g, a + 4e) addressed; lane (g, a + 4e) addresses row 4g + e, columns 16 it + 4a .. +3, so
// lane (g, i) receives K[tok0 + 4g + e][16 it + i] for e = 0..3 (slots 0-3, or 4-7 for the
// second 16 tokens).
template <int ROWB>
__device__ __forceinline__ bf16x8 ktfrag(const char* sK, int it, int kbp, int lane) {
  const int g = lane >> 4, s = lane & 15, a = s & 3, e = s >> 2;
  bf16x8 f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int row = 32 * kbp + 16 * hf + 4 * g + e;
    const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(sK + swz_off<ROWB, 2>(row, 16 * it + 4 * a)));
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
        sK + swz_off<ROWB, 4>(32 * kbp + kslot(g, s), 16 * it + idx));
  return f;
}

// Raw element loads for register prefetch. A bf16 element is fetched as the aligned 32-bit
// word that holds it (no narrowing or masking right after the load, which would make the
// compiler wait for it there) and its half is selected where it is used.
__device__ __forceinline__ uint32_t load_raw(const bf16* p, int col) {
  return *reinterpret_cast<const uint32_t*>(p + (col & ~1));
}
__device__ __forceinline__ float load_raw(const float* p, int col) { return p[col]; }
__device__ __forceinline__ float raw_to_f32(uint32_t x, int col) {
  return __uint_as_float((col & 1) ? (x & 0xffff0000u) : (x << 16));
}
__device__ __forceinline__ float raw_to_f32(float x, int) { return x; }

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

constexpr int kRecUnits = kWsRecordBytes / 16;               // 16-byte units per record
constexpr int kRecStage = (kWsRecordBytes + 1023) / 1024 * 1024;  // staged record bytes

// One chunk's staged data (K rows, Q rows, workspace record), prefetched into registers with
// ordinary 16-byte global loads one chunk ahead and written to LDS at the start of the chunk
// that uses it. (global_load_lds reaches only ~38 B/clk per CU on this part; plain loads into
// registers several times that.) Unit j of 1 KiB goes to LDS bytes [1024 j, 1024 j + 1024):
// units [0, KI) are K rows, [KI, 2 KI) Q rows (row-major, 16-byte XOR swizzle), then the
// record. Rows past len re-read row len - 1 (finite values that only meet zero
// coefficients); record lanes past its end re-read its last 16 bytes into the padding.
template <typename Mode, int D, int NWAVES>
struct Stager {
  using in_t = typename Mode::in_t;
  static constexpr int ROWB = D * (int)sizeof(in_t), NCH = ROWB / 16, KBYTES = 64 * ROWB;
  static constexpr int KI = KBYTES / 1024, RI = kRecStage / 1024, TOTAL = 2 * KI + RI;
  static constexpr int PER = (TOTAL + NWAVES - 1) / NWAVES;
  f32x4 r[PER];

  __device__ __forceinline__ void load(const in_t* Kg, const in_t* Qg, const char* rec, int t0,
                                       int len, size_t rstride, int m, int wave, int lane) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = wave + NWAVES * u;
      if (j < TOTAL) {
        const char* src;
        if (j < 2 * KI) {
          const bool isq = j >= KI;
          const int P = 64 * (isq ? j - KI : j) + lane;
          const int row = P / NCH, ch = (P % NCH) ^ swz<ROWB>(P / NCH);
          const int rr = row < len ? row : len - 1;
          src = reinterpret_cast<const char*>((isq ? Qg : Kg) + (size_t)(t0 + rr) * rstride +
                                              (size_t)m * D) + 16 * ch;
        } else {
          const int P = min(64 * (j - 2 * KI) + lane, kRecUnits - 1);
          src = rec + 16 * P;
        }
        r[u] = *reinterpret_cast<const f32x4*>(src);
      }
    }
  }
  __device__ __forceinline__ void commit(char* S, int wave, int lane) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int j = wave + NWAVES * u;
      if (j < TOTAL) *reinterpret_cast<f32x4*>(S + 1024 * j + 16 * lane) = r[u];
    }
  }
};

template <typename Mode, int D, int NT, int RW, typename OutT>
__global__ __launch_bounds__(NT * RW * 64) void chunk_scan_kernel(ScanParams p) {
  using in_t = typename Mode::in_t;
  using Op = typename Mode::Op;
  using F = Frags<Mode, D * (int)sizeof(in_t)>;
  constexpr int ROWB = D * (int)sizeof(in_t);
  constexpr int KBYTES = 64 * ROWB;
  constexpr int KB = D / 32;        // 32-deep blocks over d_k
  constexpr int R = 4 / RW;         // row tiles per wave
  constexpr int NWAVES = NT * RW;
  constexpr int STAGE_BYTES = 2 * KBYTES + kRecStage;
  constexpr int OWN = (KB + RW - 1) / RW;  // state blocks owned by one wave
  // Per-tile exchange area (RW > 1): H blocks, then Y, V', V'' (2 blocks each), 2 KiB blocks.
  constexpr int XH = 0, XY = KB * 2048, XV = XY + 2 * 2048, XD = XV + 2 * 2048;
  constexpr int XBYTES = RW > 1 ? XD + 2 * 2048 : 0;
  static_assert(RW == 1 || RW == 2 || RW == 4, "row waves");
  static_assert(STAGE_BYTES + NT * XBYTES <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) char smem[STAGE_BYTES + NT * XBYTES + 16];

  const int tid = threadIdx.x, lane = tid & 63, idx = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int tile = wave / RW, rg = wave % RW;
  constexpr int NB = D / 16 / NT;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int dvb = lid % NB, nh = lid / NB;
  const int h = nh % p.hv, n = nh / p.hv;
  const int G = p.hv / p.hqk, m = h / G;
  const int col = 16 * (dvb * NT + tile) + idx;
  char* X = smem + STAGE_BYTES + tile * XBYTES;

  const in_t* Qg = static_cast<const in_t*>(p.q);
  const in_t* Kg = static_cast<const in_t*>(p.k);
  const in_t* Vg = static_cast<const in_t*>(p.v);
  OutT* Og = static_cast<OutT*>(p.o);
  const size_t rstride = (size_t)p.hqk * D;

  // Owned state blocks: kb = rg + RW * o; Hc[o][hf][r] = H[16 (2 kb + hf) + 4 grp + r][col].
  f32x4 Hc[OWN][2];
  {
    const float* H0 = p.h0 ? p.h0 + (size_t)nh * D * D : nullptr;
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int kb = rg + RW * o;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Hc[o][hf][r] = (H0 && kb < KB) ? H0[(size_t)(16 * (2 * kb + hf) + 4 * grp + r) * D + col]
                                         : 0.f;
      if constexpr (RW > 1) {
        if (kb < KB) {
          float x[8];
          pack_c_pair(Hc[o][0], Hc[o][1], x);
          Mode::store_block(X + XH + kb * 2048, lane, Mode::make(x));
        }
      }
    }
  }

  const int start = p.cu[n];
  const int L = p.cu[n + 1] - start;
  const int nchunks = (L + kChunk - 1) / kChunk;
  const int slot0 = slot_base(p.cu, n);
  auto rec_of = [&](int c) {
    return p.ws + ((size_t)(slot0 + c) * p.hv + h) * kWsRecordBytes;
  };
  // v rows of this wave (row tiles rg*R .. rg*R+R-1) in C-fragment order, one chunk ahead.
  // Rows past the chunk end read the last valid row and are zeroed where used. The values
  // stay raw (one element per 32-bit register) until used, so that nothing waits on the
  // loads before the next chunk.
  using reg_t = typename std::conditional<std::is_same<in_t, bf16>::value, uint32_t, float>::type;
  auto load_v = [&](int c, reg_t (&dst)[R][4]) {
    const int t0c = start + kChunk * c, lenc = min(kChunk, L - kChunk * c);
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = min(16 * (rg * R + i) + 4 * grp + r, lenc - 1);
        dst[i][r] = load_raw(Vg + ((size_t)(t0c + t) * p.hv + h) * D, col);
      }
  };
  reg_t vnext[R][4];
  Stager<Mode, D, NWAVES> st;
  if (nchunks > 0) {
    load_v(0, vnext);
    st.load(Kg, Qg, rec_of(0), start, min(kChunk, L), rstride, m, wave, lane);
  }
  // Output rows of the previous chunk, stored after the next chunk's barrier so that the
  // wait for the prefetch never waits for fresh stores.
  f32x4 Oprev[R];
  int t0prev = 0, lenprev = 0;
  auto store_prev = [&]() {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * (rg * R + i) + 4 * grp + r;
        if (t < lenprev) Og[((size_t)(t0prev + t) * p.hv + h) * D + col] = from_f32<OutT>(Oprev[i][r]);
      }
  };

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = start + kChunk * c;
    const int len = min(kChunk, L - kChunk * c);
    char* S = smem;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk c (and its v rows) landed
    lds_barrier();                  // every wave is done with chunk c-1's LDS
    st.commit(S, wave, lane);
    lds_barrier();                  // chunk c staged
    float vv[R][4];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vv[i][r] = (16 * (rg * R + i) + 4 * grp + r < len) ? raw_to_f32(vnext[i][r], col) : 0.f;
    if (c + 1 < nchunks) {
      load_v(c + 1, vnext);
      st.load(Kg, Qg, rec_of(c + 1), t0 + kChunk, min(kChunk, L - kChunk * (c + 1)), rstride, m,
              wave, lane);
    }
    if (c > 0) store_prev();
    const char* sK = S;
    const char* sQ = S + KBYTES;
    const char* sTP = S + 2 * KBYTES;
    const float* sgam = reinterpret_cast<const float*>(sTP + kWsGOff);
    const float* sdel = reinterpret_cast<const float*>(sTP + kWsDOff);

    // (a) state as split B fragments over d_k
    Op HB[KB];
    if constexpr (RW == 1) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float x[8];
        pack_c_pair(Hc[kb][0], Hc[kb][1], x);
        HB[kb] = Mode::make(x);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) HB[kb] = Mode::load_block(X + XH + kb * 2048, lane);
    }

    // (b) K H, Q H on this wave's row tiles; Y = V - gamma K H, gamma Q H
    f32x4 QH[R], Y[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int rt = rg * R + i;
      f32x4 kh = {0.f, 0.f, 0.f, 0.f}, qh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        kh = Mode::mma_xs(kh, F::a(sK, 16 * rt + idx, kb, grp), HB[kb]);
        qh = Mode::mma_xs(qh, F::a(sQ, 16 * rt + idx, kb, grp), HB[kb]);
      }
      const f32x4 gam = *reinterpret_cast<const f32x4*>(sgam + 16 * rt + 4 * grp);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Y[i][r] = vv[i][r] - gam[r] * kh[r];
        QH[i][r] = gam[r] * qh[r];
      }
    }

    // (c) Y as split B fragments over tokens (blocks of 32)
    Op YB[2];
    if constexpr (RW == 1) {
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
        store_half(Mode{}, X + XY + (rt >> 1) * 2048, lane, rt & 1, Y[i]);
      }
      lds_barrier();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (2 * kb <= rg * R + R - 1) YB[kb] = Mode::load_block(X + XY + kb * 2048, lane);
    }

    // (d) V' = (T diag(beta)) Y on this wave's row tiles (block lower triangular)
    f32x4 Vp[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int rt = rg * R + i;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb <= (rt >> 1))
          acc = Mode::mma_ss(acc, Mode::load_block(sTP + kWsTOff + tri_block(rt, kb) * 2048, lane),
                             YB[kb]);
      Vp[i] = acc;
    }

    // (e) V' and V'' = diag(e^{b_C - b}) V' as split B fragments over tokens
    Op VB[2], DB[2];
    if constexpr (RW == 1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8], d[8];
        pack_c_pair(Vp[2 * kb], Vp[2 * kb + 1], x);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(sdel + 32 * kb + 4 * grp);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(sdel + 32 * kb + 16 + 4 * grp);
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
        const f32x4 dl = *reinterpret_cast<const f32x4*>(sdel + 16 * rt + 4 * grp);
        store_half(Mode{}, X + XV + (rt >> 1) * 2048, lane, rt & 1, Vp[i]);
        store_half(Mode{}, X + XD + (rt >> 1) * 2048, lane, rt & 1, Vp[i] * dl);
      }
      lds_barrier();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        VB[kb] = Mode::load_block(X + XV + kb * 2048, lane);
        DB[kb] = Mode::load_block(X + XD + kb * 2048, lane);
      }
    }

    // (g) owned state blocks first (the next chunk waits on them): H <- gamma_C H + K^T V''
    const float gC = sgam[kChunk - 1];
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int kb = rg + RW * o;
      if (kb < KB) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          f32x4 acc = Hc[o][hf] * gC;
#pragma unroll
          for (int kbp = 0; kbp < 2; ++kbp)
            acc = Mode::mma_xs(acc, F::kt(sK, 2 * kb + hf, kbp, lane), DB[kbp]);
          Hc[o][hf] = acc;
        }
        if constexpr (RW > 1) {
          float x[8];
          pack_c_pair(Hc[o][0], Hc[o][1], x);
          Mode::store_block(X + XH + kb * 2048, lane, Mode::make(x));
        }
      }
    }

    // (f) O = scale (gamma Q H + P V') on this wave's row tiles (stored next iteration)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int rt = rg * R + i;
      f32x4 acc = QH[i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb <= (rt >> 1))
          acc = Mode::mma_ss(acc, Mode::load_block(sTP + kWsPOff + tri_block(rt, kb) * 2048, lane),
                             VB[kb]);
      Oprev[i] = acc * p.scale;
    }
    t0prev = t0;
    lenprev = len;
  }
  if (nchunks > 0) store_prev();

  if (p.ht) {
    float* HT = p.ht + (size_t)nh * D * D;
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int kb = rg + RW * o;
      if (kb < KB)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            HT[(size_t)(16 * (2 * kb + hf) + 4 * grp + r) * D + col] = Hc[o][hf][r];
    }
  }
}

template <typename Mode, int D, int NT, int RW, typename OutT>
hipError_t launch_scan_cfg(const ScanParams& p, long long heads, hipStream_t stream) {
  static_assert(D / 16 % NT == 0, "d_v tiles per workgroup");
  const unsigned blocks = (unsigned)(heads * (D / 16 / NT));
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((chunk_scan_kernel<Mode, D, NT, RW, OutT>), dim3(blocks), dim3(NT * RW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

// GDN_SCAN_LAYOUT=rows|tiles overrides the choice below (both layouts compute bit-identical
// results; the tests use it to check that).
int forced_layout() {
  static const int v = [] {
    const char* e = getenv("GDN_SCAN_LAYOUT");
    if (!e) return 0;
    if (!strcmp(e, "rows")) return 1;
    if (!strcmp(e, "tiles")) return 2;
    return 0;
  }();
  return v;
}

template <typename Mode, int D, typename OutT>
hipError_t launch_scan_t(const gdn_shape_t& s, const ScanParams& p, hipStream_t stream) {
  const long long heads = (long long)s.num_seqs * s.num_v_heads;
  constexpr int tiles = D / 16;
  // Few (sequence, head) chains: 4 waves per 16-column tile so that every SIMD gets work.
  // Many chains: 1 wave per tile, 4 tiles per workgroup sharing the staged chunk.
  const int forced = forced_layout();
  if (forced == 1 || (forced == 0 && heads * tiles <= 512))
    return launch_scan_cfg<Mode, D, 1, 4, OutT>(p, heads, stream);
  if constexpr (tiles % 4 == 0) return launch_scan_cfg<Mode, D, 4, 1, OutT>(p, heads, stream);
  else return launch_scan_cfg<Mode, D, 2, 1, OutT>(p, heads, stream);
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
