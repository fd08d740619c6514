// gdn_device.hpp -- device helpers shared by the gfx950 kernels of libgdn.
//
// Fragment convention of every 16x16 MFMA tile in this library (wave64):
//   lane l: idx = l % 16, grp = l / 16.
//   C fragment (f32x4): lane holds C[4*grp + r][idx], r = 0..3.
//   32-deep operand fragment (8 values per lane), slot s = 0..7, logical depth index
//       kslot(grp, s) = (s < 4) ? 4*grp + s : 16 + 4*grp + (s - 4).
//   A operand (16 x 32): lane holds A[idx][kslot(grp, s)].
//   B operand (32 x 16): lane holds B[kslot(grp, s)][idx].
// kslot is a bijection of (grp, s) onto 0..31 and A and B use the same one, so every MFMA
// below computes sum_k A[i][k] B[k][j] exactly once per k. Its point: the C fragments of two
// stacked 16-row tiles (rows 0-15 in slots 0-3, rows 16-31 in slots 4-7) ARE the B fragment
// of a 32-deep product over those rows, and the C fragment of X is also the A fragment of
// X^T. Results of one product feed the next without touching LDS.
//
// bf16 path: v_mfma_f32_16x16x32_bf16 consumes the 8 slots in one instruction.
// fp32 path: v_mfma_f32_16x16x4f32 consumes one slot per instruction (8 instructions), the
//            hardware depth index of instruction s being grp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;  // chunk length (tokens); one token per lane of a wave
constexpr int kWave = 64;

__device__ __forceinline__ int kslot(int grp, int s) {
  return (s < 4) ? 4 * grp + s : 16 + 4 * grp + (s - 4);
}

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ f32x4 mma32(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

// Precision modes.
//   Bf16Mode: inputs q, k, v are bf16 (exact MFMA operands). Every operand the kernels compute
//     (state, T, P, Y, V') is carried as a hi + lo pair of bf16 (x = hi + lo to ~2^-16
//     relative), and a product of two such operands takes hi*hi + hi*lo + lo*hi, all on
//     bf16 MFMA with fp32 accumulation.
//   F32Mode: inputs and operands are fp32 on fp32 MFMA.
//   F32SplitMode (below): fp32 inputs, every operand a hi + lo pair on bf16 MFMA.
struct Bf16Mode {
  using in_t = bf16;
  using frag_t = bf16x8;
  static constexpr bool kSplit = true;
  struct Op {
    bf16x8 hi, lo;
  };
  // hi = RNE(x), lo = RNE(x - hi), two slots per packed conversion; the float value of a hi
  // half is its bits moved to the top of a word, so no slot is converted twice.
  __device__ __forceinline__ static Op make(const float (&x)[8]) {
    Op o;
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
      const bf16x2 h = __builtin_convertvector((f32x2){x[s], x[s + 1]}, bf16x2);
      const uint32_t u = __builtin_bit_cast(uint32_t, h);
      const float h0 = __builtin_bit_cast(float, u << 16);
      const float h1 = __builtin_bit_cast(float, u & 0xffff0000u);
      const bf16x2 l = __builtin_convertvector((f32x2){x[s] - h0, x[s + 1] - h1}, bf16x2);
      o.hi[s] = h[0];
      o.hi[s + 1] = h[1];
      o.lo[s] = l[0];
      o.lo[s + 1] = l[1];
    }
    return o;
  }
  // exact x split
  __device__ __forceinline__ static f32x4 mma_xs(f32x4 c, const frag_t& a, const Op& b) {
    c = mma32(a, b.hi, c);
    return mma32(a, b.lo, c);
  }
  // split x exact (the split operand as A)
  __device__ __forceinline__ static f32x4 mma_sx(f32x4 c, const Op& a, const frag_t& b) {
    c = mma32(a.hi, b, c);
    return mma32(a.lo, b, c);
  }
  // split x split (lo*lo dropped: below fp32 rounding of the sum)
  __device__ __forceinline__ static f32x4 mma_ss(f32x4 c, const Op& a, const Op& b) {
    c = mma32(a.hi, b.hi, c);
    c = mma32(a.hi, b.lo, c);
    return mma32(a.lo, b.hi, c);
  }
  // split x split with the roles of the operands exchanged: the same three products accumulated
  // in the order mma_ss(c, b, a) accumulates them, so that a product computed transposed
  // (C^T = B^T A^T) rounds exactly like the untransposed one
  __device__ __forceinline__ static f32x4 mma_ss_t(f32x4 c, const Op& a, const Op& b) {
    c = mma32(a.hi, b.hi, c);
    c = mma32(a.lo, b.hi, c);
    return mma32(a.hi, b.lo, c);
  }
  // Op stored as [hi fragments of 64 lanes][lo fragments of 64 lanes] = 2 KiB per block.
  __device__ __forceinline__ static Op load_block(const char* blk, int lane) {
    Op o;
    o.hi = *reinterpret_cast<const bf16x8*>(blk + lane * 16);
    o.lo = *reinterpret_cast<const bf16x8*>(blk + 1024 + lane * 16);
    return o;
  }
  __device__ __forceinline__ static void store_block(char* blk, int lane, const Op& o) {
    *reinterpret_cast<bf16x8*>(blk + lane * 16) = o.hi;
    *reinterpret_cast<bf16x8*>(blk + 1024 + lane * 16) = o.lo;
  }
  // Half block (slots 4-7 zero): [hi slots 0-3 of 64 lanes][lo slots 0-3 of 64 lanes] = 1 KiB.
  __device__ __forceinline__ static Op load_half(const char* blk, int lane) {
    const bf16x4 h = *reinterpret_cast<const bf16x4*>(blk + lane * 8);
    const bf16x4 l = *reinterpret_cast<const bf16x4*>(blk + 512 + lane * 8);
    const bf16 z = (bf16)0.f;
    Op o;
    o.hi = bf16x8{h[0], h[1], h[2], h[3], z, z, z, z};
    o.lo = bf16x8{l[0], l[1], l[2], l[3], z, z, z, z};
    return o;
  }
  __device__ __forceinline__ static void store_half(char* blk, int lane, const Op& o) {
    *reinterpret_cast<bf16x4*>(blk + lane * 8) = bf16x4{o.hi[0], o.hi[1], o.hi[2], o.hi[3]};
    *reinterpret_cast<bf16x4*>(blk + 512 + lane * 8) = bf16x4{o.lo[0], o.lo[1], o.lo[2], o.lo[3]};
  }
  // A full or a half block without a branch: the same four 8-byte loads either way (for a half
  // block the second of each pair reads the next lane's slots, or for lane 63 the first bytes
  // after the block, and is replaced by zeros).
  __device__ __forceinline__ static Op load_sel(const char* blk, int lane, bool half) {
    const int st = half ? 8 : 16, lo = half ? 512 : 1024;
    const bf16x4 h0 = *reinterpret_cast<const bf16x4*>(blk + lane * st);
    const bf16x4 h1 = *reinterpret_cast<const bf16x4*>(blk + lane * st + 8);
    const bf16x4 l0 = *reinterpret_cast<const bf16x4*>(blk + lo + lane * st);
    const bf16x4 l1 = *reinterpret_cast<const bf16x4*>(blk + lo + lane * st + 8);
    const uint64_t keep = half ? 0ull : ~0ull;
    const bf16x4 h1k = __builtin_bit_cast(bf16x4, __builtin_bit_cast(uint64_t, h1) & keep);
    const bf16x4 l1k = __builtin_bit_cast(bf16x4, __builtin_bit_cast(uint64_t, l1) & keep);
    Op o;
    o.hi = bf16x8{h0[0], h0[1], h0[2], h0[3], h1k[0], h1k[1], h1k[2], h1k[3]};
    o.lo = bf16x8{l0[0], l0[1], l0[2], l0[3], l1k[0], l1k[1], l1k[2], l1k[3]};
    return o;
  }
};

// fp16 operands of the scan's two products with the state when q / k / v are bf16: K H and Q H.
// K and Q are staged as fp16 (a bf16 value converts exactly unless it lies below 2^-14 in
// magnitude, where the fp16 spacing is 2^-24, or beyond 65504); the state slice is rounded once
// per chunk to fp16 (RNE) for these products, while the state itself stays fp32. Each such
// product is one v_mfma_f32_16x16x32_f16 per 32-deep block instead of the two of an exact x
// hi/lo pair. The update K^T diag(delta) V', T diag(beta) Y and P V' keep bf16 hi/lo pairs (K^T
// converted back from the staged fp16 rows, exactly).
struct Half {
  // 8 slots rounded to fp16 (RNE), two per packed conversion
  __device__ __forceinline__ static f16x8 make(const float (&x)[8]) {
    f16x8 o;
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
      const f16x2 h = __builtin_convertvector((f32x2){x[s], x[s + 1]}, f16x2);
      o[s] = h[0];
      o[s + 1] = h[1];
    }
    return o;
  }
  __device__ __forceinline__ static f32x4 mma(const f16x8& a, const f16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // 16 bytes of 8 bf16 values rewritten as 8 fp16 values (the staging of K and Q rows)
  __device__ __forceinline__ static f32x4 from_bf16(const f32x4& raw) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&raw);
    f32x4 out;
    uint32_t* ow = reinterpret_cast<uint32_t*>(&out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __builtin_bit_cast(float, w[i] << 16);
      const float hi = __builtin_bit_cast(float, w[i] & 0xffff0000u);
      ow[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
    }
    return out;
  }
  // 4 fp16 values (as read by ds_read_b64_tr_b16) to bf16 (RNE; exact for values that were bf16)
  __device__ __forceinline__ static bf16x4 to_bf16(const s16x4& raw) {
    typedef f16 f16x4 __attribute__((ext_vector_type(4)));
    const f16x4 h = __builtin_bit_cast(f16x4, raw);
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const bf16x2 b = __builtin_convertvector((f32x2){(float)h[e], (float)h[e + 1]}, bf16x2);
      o[e] = b[0];
      o[e + 1] = b[1];
    }
    return o;
  }
  __device__ __forceinline__ static bf16x8 to_bf16(const f16x8& h) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 b = __builtin_convertvector((f32x2){(float)h[e], (float)h[e + 1]}, bf16x2);
      o[e] = b[0];
      o[e + 1] = b[1];
    }
    return o;
  }
  // 1 KiB block: the 16-byte fragments of 64 lanes
  __device__ __forceinline__ static f16x8 load_block(const char* blk, int lane) {
    return *reinterpret_cast<const f16x8*>(blk + lane * 16);
  }
  __device__ __forceinline__ static void store_block(char* blk, int lane, const f16x8& o) {
    *reinterpret_cast<f16x8*>(blk + lane * 16) = o;
  }
};

struct F32Mode {
  using in_t = float;
  using frag_t = f32x8;
  static constexpr bool kSplit = false;
  struct Op {
    f32x8 v;
  };
  __device__ __forceinline__ static Op make(const float (&x)[8]) {
    Op o;
#pragma unroll
    for (int s = 0; s < 8; ++s) o.v[s] = x[s];
    return o;
  }
  __device__ __forceinline__ static f32x4 mma_xs(f32x4 c, const frag_t& a, const Op& b) {
    return mma32(a, b.v, c);
  }
  __device__ __forceinline__ static f32x4 mma_ss(f32x4 c, const Op& a, const Op& b) {
    return mma32(a.v, b.v, c);
  }
  // Op stored as 64 lanes x 8 fp32 = 2 KiB per block.
  __device__ __forceinline__ static Op load_block(const char* blk, int lane) {
    Op o;
    o.v = *reinterpret_cast<const f32x8*>(blk + lane * 32);
    return o;
  }
  __device__ __forceinline__ static void store_block(char* blk, int lane, const Op& o) {
    *reinterpret_cast<f32x8*>(blk + lane * 32) = o.v;
  }
  // Half block (slots 4-7 zero): slots 0-3 of 64 lanes = 1 KiB.
  __device__ __forceinline__ static Op load_half(const char* blk, int lane) {
    const f32x4 h = *reinterpret_cast<const f32x4*>(blk + lane * 16);
    Op o;
    o.v = f32x8{h[0], h[1], h[2], h[3], 0.f, 0.f, 0.f, 0.f};
    return o;
  }
  __device__ __forceinline__ static void store_half(char* blk, int lane, const Op& o) {
    *reinterpret_cast<f32x4*>(blk + lane * 16) = f32x4{o.v[0], o.v[1], o.v[2], o.v[3]};
  }
  // A full or a half block without a branch (as Bf16Mode::load_sel: two 16-byte loads).
  __device__ __forceinline__ static Op load_sel(const char* blk, int lane, bool half) {
    const int st = half ? 16 : 32;
    const f32x4 a = *reinterpret_cast<const f32x4*>(blk + lane * st);
    const f32x4 b = *reinterpret_cast<const f32x4*>(blk + lane * st + 16);
    Op o;
    o.v = f32x8{a[0], a[1], a[2], a[3], half ? 0.f : b[0], half ? 0.f : b[1], half ? 0.f : b[2],
                half ? 0.f : b[3]};
    return o;
  }
};

// F32SplitMode: q / k / v stored as fp32 and every product taken on bf16 MFMA with both operands
// as hi + lo bf16 pairs: the inputs are split when they are staged or read, and the workspace
// blocks (stored in F32Mode's layout) when they are read. An operand then
// keeps about 16 significant bits (x = hi + lo to ~2^-17 relative) instead of fp32's 24, and a
// 32-deep block costs three bf16 MFMAs instead of eight fp32 ones. For fp32 q / k / v that
// stand for bf16-derived values (a front end's output) where the fp32 bar is not the contract.
struct F32SplitMode {
  using in_t = float;
  using Op = Bf16Mode::Op;
  using frag_t = Op;
  static constexpr bool kSplit = true;
  __device__ __forceinline__ static Op make(const float (&x)[8]) { return Bf16Mode::make(x); }
  __device__ __forceinline__ static Op split(const f32x8& v) {
    float x[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = v[s];
    return Bf16Mode::make(x);
  }
  __device__ __forceinline__ static f32x4 mma_xs(f32x4 c, const frag_t& a, const Op& b) {
    return Bf16Mode::mma_ss(c, a, b);
  }
  __device__ __forceinline__ static f32x4 mma_ss(f32x4 c, const Op& a, const Op& b) {
    return Bf16Mode::mma_ss(c, a, b);
  }
  __device__ __forceinline__ static f32x4 mma_ss_t(f32x4 c, const Op& a, const Op& b) {
    return Bf16Mode::mma_ss_t(c, a, b);
  }
  // Blocks in F32Mode's layout, split on the way in.
  __device__ __forceinline__ static Op load_block(const char* blk, int lane) {
    return split(F32Mode::load_block(blk, lane).v);
  }
  __device__ __forceinline__ static Op load_half(const char* blk, int lane) {
    return split(F32Mode::load_half(blk, lane).v);
  }
  __device__ __forceinline__ static Op load_sel(const char* blk, int lane, bool half) {
    return split(F32Mode::load_sel(blk, lane, half).v);
  }
};

// 8 values of a 32-deep B fragment from two C fragments (rows 0-15 and 16-31 of the depth).
__device__ __forceinline__ void pack_c_pair(const f32x4& c0, const f32x4& c1, float (&x)[8]) {
  x[0] = c0[0];
  x[1] = c0[1];
  x[2] = c0[2];
  x[3] = c0[3];
  x[4] = c1[0];
  x[5] = c1[1];
  x[6] = c1[2];
  x[7] = c1[3];
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    float y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x;
}
// 4 consecutive doubles (32 bytes, two 16-byte accesses)
typedef double f64x2 __attribute__((ext_vector_type(2)));
struct f64x4 {
  double v[4];
  __device__ double operator[](int i) const { return v[i]; }
};
__device__ __forceinline__ f64x4 ld_f64x4(const double* p) {
  const f64x2 a = *reinterpret_cast<const f64x2*>(p), b = *reinterpret_cast<const f64x2*>(p + 2);
  return f64x4{{a[0], a[1], b[0], b[1]}};
}
__device__ __forceinline__ double wave_inclusive_scan_f64(double x, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x;
}

// Workspace record of one (chunk slot, V head), written by the intra kernel and read by the
// scan kernel. Both matrices are stored as the A operands of 64x64 @ 64x16 products: six
// 32-deep blocks (row tile rt, depth block kb) with kb <= rt/2, block b = tri_block(rt, kb),
// 2 KiB each in the fragment layout of the mode. Blocks 0 (rows 0-15, columns 0-31) and 3
// (rows 32-47, columns 32-63) hold zeros in slots 4-7 of every lane (the 16 columns past the
// diagonal tile of a lower-triangular matrix): they are stored as half blocks, slots 0-3 only.
constexpr int kWsBlockBytes = 2048;
__host__ __device__ constexpr int tri_block(int rt, int kb) {
  return rt < 2 ? rt : 2 + 2 * (rt - 2) + kb;
}
__host__ __device__ constexpr bool ws_half_block(int b) { return b == 0 || b == 3; }
__host__ __device__ constexpr int ws_block_off(int b) {  // 0, 1024, 3072, 5120, 6144, 8192
  return b * kWsBlockBytes - (b > 0 ? kWsBlockBytes / 2 : 0) - (b > 3 ? kWsBlockBytes / 2 : 0);
}
constexpr int kWsMatBytes = ws_block_off(6);    // 10240 bytes per matrix
constexpr int kWsTOff = 0;                      // T*diag(beta)
constexpr int kWsPOff = kWsMatBytes;            // masked decayed Q K^T (times the output scale)
constexpr int kWsGOff = 2 * kWsMatBytes;        // gamma_t = e^{b_t}: 64 fp32
constexpr int kWsDOff = kWsGOff + 256;          // delta_t = e^{b_C - b_t}: 64 fp32
constexpr int kWsRecordBytes = kWsDOff + 256;   // 20992 bytes
static_assert(kWsMatBytes == 10240 && kWsRecordBytes == 20992, "record layout");

// Block b of a record matrix starting at `mat` (global memory or a verbatim LDS copy).
template <typename M>
__device__ __forceinline__ void ws_store(char* mat, int b, int lane, const typename M::Op& o) {
  if (ws_half_block(b))
    M::store_half(mat + ws_block_off(b), lane, o);
  else
    M::store_block(mat + ws_block_off(b), lane, o);
}
template <typename M>
__device__ __forceinline__ typename M::Op ws_load(const char* mat, int b, int lane) {
  return ws_half_block(b) ? M::load_half(mat + ws_block_off(b), lane)
                          : M::load_block(mat + ws_block_off(b), lane);
}
// The same for a block index known only at run time, without a branch (loads that must stay in
// flight across code whose waits the compiler counts exactly). Reads up to 8 (bf16) or 16
// (fp32) bytes past a half block: the next block of the same matrix.
template <typename M>
__device__ __forceinline__ typename M::Op ws_load_nb(const char* mat, int b, int lane) {
  return M::load_sel(mat + ws_block_off(b), lane, ws_half_block(b));
}

// Chunk slot of chunk c of sequence n: n + floor(cu[n] / 64) + c. Injective over all
// (n, c) with c < ceil(len_n / 64), and below num_seqs + floor(total_tokens / 64).
__device__ __forceinline__ int slot_base(const int32_t* cu, int n) { return n + cu[n] / kChunk; }

// Largest n in [0, num_seqs) with slot_base(n) <= slot (slot_base is strictly increasing).
__device__ __forceinline__ int slot_to_seq(const int32_t* cu, int num_seqs, int slot) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (slot_base(cu, mid) <= slot)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}



// ---- LDS staging and operand fragments from staged rows -------------------------------




// 16-byte XOR swizzle of a staged row (keeps the 8 rows that a fragment read touches on
// different LDS banks).
template <int ROWB>
__device__ __forceinline__ int swz(int row) {
  constexpr int NCH = ROWB / 16;
  return (2 * row) & (NCH - 1) & ~1;
}
template <int ROWB, int ES>
__device__ __forceinline__ int swz_off(int row, int col) {
  const int byte = col * ES;
  return row * ROWB + (((byte >> 4) ^ swz<ROWB>(row)) << 4) + (byte & 15);
}

// A fragment of a [64 x D] row-major staged matrix (rows = tokens, depth = d_k). Contractions
// over d_k use a column-contiguous depth order: lane (idx, grp) gets row `row`, columns
// 32 kb + 8 grp + s for slot s = 0..7, i.e. one 16-byte (bf16) or 32-byte (f32) piece. Both
// operands of a d_k contraction must use this order; the scan keeps its state rows in it.
template <int ROWB>
__device__ __forceinline__ bf16x8 afrag(const char* buf, int row, int kb, int grp) {
  return *reinterpret_cast<const bf16x8*>(buf + swz_off<ROWB, 2>(row, 32 * kb + 8 * grp));
}
template <int ROWB>
__device__ __forceinline__ f32x8 afrag_f32(const char* buf, int row, int kb, int grp) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(buf + swz_off<ROWB, 4>(row, 32 * kb + 8 * grp));
  const f32x4 hi =
      *reinterpret_cast<const f32x4*>(buf + swz_off<ROWB, 4>(row, 32 * kb + 8 * grp + 4));
  f32x8 f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f[s] = lo[s];
    f[4 + s] = hi[s];
  }
  return f;
}

// ---- 8-value vector accesses (one 16-byte bf16 / two 16-byte fp32 accesses) ------------

// Eight consecutive input values kept as loaded (converted where used), so that many loads
// can be in flight before the first one is consumed.
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16> {
  bf16x8 r;
  __device__ __forceinline__ void load(const bf16* p) { r = *reinterpret_cast<const bf16x8*>(p); }
  // streaming read (data used once): nontemporal hint
  __device__ __forceinline__ void load_nt(const bf16* p) {
    r = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
  }
  __device__ __forceinline__ void to(float (&x)[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)r[e];
  }
  __device__ __forceinline__ float at(int e) const { return (float)r[e]; }  // e compile-time
  __device__ __forceinline__ bf16 raw(int e) const { return r[e]; }
};
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void load_nt(const float* p) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  __device__ __forceinline__ void to(float (&x)[8]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[4 + e] = b[e];
    }
  }
  __device__ __forceinline__ float at(int e) const { return e < 4 ? a[e] : b[e - 4]; }
  __device__ __forceinline__ float raw(int e) const { return at(e); }
};

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&x)[8]);
template <>
__device__ __forceinline__ void store8<bf16>(bf16* p, const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)x[e];
  *reinterpret_cast<bf16x8*>(p) = r;
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&x)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = x[e];
    b[e] = x[4 + e];
  }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// Eight stored values moved as they are (no arithmetic), nontemporal.
__device__ __forceinline__ void store8_raw_nt(bf16* p, const bf16 (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e];
  __builtin_nontemporal_store(r, reinterpret_cast<bf16x8*>(p));
}
__device__ __forceinline__ void store8_raw_nt(float* p, const float (&x)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = x[e];
    b[e] = x[4 + e];
  }
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p + 4));
}

// Streaming write (not read again by this kernel): nontemporal hint.
template <typename T>
__device__ __forceinline__ void store8_nt(T* p, const float (&x)[8]);
template <>
__device__ __forceinline__ void store8_nt<bf16>(bf16* p, const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)x[e];
  __builtin_nontemporal_store(r, reinterpret_cast<bf16x8*>(p));
}
template <>
__device__ __forceinline__ void store8_nt<float>(float* p, const float (&x)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = x[e];
    b[e] = x[4 + e];
  }
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p + 4));
}

// Barrier for LDS traffic only: waits for this wave's own LDS reads and writes (lgkmcnt) and
// for the other waves, but not for outstanding global loads (a fence would wait for those too,
// serialising the prefetch of the next chunk with this one). The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- 64x64 fp32 matrices in LDS (the chunk's triangular systems) ------------------------

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

// T = (I + A)^-1 of a unit-lower-triangular 64x64 matrix, in place: on entry the fp32 matrix at
// M (row stride kLd, in LDS) holds A in its lower triangle (diagonal blocks: strictly lower part
// and zeros above; blocks above the diagonal are never read), on exit T on and below the
// diagonal (its diagonal blocks hold zeros above their diagonal; blocks above the diagonal keep
// whatever they held). Every wave of the workgroup calls this (it has three workgroup
// barriers and ends with a fourth); a wave may serve two matrices at once:
//   msub  (or null): this wave inverts the four 16x16 diagonal blocks of msub by forward
//         substitution, lane (blk, c) = (lane / 16, lane % 16) solving for column c of block
//         blk: x_i = delta_ic - sum_{j<i} A_ij x_j; row i of a block is read as 16-byte pieces
//         that the block's 16 lanes share (one address per lane group);
//   mpair (or null), wl in {0, 1}: this wave is wave wl of the pair that forms the blocks below
//         the diagonal of mpair (after the diagonal blocks) by 16x16 fp32 MFMA products:
//         level 2: T_10 = -T_11 A_10 T_00 (wl = 0), T_32 = -T_33 A_32 T_22 (wl = 1);
//         level 3, column block jb = wl: X_i = sum_{kb=jb..1} A_{i,kb} T_{kb,jb} (i = 2, 3),
//         T_{2,jb} = -T_22 X_2, T_{3,jb} = -(T_32 X_2 + T_33 X_3).
__device__ __forceinline__ void invert_unit_lower64(float* msub, float* mpair, int wl, int lane) {
  const int idx = lane & 15, grp = lane >> 4;
  if (msub) {
    const int blk = lane >> 4, c = lane & 15;
    float* Ab = msub + (16 * blk) * kLd + 16 * blk;
    float x[16];
    x[0] = c == 0 ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      float a[16];
#pragma unroll
      for (int q = 0; q < (i + 3) / 4; ++q) {
        const f32x4 a4 = row4(Ab + i * kLd + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[4 * q + e] = a4[e];
      }
      float part[4] = {0.f, 0.f, 0.f, 0.f};  // 4 independent chains
#pragma unroll
      for (int jj = 0; jj < i; ++jj) part[jj & 3] = fmaf(a[jj], x[jj], part[jj & 3]);
      x[i] = (i == c) ? 1.f : -((part[0] + part[1]) + (part[2] + part[3]));
    }
    // row i is written after its own read (x_i depends on it); other rows are disjoint
#pragma unroll
    for (int i = 0; i < 16; ++i) Ab[i * kLd + c] = x[i];
  }
  lds_barrier();
  // level 2 (over A_10, A_32: each wave reads its block into M before writing it)
  if (mpair) {
    const int ib = 2 * wl + 1, jb = 2 * wl;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const f32x4 M = mm16_ll(mpair + 16 * ib * kLd + 16 * jb, mpair + 16 * jb * kLd + 16 * jb, z,
                            idx, grp);
    const f32x4 R = mm16_lr(mpair + 16 * ib * kLd + 16 * ib, M, z, idx, grp);
    store_c16(mpair + 16 * ib * kLd + 16 * jb, R, idx, grp, -1.f);
  }
  lds_barrier();
  // level 3: wave 0 of the pair reads A_21 and A_31, which wave 1 overwrites, so the stores
  // wait for a barrier
  f32x4 T2 = {0.f, 0.f, 0.f, 0.f}, T3 = {0.f, 0.f, 0.f, 0.f};
  if (mpair) {
    const int jb = wl;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 X2 = z, X3 = z;
    for (int kb = jb; kb < 2; ++kb) {
      const float* Tk = mpair + 16 * kb * kLd + 16 * jb;
      X2 = mm16_ll(mpair + 32 * kLd + 16 * kb, Tk, X2, idx, grp);
      X3 = mm16_ll(mpair + 48 * kLd + 16 * kb, Tk, X3, idx, grp);
    }
    T2 = mm16_lr(mpair + 32 * kLd + 32, X2, z, idx, grp);
    T3 = mm16_lr(mpair + 48 * kLd + 32, X2, z, idx, grp);
    T3 = mm16_lr(mpair + 48 * kLd + 48, X3, T3, idx, grp);
  }
  lds_barrier();
  if (mpair) {
    store_c16(mpair + 32 * kLd + 16 * wl, T2, idx, grp, -1.f);
    store_c16(mpair + 48 * kLd + 16 * wl, T3, idx, grp, -1.f);
  }
  lds_barrier();
}

}  // namespace gdn
