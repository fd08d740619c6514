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
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

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
struct Bf16Mode {
  using in_t = bf16;
  using frag_t = bf16x8;
  static constexpr bool kSplit = true;
  struct Op {
    bf16x8 hi, lo;
  };
  __device__ __forceinline__ static Op make(const float (&x)[8]) {
    Op o;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16 h = (bf16)x[s];
      o.hi[s] = h;
      o.lo[s] = (bf16)(x[s] - (float)h);
    }
    return o;
  }
  // exact x split
  __device__ __forceinline__ static f32x4 mma_xs(f32x4 c, const frag_t& a, const Op& b) {
    c = mma32(a, b.hi, c);
    return mma32(a, b.lo, c);
  }
  // split x split (lo*lo dropped: below fp32 rounding of the sum)
  __device__ __forceinline__ static f32x4 mma_ss(f32x4 c, const Op& a, const Op& b) {
    c = mma32(a.hi, b.hi, c);
    c = mma32(a.hi, b.lo, c);
    return mma32(a.lo, b.hi, c);
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

// Workspace record of one (chunk slot, V head), written by the intra kernel and read by the
// scan kernel. Both matrices are stored as the A operands of 64x64 @ 64x16 products: six
// 32-deep blocks (row tile rt, depth block kb) with kb <= rt/2, 2 KiB each.
constexpr int kWsBlockBytes = 2048;
constexpr int kWsTOff = 0;                      // T*diag(beta): 6 blocks
constexpr int kWsPOff = 6 * kWsBlockBytes;      // masked decayed Q K^T: 6 blocks
constexpr int kWsGOff = 12 * kWsBlockBytes;     // gamma_t = e^{b_t}: 64 fp32
constexpr int kWsDOff = kWsGOff + 256;          // delta_t = e^{b_C - b_t}: 64 fp32
constexpr int kWsRecordBytes = kWsDOff + 256;   // 25088 bytes

__host__ __device__ constexpr int tri_block(int rt, int kb) {
  return rt < 2 ? rt : 2 + 2 * (rt - 2) + kb;
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


typedef short s16x4 __attribute__((ext_vector_type(4)));


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

}  // namespace gdn
