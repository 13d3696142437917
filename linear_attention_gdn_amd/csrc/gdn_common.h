// Shared host/device definitions for libgdnspec (gfx950 / CDNA4).
//
// Factor-record layout, bf16 helpers and the MFMA fragment
// conventions used by the verification and commit kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdnspec.h"

namespace gdn {

constexpr int kMaxNodes = 64;  // one wave64 lane / one uint64 mask bit per node
constexpr int kMaxDim = 256;
constexpr int kMaxLds = 160 * 1024;  // LDS bytes one workgroup may hold (gfx950)
constexpr size_t kAlign = 256;

__host__ __device__ inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline size_t elem_bytes(int dtype) { return dtype == GDN_BF16 ? 2 : 4; }

// Factor record: [u' f32 B*H*N*dv | G f32 B*H*N | K B*H*N*dk | parents i32 B*N | mask u64 B*N]
struct RecordLayout {
  size_t off[5];
  size_t total;
};

inline RecordLayout record_layout(int B, int N, int H, int dk, int dv, int dtype) {
  RecordLayout L;
  const size_t bhn = (size_t)B * H * N;
  size_t o = 0;
  L.off[0] = o;
  o = align_up(o + bhn * dv * 4);
  L.off[1] = o;
  o = align_up(o + bhn * 4);
  L.off[2] = o;
  o = align_up(o + bhn * dk * elem_bytes(dtype));
  L.off[3] = o;
  o = align_up(o + (size_t)B * N * 4);
  L.off[4] = o;
  o = align_up(o + (size_t)B * N * 8);
  L.total = o;
  return L;
}

// Device views of a factor record.
template <typename KT>
struct Record {
  float* up;         // [B][H][N][dv]
  float* G;          // [B][H][N]
  KT* K;             // [B][H][N][dk]
  int32_t* parents;  // [B][N]
  uint64_t* mask;    // [B][N]
};

template <typename KT>
inline Record<KT> record_views(void* base, const RecordLayout& L) {
  char* p = static_cast<char*>(base);
  Record<KT> r;
  r.up = reinterpret_cast<float*>(p + L.off[0]);
  r.G = reinterpret_cast<float*>(p + L.off[1]);
  r.K = reinterpret_cast<KT*>(p + L.off[2]);
  r.parents = reinterpret_cast<int32_t*>(p + L.off[3]);
  r.mask = reinterpret_cast<uint64_t*>(p + L.off[4]);
  return r;
}

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------

typedef uint16_t bf16_t;  // bfloat16 storage bits

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

__device__ inline float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }
// FP32 -> bf16, round to nearest even
__device__ inline bf16_t to_bf16(float x) { return __builtin_bit_cast(bf16_t, (__bf16)x); }
// SiLU(x) = x sigmoid(x), as the output gate and the convolution use it
__device__ inline float silu(float x) { return x / (1.0f + expf(-x)); }

// Load 4 consecutive elements as float.
__device__ inline f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ inline f32x4 load4(const bf16_t* p) {
  u32x2 w = *reinterpret_cast<const u32x2*>(p);
  f32x4 r;
  r.x = __uint_as_float(w.x << 16);
  r.y = __uint_as_float(w.x & 0xffff0000u);
  r.z = __uint_as_float(w.y << 16);
  r.w = __uint_as_float(w.y & 0xffff0000u);
  return r;
}

// Raw 4-element vectors: kept as loaded (bf16 bits or FP32) so that the load
// is not consumed (and waited for) before it is needed; widen4 converts.
template <typename T>
struct Raw4;
template <>
struct Raw4<float> {
  using type = f32x4;
};
template <>
struct Raw4<bf16_t> {
  using type = u32x2;
};
template <typename T>
__device__ inline typename Raw4<T>::type raw4(const T* p) {
  return *reinterpret_cast<const typename Raw4<T>::type*>(p);
}
__device__ inline f32x4 widen4(const f32x4& x) { return x; }
__device__ inline f32x4 widen4(const u32x2& w) {
  f32x4 r;
  r.x = __uint_as_float(w.x << 16);
  r.y = __uint_as_float(w.x & 0xffff0000u);
  r.z = __uint_as_float(w.y << 16);
  r.w = __uint_as_float(w.y & 0xffff0000u);
  return r;
}
__device__ inline float widen1(float x) { return x; }
__device__ inline float widen1(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Split 8 floats into bf16 hi + lo with x = hi + lo + r, |r| <= 2^-16 |x|
// (both roundings to nearest even; x - hi is exact in fp32).
__device__ inline void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
  float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h = (__bf16)x[e];
    hi[e] = h;
    lo[e] = (__bf16)(x[e] - (float)h);
  }
}

// Loads are issued unconditionally from a clamped (always valid) address and
// masked afterwards: a load under a branch makes the compiler wait for it
// before the branch joins, which serialises memory round trips.
__device__ inline int clampi(int x, int hi) { return x < hi ? x : hi; }
__device__ inline f32x4 mask4(const f32x4& x, bool ok) {
  return ok ? x : f32x4{0.f, 0.f, 0.f, 0.f};
}

// 8 bf16 values already in bf16: reinterpret a 16-byte load.
__device__ inline bf16x8 load_bf16x8(const bf16_t* p) {
  u32x4 w = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, w);
}

__device__ inline bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

// Sum over each row of 16 lanes with DPP (VALU-speed cross-lane moves inside
// a row): rotate-by-8 and rotate-by-4 fold the row to four partial sums,
// two quad permutations finish it.  Every lane of the row ends with the sum.
// These patterns never read outside the row, so bound_ctrl may be set, which
// lets the compiler fuse each move into its add (one v_add_f32 with a DPP
// source per stage).
template <int CTRL>
__device__ inline float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ inline float row16_sum(float x) {
  x += dpp_f32<0x128>(x);  // row_ror:8
  x += dpp_f32<0x124>(x);  // row_ror:4
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  return x;
}

// Sum over each half-wave (32 lanes): the 16-lane row sums, then
// v_permlane16_swap exchanges the two rows of each half on the VALU (no LDS
// round trip), so every lane of the half ends with the total.  The empty asm
// copy keeps the swap's two operands distinct to the compiler, which otherwise
// folds a swap of a value with itself.
__device__ inline float half32_sum(float x) {
  x = row16_sum(x);
  const unsigned a = __builtin_bit_cast(unsigned, x);
  unsigned b;
  asm("" : "=v"(b) : "0"(a));
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Sum over the whole wave (64 lanes) into every lane: the 16-lane row sums,
// then v_permlane16_swap (rows 0<->1, 2<->3) and v_permlane32_swap (the two
// halves) exchange partial sums on the VALU.
__device__ inline float wave64_sum(float x) {
  x = row16_sum(x);
  unsigned a = __builtin_bit_cast(unsigned, x);
  unsigned b;
  asm("" : "=v"(b) : "0"(a));
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  x = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  a = __builtin_bit_cast(unsigned, x);
  asm("" : "=v"(b) : "0"(a));
  const auto r2 = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return __builtin_bit_cast(float, (unsigned)r2[0]) + __builtin_bit_cast(float, (unsigned)r2[1]);
}

// Sum over the whole wave delivered only to its last row (lanes 48..63): the
// row sums, then DPP row_bcast:15 (each row adds the previous row's sum; row 0
// reads zero) and row_bcast:31 (rows 2 and 3 add lane 31, which then holds
// rows 0 + 1).  Full row masks with bound_ctrl let each step fuse into one
// v_add_f32_dpp; rows 0..2 end with partial sums.
__device__ inline float wave64_sum_hi(float x) {
  x = row16_sum(x);
  x += dpp_f32<0x142>(x);  // row_bcast:15
  x += dpp_f32<0x143>(x);  // row_bcast:31
  return x;
}

// Sum over the whole wave as a wave-uniform value: the last row's complete
// sum (wave64_sum_hi) read from lane 63 into a scalar register.  The row
// sums are added in the same pairs as in wave64_sum, (r3 + r2) + (r1 + r0)
// against (r0 + r1) + (r2 + r3), so the result is bitwise the same.
__device__ inline float wave64_sum_uniform(float x) {
  x = wave64_sum_hi(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Two sums over the whole wave, both as wave-uniform values, from one
// reduction: v_permlane32_swap of the two registers leaves a's upper-half
// lanes beside a's lower half and b's lower half beside b's upper half, so
// one add gives lanes 0..31 a's and lanes 32..63 b's pairwise partials; the
// DPP row sums and one row broadcast then complete a in lane 31 and b in
// lane 63, read into scalar registers.
__device__ inline void wave64_sum2_uniform(float a, float b, float& sa, float& sb) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                   __builtin_bit_cast(unsigned, b), false, false);
  float x = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  x = row16_sum(x);
  x += dpp_f32<0x142>(x);  // row_bcast:15: rows 1 and 3 complete
  sa = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  sb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].
// Fragment convention (lane l of a wave64):
//   A: row i = l % 16, k = 8 * (l / 16) + e, e = 0..7
//   B: col j = l % 16, k = 8 * (l / 16) + e
//   D: row i = 4 * (l / 16) + r, col j = l % 16, r = 0..3
__device__ inline f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: D[16x16] += A[16x16] * B[16x16], operands as the
// bit patterns of 4 bf16 values:
//   A: row i = l % 16, k = 4 * (l / 16) + e, e = 0..3
//   B: col j = l % 16, k = 4 * (l / 16) + e
//   D: row i = 4 * (l / 16) + r, col j = l % 16, r = 0..3
// A lane's four D rows of one product are exactly its B operand for the same
// 16-wide block of k in the next product, so a chain of products over a
// 16-row blocking passes its intermediate from registers to registers.
typedef __attribute__((ext_vector_type(4))) short s16x4;
__device__ inline f32x4 mfma16x16x16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Split 4 floats into bf16 hi + lo operand bits (as split8).
__device__ inline void split4(const f32x4& x, s16x4& hi, s16x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 h = (__bf16)x[e];
    hi[e] = __builtin_bit_cast(short, h);
    lo[e] = __builtin_bit_cast(short, (__bf16)(x[e] - (float)h));
  }
}

}  // namespace gdn
