// Helpers shared by the tree verification kernels (gfx950): LDS layouts of
// the N x N matrices, bf16 hi + lo splitting, the per-node path solves of
// T = (I + A)^{-1}, XCD-aware workgroup numbering and the MFMA helpers.
#pragma once

#include "gdn_common.h"

namespace gdn {

__device__ inline void copy4e(float* d, const float* s) {
  *reinterpret_cast<f32x4*>(d) = *reinterpret_cast<const f32x4*>(s);
}

// 8-element k-slice of a global row as MFMA operand(s): FP32 input is split
// into bf16 hi + lo (used only on the FP32-input path).
__device__ inline void frag_global(const float* p, bool ok, bf16x8& hi, bf16x8& lo) {
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
  if (ok) {
    a = load4(p);
    b = load4(p + 4);
  }
  split8(a, b, hi, lo);
}

__device__ inline bf16x8 lds_bf16x8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Store 4 floats as bf16 hi (at p) and lo (at p + lo_off), 8 bytes each.
__device__ inline void store_split4(bf16_t* p, int lo_off, const f32x4& x) {
  u32x2 hi, lo;
  float r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 hb = (__bf16)x[e];
    r[e] = x[e] - (float)hb;
    reinterpret_cast<__bf16*>(&hi)[e] = hb;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) reinterpret_cast<__bf16*>(&lo)[e] = (__bf16)r[e];
  *reinterpret_cast<u32x2*>(p) = hi;
  *reinterpret_cast<u32x2*>(p + lo_off) = lo;
}

// Store one float as bf16 hi (at p) and lo (at p + lo_off).
__device__ inline void store_split1(bf16_t* p, int lo_off, float x) {
  const __bf16 hb = (__bf16)x;
  reinterpret_cast<__bf16*>(p)[0] = hb;
  reinterpret_cast<__bf16*>(p)[lo_off] = (__bf16)(x - (float)hb);
}

// Hardware dispatches workgroup ids round-robin over the 8 XCDs; renumber so
// that consecutive logical ids (the tiles of one head) share an XCD.
__device__ inline int xcd_logical_id(int bid, int nblocks) {
  constexpr int kXcds = 8;
  if (nblocks % kXcds) return bid;
  return (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
}

// LDS row strides.  FP32 N x N rows of 272 B: the four row groups of a
// 16 x 16 tile's stores (rows 4 lg + r) start 16 banks apart.  Split bf16
// rows of 144 B keep every row 16-byte aligned for the 4-wave kernel's
// 16-byte fragment reads.  Staged Q/K rows of 544 B: a 16-byte fragment read
// of 16 rows is free of bank conflicts (528-byte rows measured eight times
// the conflict stalls of the whole kernel).
constexpr int kLd = kMaxNodes + 4;         // row stride (floats) of FP32 N x N matrices
constexpr int kLdH = kMaxNodes + 8;        // row stride (bf16) of split matrices
constexpr int kSplitLo = kMaxNodes * kLdH; // bf16 offset of the lo half of a split matrix
constexpr int kMatFloats = kMaxNodes * kLdH; // floats of a region holding either form
constexpr int kQKRows = 2 * kMaxNodes;     // Q rows then K rows
constexpr int kQKStride = kMaxDim + 16;    // bf16 elements per staged row
constexpr int kQKBytes = kQKRows * kQKStride * 2;
constexpr int kPathMax = 16;               // register-resident path solve up to this depth

// Row t of T on t's root path p_0..p_{d-1} = t, for d <= kPathMax:
//   x_{d-1} = 1,  x_b = -sum_{a > b} x_a A[p_a][p_b]
// solves x^T (I + A)|_path = e_t^T and T[t][p_b] = x_b.  Terms with a <= b or
// a >= d vanish on their own (x_a not yet set, or the padding), so the sum is
// unconditional and its LDS reads issue together.
template <typename Put>
__device__ inline void path_solve_registers(int t, uint64_t m, int d, const float* A, Put put) {
  int p[kPathMax];
  float x[kPathMax];
  uint64_t mm = m;
#pragma unroll
  for (int a = 0; a < kPathMax; ++a) {
    p[a] = mm ? __builtin_ctzll(mm) : t;
    mm &= mm - 1ull;
    x[a] = (a == d - 1) ? 1.f : 0.f;
  }
  put(t, 1.f);
  for (int b = d - 2; b >= 0; --b) {
    int pb = t;
#pragma unroll
    for (int a = 0; a < kPathMax; ++a)
      if (a == b) pb = p[a];
    float acc = 0.f;
#pragma unroll
    for (int a = 0; a < kPathMax; ++a) acc = fmaf(x[a], A[p[a] * kLd + pb], acc);
    const float xb = -acc;
    put(pb, xb);
#pragma unroll
    for (int a = 0; a < kPathMax; ++a)
      if (a == b) x[a] = xb;
  }
}

// The same for paths of at most P nodes with the path's P x P block of A read
// into registers first (one round of LDS reads), then substituted in
// registers: each step is a few FMAs instead of a wait on LDS.  The sums run
// over a = b+1 .. P-1 in the order path_solve_registers uses (its terms with
// a <= b are exact zeros), so every P gives the same bits.
template <int P, typename Put>
__device__ inline void path_solve_block(int t, uint64_t m, int d, const float* A, Put put) {
  int p[P];
  uint64_t mm = m;
#pragma unroll
  for (int a = 0; a < P; ++a) {
    p[a] = mm ? __builtin_ctzll(mm) : t;
    mm &= mm - 1ull;
  }
  float Ab[P][P];  // Ab[a][b] = A[p_a][p_b] for a > b (zero above the path)
#pragma unroll
  for (int a = 0; a < P; ++a)
#pragma unroll
    for (int b = 0; b < a; ++b) Ab[a][b] = A[p[a] * kLd + p[b]];
  float x[P];
#pragma unroll
  for (int a = 0; a < P; ++a) x[a] = (a == d - 1) ? 1.f : 0.f;
  // x_b = -sum_{a > b} x_a A[p_a][p_b], b = d-2 .. 0; entries a >= d have x_a = 0
#pragma unroll
  for (int b = P - 2; b >= 0; --b) {
    float acc = 0.f;
#pragma unroll
    for (int a = b + 1; a < P; ++a) acc = fmaf(x[a], Ab[a][b], acc);
    if (b < d - 1) x[b] = -acc;
  }
  put(t, 1.f);
#pragma unroll
  for (int b = 0; b < P; ++b)
    if (b < d - 1) put(p[b], x[b]);
}

// v_mfma_f32_16x16x4f32: D[16x16] += A[16x4] * B[4x16] in FP32.  Lane l holds
// A[l % 16][l / 16] and B[l / 16][l % 16]; D as for the bf16 form (row
// 4 * (l / 16) + r, column l % 16).
__device__ inline f32x4 mfma16x16x4f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Wait states after the last MFMA of a chain whose accumulators are read on
// the far side of a branch.  The compiler pads a read of an MFMA result in
// the same basic block, but not on a path that leaves the block right after
// the MFMA: after the Y contraction, a wave that is last at the following
// barrier passes it at once and, through the uniform branch behind it, read
// the last accumulator register before the MFMA had written it (a few
// outputs then varied from run to run in the last bits).  Two s_nop 7 give
// 16 wait states on every path, more than any MFMA here needs.
__device__ inline void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The same, with the accumulators passed through the asm as operands: the
// MFMAs that produce them cannot then be moved below the wait states (an
// ordering that sched_barrier alone does not guarantee to every pass), and a
// copy out of accumulator registers happens in straight-line code, where the
// compiler pads it itself.
template <typename X>
__device__ inline void pin_vgpr(X& x) {
  asm volatile("" : "+v"(x));
}
template <typename... Acc>
__device__ inline void mfma_drain(Acc&... acc) {
  (pin_vgpr(acc), ...);
  mfma_drain();
}
template <int NA>
__device__ inline void mfma_drain_all(f32x4 (&acc)[NA]) {
#pragma unroll
  for (int i = 0; i < NA; ++i) pin_vgpr(acc[i]);
  mfma_drain();
}

// SiLU output gate fused into the epilogue (the GATE variants, bf16 q/k/v
// only): Y = bf16(O * SiLU(gate)) with gate row t at gate + (b N + t) ldg + h dv
// (the gate block of the layer's projection output), written instead of O.
// A compile-time variant: the gate's loads and registers would otherwise
// slow every plain verification.
struct GateArgs {
  const float* gate;
  int ldg;
  bf16_t* Y;
};

}  // namespace gdn
