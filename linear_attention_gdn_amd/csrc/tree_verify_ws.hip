// Tree verification with split wave roles (gfx950), bf16 q/k/v: the form
// gdn_tree_verify, gdn_tree_verify_delayed and the gated layer verify take
// for bf16 inputs, with 16, 32 or 64 state rows per tile (one state wave per
// 16 rows), the tile width chosen by the caller from the number of heads so
// that the grid covers the GPU.
//
// SpecLA review, "What carries the argument" and Figures, Figure 4 caption:
// the same factorized verification as tree_verify.hip (one workgroup per
// (sequence, head, tile of state rows); outputs, factor record and the
// delayed commit identical in definition), organised for this GPU so that the
// long read of the state tile overlaps the chain of small per-head steps
// instead of preceding it.  Two roles:
//
//   head waves (0-3): load and stage Q and K in LDS, build the topology
//     (wave 0, pointer jumping), the Gram blocks Q K^T and K K^T (bf16 MFMA),
//     the masked and scaled A and Attn, and T = (I + A)^{-1} (per-node path
//     solves; blocked forward substitution for paths deeper than 16);
//   state waves (4 .. 3 + SW): wave 4 + c owns state rows 16 c .. 16 c + 15
//     of the tile (16- and 32-row tiles of the delayed form instead have
//     four, waves 4-7, 4 / SW per 16-row group, each with one part of the
//     group's columns, the others handing their contraction sums to the
//     group's first, which alone runs the epilogue).  They request their state rows and V at once (straight
//     into MFMA operand registers); for the delayed form each finds the
//     previous draft's accepted path itself and requests the path's k rows
//     (staged in LDS together) and u' of its rows, and the path is applied to
//     its rows either block by block inside the contraction (64-row tiles,
//     where the state rows arrive only as fast as the memory system drains
//     them) or at once while the head waves still wait for Q and K (narrower
//     tiles).  They run the contraction [Q; K] S0^T on bf16 MFMA (FP32 state
//     split into bf16 hi + lo) while writing the committed rows back, form
//     R = beta (V - e^G K S0^T), and after T is ready chain
//     U' = T R and O = scale e^G Q S0^T + Attn U' through registers as
//     16x16x16 products, the transposed products giving each lane four
//     consecutive state rows of one node, stored as 16-byte vectors.
//
// The head waves synchronise among themselves through an LDS counter (the
// state waves only wait for the staging and topology), and the two roles
// meet at one workgroup barrier where T is complete.  A head wave and a state
// wave share a SIMD, so the head's scalar-heavy steps and the state's matrix
// products issue side by side.
#include <type_traits>

#include "tree_common.h"

namespace gdn {

constexpr int kWsChunk = 16;  // accepted-path nodes staged per round by each state wave

// Split bf16 matrices (Attn, T) here have 136-byte rows, read 8 bytes at a
// time: the four row groups of a tile's stores then start on different banks.
constexpr int kLdS = kMaxNodes + 4;
constexpr int kSplitLoS = kMaxNodes * kLdS;
// Staged k rows of the delayed commit: 576-byte rows, so the commit's reads
// of four path nodes' rows (one per lane group) start on different banks.
constexpr int kCkStride = kMaxDim + 32;

// State waves per tile: one per 16 rows, except with a delayed commit, where
// 16- and 32-row tiles also have four, one per SIMD: each 16-row group's rows
// are shared by 4 / SW waves that split the state's columns (the commit and
// the contraction then run on all four).
template <int SW, bool DLY>
constexpr int ws_state_waves() { return DLY && SW < 4 ? 4 : SW; }

template <bool DLY, int SW>
struct WsLds {
  static constexpr int NSW = ws_state_waves<SW, DLY>();
  alignas(16) bf16_t qk[kQKRows * kQKStride];  // Q rows, then K rows (bf16, zero-padded)
  alignas(16) float A[kMatFloats];        // A (FP32)
  alignas(16) float QK[kMatFloats];       // Attn (split bf16)
  alignas(16) float T[kMatFloats];        // T: zeros, then FP32 rows or split bf16
  uint64_t mask[kMaxNodes];
  float G[kMaxNodes], eG[kMaxNodes], beta[kMaxNodes];
  int bad;
  int sync;   // arrivals at the head waves' own barriers
  int csync;  // arrivals of the state waves at the staged k rows
  int ysync[4];  // per 16-row group: arrivals of the other parts' contractions in yx
  // delayed commit: per state wave the accepted path (root first) and its
  // coefficients; the k rows of the path's first kWsChunk nodes (zero rows
  // past the path), staged by the state waves together
  int dnode[DLY ? NSW : 1][kMaxNodes];
  float dc[DLY ? NSW : 1][kMaxNodes];
  alignas(16) bf16_t ck[DLY ? kWsChunk * kCkStride : 8];
  // split tiles: the other parts' contraction accumulators [group][part - 1][i][lane]
  alignas(16) f32x4 yx[NSW > SW ? SW : 1][NSW > SW ? NSW / SW - 1 : 1][NSW > SW ? 2 * (kMaxNodes / 16) : 1][64];
};

// The head waves synchronise among themselves through an LDS counter, so the
// state waves, busy issuing the loads of their state rows (which the memory
// system accepts only as fast as it drains them), never hold them up: each
// head wave completes its LDS operations, adds one, and waits until the
// counter reaches `target` (four arrivals per round).  A state wave waits
// without arriving (the state waves arrive only at a second counter of the
// same kind, for the delayed commit's staged k rows).  One wave's LDS operations complete in order, and LDS is
// one memory, so the data written before an arrival is visible to every wave
// that has seen the count.  The wait is bounded (far beyond any real wait),
// so a wave can never spin forever.
__device__ inline void ws_arrive(int* ctr) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ inline void ws_wait(int* ctr, int target) {
  for (int i = 0; i < (1 << 22); ++i) {
    const int c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (__builtin_amdgcn_readfirstlane(c) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}
__device__ inline void ws_sync(int* ctr, int target) {
  ws_arrive(ctr);
  ws_wait(ctr, target);
}

template <int NQT, bool DLY, int SW, bool GATE>
__global__ __launch_bounds__((256 + 64 * ws_state_waves<SW, DLY>())) void tree_ws_kernel(
    int N, int H, int dk, int dv, int ntiles, float* __restrict__ S0,
    const int32_t* __restrict__ parents, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ g, float scale, float* __restrict__ out, Record<bf16_t> rec,
    uint64_t* __restrict__ mask_out, int32_t* __restrict__ dev_status, Record<bf16_t> prev,
    int Npv, const int32_t* __restrict__ last_acc, int32_t* __restrict__ commit_status,
    GateArgs ga) {
  constexpr int BV = 16 * SW;  // state rows per tile: 16 per state wave
  constexpr int Np = 16 * NQT;
  constexpr int KS = kMaxDim / 32;          // 32-wide k steps of the contraction
  // 16- and 32-row tiles with a delayed commit: 4 / SW state waves on the
  // same 16 rows, each holding, committing and contracting one part of the
  // state's columns (k steps kbase .. + KSL - 1); otherwise one state wave
  // per 16 rows with every column
  constexpr int NSW = ws_state_waves<SW, DLY>();
  constexpr bool KSPLIT = NSW > SW;
  // Without the delayed commit the one state wave of a 16-row group sums the
  // same column parts apart (the parts after the first in two accumulator
  // sets used in turn) and adds them in part order, the split form's order,
  // so that the delayed form with no path to apply is bitwise this one
  constexpr int kParts = SW < 4 ? 4 / SW : 1;  // column parts per 16-row group
  constexpr int KPART = KS / kParts;          // k steps per part
  constexpr bool kHalves = kParts > 1 && !KSPLIT;
  constexpr int KSL = KSPLIT ? KPART : KS;

  __shared__ WsLds<DLY, SW> sm;
  bf16_t* const QKs = sm.qk;
  float* const KK = sm.A;
  bf16_t* const Attn = reinterpret_cast<bf16_t*>(sm.QK);
  float* const Tl = sm.T;
  bf16_t* const Ts = reinterpret_cast<bf16_t*>(sm.T);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool head = wave < 4;  // uniform per wave
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int koff = 8 * lg;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int tile = lid % ntiles;
  const int bh = lid / ntiles;
  const int b = bh / H;
  const int h = bh % H;
  const int r0 = tile * BV;
  // state waves: rows 16 cj .. 16 cj + 15 of the tile; lane l16's row (as an
  // MFMA operand) and the four rows 16 cj + 4 lg .. + 3 (as a transposed result)
  const int cj = wave >= 4 ? (KSPLIT ? (wave - 4) / kParts : wave - 4) : 0;
  const int kbase = (wave >= 4 && KSPLIT) ? KSL * ((wave - 4) % kParts) : 0;  // first k step of this wave
  const int srow = r0 + 16 * cj + l16;
  const bool sok = srow < dv;
  const int srow4 = r0 + 16 * cj + 4 * lg;
  const bool sok4 = srow4 < dv;  // dv % 4 == 0: all four rows or none

  if (tid == 0) sm.sync = 0, sm.csync = 0, sm.ysync[0] = sm.ysync[1] = sm.ysync[2] = sm.ysync[3] = 0;
  __syncthreads();  // the counter is zero before any wave arrives
  // the head waves carry the chain of dependent per-head steps: their
  // instructions go first when both roles compete for a SIMD or the memory
  // pipeline
  if (head) __builtin_amdgcn_s_setprio(3);

  // ---- 0. loads.  Head waves: Q/K (staged in LDS), parents, g, beta (and the
  // previous record's masks and G).  State waves: the state rows and V.
  constexpr int qk_cpr = kMaxDim / 8;  // 16-byte chunks per staged row
  constexpr int qk_total = 2 * Np * qk_cpr;
  constexpr int QKB = qk_total / 256;  // chunks per head thread
  static_assert(qk_total % 256 == 0, "every head thread stages QKB chunks");
  f32x4 Sraw[KSL][2];  // this wave's state columns 32 (kbase + i) + 8 lg .. + 7 of its row
  bf16_t vreg[NQT][4];
  int dn_s = 0;  // state waves: length of the previous draft's accepted path
  // Delayed commit (state waves): the previous draft's accepted path applied
  // to this wave's rows in the commit kernel's operation order (scale by
  // e^{G_last}, then one fmaf per path node in path order).  Each state wave
  // finds the path itself from the last accepted node's ancestor mask and the
  // path's G, and requests the path's k rows (its share of them, staged in
  // LDS for all state waves) and u' of its own rows before its state rows,
  // so that they arrive first.
  const int sw = wave >= 4 ? wave - 4 : 0;
  // Two schedules.  With four state waves (a grid that fills the GPU, whose
  // memory system accepts the state rows only as fast as it drains them) the
  // path's operands are requested ahead of the state rows and the commit is
  // applied block by block inside the contraction, as the rows arrive.  With
  // fewer (an idle memory system, the state rows arriving at once) they are
  // requested after the state rows and the whole commit is applied while the
  // head waves still wait for Q and K.
  constexpr bool kBlockCommit = SW == 4;
  constexpr int KQ = kWsChunk * (kMaxDim / 8) / (64 * NSW);  // 16-byte k chunks per lane
  u32x4 kq[DLY ? KQ : 1];
  float upr[kWsChunk / 4];  // u' of path node 4 m + lg for this lane's state row
  float s0c = 1.f;          // e^{G_last}
  auto path_fetch = [&](int last_v, uint64_t pmask_l, float pG_l) -> int {
    int* const dnode = sm.dnode[DLY ? sw : 0];
    float* const dc = sm.dc[DLY ? sw : 0];
    const int lst = __builtin_amdgcn_readfirstlane(last_v);
    const bool in_rng = lst >= 0 && lst < Npv;
    const int lc = in_rng ? lst : 0;
    const uint64_t valid = Npv >= 64 ? ~0ull : ((1ull << Npv) - 1ull);
    const uint32_t mlo = __builtin_amdgcn_readlane((uint32_t)pmask_l, lc);
    const uint32_t mhi = __builtin_amdgcn_readlane((uint32_t)(pmask_l >> 32), lc);
    const uint64_t pm = in_rng ? ((((uint64_t)mhi << 32) | mlo) & valid) : 0ull;
    const bool okp = in_rng && ((pm >> lst) & 1ull);
    const float Glast =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pG_l), lc));
    if (okp && ((pm >> lane) & 1ull)) {  // lane = node of the previous draft
      const int pos = __popcll(pm & ((1ull << lane) - 1ull));
      dnode[pos] = lane;
      dc[pos] = expf(Glast - pG_l);  // the commit kernel's coefficient
    }
    s0c = expf(Glast);
    const int dn = okp ? __popcll(pm) : 0;
    // (one wave's LDS operations complete in order: the reads below see the
    // path just written).  No branch around the loads: clamped addresses.
    const int lastp = dn > 0 ? dn - 1 : 0;
#pragma unroll
    for (int x = 0; x < KQ; ++x) {
      const int idx = 64 * KQ * sw + lane + 64 * x;
      const int c8 = clampi(8 * (idx % (kMaxDim / 8)), dk - 8);
      const int nd = dn > 0 ? dnode[clampi(idx / (kMaxDim / 8), lastp)] : 0;
      kq[x] = *reinterpret_cast<const u32x4*>(prev.K + ((size_t)bh * Npv + nd) * dk + c8);
    }
#pragma unroll
    for (int m = 0; m < kWsChunk / 4; ++m) {
      const int nd = dn > 0 ? dnode[clampi(4 * m + lg, lastp)] : 0;
      upr[m] = prev.up[((size_t)bh * Npv + nd) * dv + clampi(srow, dv - 1)];
    }
    return dn;
  };
  // this wave's share of the k rows into LDS (after the state rows were
  // requested), announced to the other state waves
  auto stage_k = [&](int dn) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int x = 0; x < KQ; ++x) {
      const int idx = 64 * KQ * sw + lane + 64 * x;
      const int j = idx / (kMaxDim / 8), c8 = 8 * (idx % (kMaxDim / 8));
      *reinterpret_cast<u32x4*>(sm.ck + j * kCkStride + c8) = (j < dn && c8 < dk) ? kq[x] : z;
    }
    ws_arrive(&sm.csync);
  };
  // The update on FP32 MFMA, four path nodes per product.  For the tile
  // (ks, half), D row 4 g + r is state column 32 ks + 8 g + 4 half + r and D
  // column j is state row 16 cj + j, so a lane's accumulator is its own
  // Sraw[ks][half]; the A operand, lane (row l16, k = lg), holds k of path
  // node 4 m + lg at that row's column, the B operand c u' of that node for
  // the lane's state row.  v_mfma_f32_16x16x4_f32 adds its four products one
  // after another, each as a fused multiply-add in k order, so node by node
  // in path order this is bitwise the commit kernel's fmaf sequence.  Past
  // the path the operands are 0 and -0, whose product leaves every
  // accumulator bit unchanged (x + -0 = x).
  const int kcol = 8 * (l16 >> 2) + (l16 & 3);
  // Paths of at most kWsChunk nodes (the usual case): the 32-column blocks
  // ks are committed one by one inside the contraction, each issued one
  // block ahead of the contraction products that take it, so the commit
  // overlaps the arrival of the state rows as the contraction does and its
  // products are complete when the block is written back and split.
  auto commit_ks = [&](int ks, int ng, const float (&cuv)[kWsChunk / 4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Sraw[ks][0][e] = Sraw[ks][0][e] * s0c;
      Sraw[ks][1][e] = Sraw[ks][1][e] * s0c;
    }
#pragma unroll
    for (int m = 0; m < kWsChunk / 4; ++m) {
      if (m < ng) {  // uniform
        const bf16_t* kr0 = sm.ck + (4 * m + lg) * kCkStride + 32 * (kbase + ks) + kcol;
        Sraw[ks][0] = mfma16x16x4f32(widen1(kr0[0]), cuv[m], Sraw[ks][0]);
        Sraw[ks][1] = mfma16x16x4f32(widen1(kr0[4]), cuv[m], Sraw[ks][1]);
      }
    }
  };
  // Longer paths, and drafts that failed validation: every operand read from
  // global memory, four path nodes at a time, the whole commit done before
  // the contraction (it consumes every state register before the first
  // write-back store, so no later wait on a load also waits for the stores).
  auto commit_global = [&](int dn) {
    const int* const dnode = sm.dnode[DLY ? sw : 0];
    const float* const dc = sm.dc[DLY ? sw : 0];
#pragma unroll
    for (int ks = 0; ks < KSL; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Sraw[ks][0][e] = Sraw[ks][0][e] * s0c;
        Sraw[ks][1][e] = Sraw[ks][1][e] * s0c;
      }
    for (int g0 = 0; g0 < dn; g0 += 4) {  // uniform
      const int jn = g0 + lg;
      const bool on = jn < dn;
      const int jc = clampi(jn, dn - 1);
      const int nd = dnode[jc];
      const float c = dc[jc] * prev.up[((size_t)bh * Npv + nd) * dv + clampi(srow, dv - 1)];
      const float cuv = on ? c : -0.0f;
      const bf16_t* kr0 = prev.K + ((size_t)bh * Npv + nd) * dk;
      float av[KSL][2];
#pragma unroll
      for (int ks = 0; ks < KSL; ++ks)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          av[ks][hf] = on ? widen1(kr0[clampi(32 * (kbase + ks) + 4 * hf + kcol, dk - 1)]) : 0.f;
#pragma unroll
      for (int ks = 0; ks < KSL; ++ks)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) Sraw[ks][hf] = mfma16x16x4f32(av[ks][hf], cuv, Sraw[ks][hf]);
    }
#pragma unroll
    for (int ks = 0; ks < KSL; ++ks) mfma_drain(Sraw[ks][0], Sraw[ks][1]);
  };
  // c u' of path node 4 m + lg for this lane's state row (the commit kernel's
  // product), -0 past the path
  auto make_cuv = [&](int dn, float (&cuv)[kWsChunk / 4]) {
    const float* const dc = sm.dc[DLY ? sw : 0];
#pragma unroll
    for (int m = 0; m < kWsChunk / 4; ++m) {
      const int j = 4 * m + lg;
      cuv[m] = j < dn ? dc[clampi(j, dn - 1)] * upr[m] : -0.0f;
    }
  };
  // the whole commit at once
  auto commit_all = [&](int dn) {
    if (dn > kWsChunk) {  // uniform
      commit_global(dn);
    } else {
      float cuv[kWsChunk / 4];
      make_cuv(dn, cuv);
      ws_wait(&sm.csync, NSW);  // every state wave's share of the k rows is in LDS
#pragma unroll
      for (int ks = 0; ks < KSL; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Sraw[ks][0][e] = Sraw[ks][0][e] * s0c;
          Sraw[ks][1][e] = Sraw[ks][1][e] * s0c;
        }
      // node group by node group: the group's operands read at once, then
      // 2 KS independent products
#pragma unroll
      for (int m = 0; m < kWsChunk / 4; ++m) {
        if (4 * m < dn) {  // uniform
          const bf16_t* kr0 = sm.ck + (4 * m + lg) * kCkStride + 32 * kbase + kcol;
          float av[KSL][2];
#pragma unroll
          for (int ks = 0; ks < KSL; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) av[ks][hf] = widen1(kr0[32 * ks + 4 * hf]);
#pragma unroll
          for (int ks = 0; ks < KSL; ++ks)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) Sraw[ks][hf] = mfma16x16x4f32(av[ks][hf], cuv[m], Sraw[ks][hf]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < KSL; ++ks) mfma_drain(Sraw[ks][0], Sraw[ks][1]);
    }
  };

  if (head) {
    // The topology's inputs first: wave 0 builds the topology while Q and K
    // are still in flight (loads complete in order, so inputs requested after
    // Q and K would wait for all of them).
    const int tn = clampi(lane, N - 1);
    const int pl = parents[(size_t)b * N + tn];
    const float gl = g[((size_t)b * N + tn) * H + h];
    const float bl = beta[((size_t)b * N + tn) * H + h];
    int last_v = -1;
    uint64_t pmask_l = 0;
    if (DLY && tile == 0 && h == 0 && commit_status) {
      last_v = last_acc[b];
      pmask_l = prev.mask[(size_t)b * Npv + clampi(lane, Npv - 1)];
    }
    u32x4 qkw[QKB];
#pragma unroll
    for (int x = 0; x < QKB; ++x) {
      const int idx = tid + 256 * x;
      const int r = idx / qk_cpr;
      const bool isq = r < Np;
      const int t = clampi(isq ? r : r - Np, N - 1);
      const int c8 = clampi(8 * (idx % qk_cpr), dk - 8);
      qkw[x] = *reinterpret_cast<const u32x4*>((isq ? q : k) + (((size_t)b * N + t) * H + h) * dk + c8);
    }
    // the head's loads are queued: the state waves may now request theirs
    ws_arrive(&sm.sync);
    // (while the loads are in flight) T and A start as zeros: the Gram tiles write only A's lower-triangle
    // blocks, and the path solves multiply the entries above the diagonal by
    // exact zeros, which needs them finite
    for (int idx = tid; idx < kMatFloats / 4; idx += 256) {
      reinterpret_cast<f32x4*>(Tl)[idx] = f32x4{0.f, 0.f, 0.f, 0.f};
      reinterpret_cast<f32x4*>(KK)[idx] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // 1. wave 0: parents -> validation, ancestor-or-self masks and G (its
    // global stores follow the staging, which would otherwise wait for them)
    uint64_t m = 0ull;
    float G = 0.f;
    bool anybad = false;
    if (wave == 0) {
      const int t = lane;
      const int p = t < N ? pl : -1;
      const bool bad = t < N && (p < -1 || p >= t);
      anybad = __ballot(bad) != 0ull;
      m = t < N ? (1ull << t) : 0ull;
      G = t < N ? gl : 0.f;
      int a = (t < N && !bad) ? p : -1;
      for (int r = 0; r < 6; ++r) {  // 2^6 = 64 >= path length
        if (__ballot(a >= 0) == 0ull) break;  // uniform: every path is complete
        const int src = a >= 0 ? a : t;
        const uint64_t ma = __shfl(m, src);
        const float Ga = __shfl(G, src);
        const int aa = __shfl(a, src);
        if (a >= 0) {
          m |= ma;
          G += Ga;
          a = aa;
        }
      }
      if (anybad) m = 0ull;
      sm.mask[t] = m;
      sm.G[t] = G;
      sm.eG[t] = expf(G);
      sm.beta[t] = t < N ? bl : 0.f;
      if (t == 0) sm.bad = anybad;
    }
#pragma unroll
    for (int x = 0; x < QKB; ++x) {  // no branch: a load under one is waited for at once
      const int idx = tid + 256 * x;
      const int r = idx / qk_cpr;
      const int t = r < Np ? r : r - Np;
      const int c8 = 8 * (idx % qk_cpr);
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(QKs + r * kQKStride + c8) = (t < N && c8 < dk) ? qkw[x] : z;
    }
    if (wave == 0) {
      const int t = lane;
      if (tile == 0 && t < N) {
        rec.G[(size_t)bh * N + t] = anybad ? 0.f : G;
        if (h == 0) {
          rec.parents[(size_t)b * N + t] = pl;
          rec.mask[(size_t)b * N + t] = m;
          if (mask_out) mask_out[(size_t)b * N + t] = m;
        }
      }
      if (tile == 0 && t == 0 && h == 0 && dev_status)
        dev_status[b] = anybad ? GDN_ERR_TOPOLOGY : GDN_OK;
      if (DLY && tile == 0 && h == 0 && commit_status) {  // the previous draft's last accepted node
        const int lst = __builtin_amdgcn_readfirstlane(last_v);
        const bool in_rng = lst >= 0 && lst < Npv;
        const uint32_t mlo = __builtin_amdgcn_readlane((uint32_t)pmask_l, in_rng ? lst : 0);
        const uint32_t mhi = __builtin_amdgcn_readlane((uint32_t)(pmask_l >> 32), in_rng ? lst : 0);
        const bool okp = in_rng && ((((((uint64_t)mhi << 32) | mlo)) >> lst) & 1ull);
        if (t == 0) commit_status[b] = (lst == -1 || okp) ? GDN_OK : GDN_ERR_TOPOLOGY;
      }
    }
  } else {
    // The head waves' Q and K requests go first (the state's would otherwise
    // fill the memory queues ahead of them and delay every per-head step).
    // the previous draft's last accepted node, the masks and G (the path),
    // then the path's operands (ahead of the state rows for the block-wise
    // commit, after them otherwise)
    int last_v = -1;
    uint64_t pmask_l = 0;
    float pG_l = 0.f;
    if (DLY) {
      const int tj = clampi(lane, Npv - 1);
      last_v = last_acc[b];
      pmask_l = prev.mask[(size_t)b * Npv + tj];
      pG_l = prev.G[(size_t)bh * Npv + tj];
    }
    if (DLY && kBlockCommit) dn_s = path_fetch(last_v, pmask_l, pG_l);
    ws_wait(&sm.sync, 4);
    // The state is read and written once per step: non-temporal accesses
    // stream it past the caches, which keep Q, K (read by the head's four
    // tiles) and leave less to write back when the kernel ends.
    const float* sptr = S0 + ((size_t)bh * dv + clampi(srow, dv - 1)) * dk;
#pragma unroll
    for (int ks = 0; ks < KSL; ++ks) {
      const int kk = clampi(32 * (kbase + ks) + koff, dk - 8);
      Sraw[ks][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sptr + kk));
      Sraw[ks][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sptr + kk + 4));
    }
#pragma unroll
    for (int j = 0; j < NQT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = clampi(16 * j + 4 * lg + r, N - 1);
        vreg[j][r] = v[(((size_t)b * N + t) * H + h) * dv + clampi(srow, dv - 1)];
      }
    if (DLY && !kBlockCommit) dn_s = path_fetch(last_v, pmask_l, pG_l);
    if (DLY && dn_s > 0 && dn_s <= kWsChunk) stage_k(dn_s);  // uniform
    if (DLY && !kBlockCommit && dn_s > 0) commit_all(dn_s);  // uniform
  }
  if (head)
    ws_sync(&sm.sync, 8);  // staged Q/K, T zeroed, topology, path
  else
    ws_wait(&sm.sync, 8);
  // With a delayed commit the state waves carry the longer chain from here
  // (commit, write-back and contraction against the head's Gram and solve):
  // their instructions now go first.
  if (DLY) {
    if (head)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(2);
  }

  // write-back of the committed columns 32 ks + 8 lg .. + 7 of this lane's row
  auto dly_store = [&](int ks) {
    const int col = 32 * (kbase + ks) + koff;
    if (sok && col < dk) {
      float* wp = S0 + ((size_t)bh * dv + srow) * dk + col;
      __builtin_nontemporal_store(Sraw[ks][0], reinterpret_cast<f32x4*>(wp));
      __builtin_nontemporal_store(Sraw[ks][1], reinterpret_cast<f32x4*>(wp + 4));
    }
  };

  // gated form (gdn_layer_verify): Y = bf16(O * SiLU(gate)) for node t and the
  // four state rows srow4 .. srow4 + 3, with gdn_gate_merge's arithmetic
  auto store_gated_s = [&](size_t o, const f32x4& x, const f32x4& sg) {
    u32x2 w;
    w.x = (uint32_t)to_bf16(x.x * sg.x) | ((uint32_t)to_bf16(x.y * sg.y) << 16);
    w.y = (uint32_t)to_bf16(x.z * sg.z) | ((uint32_t)to_bf16(x.w * sg.w) << 16);
    *reinterpret_cast<u32x2*>(ga.Y + o) = w;
  };
  auto store_gated = [&](int t, size_t o, const f32x4& x) {
    const float* gp = ga.gate + ((size_t)b * N + t) * ga.ldg + h * dv + srow4;
    u32x2 w;
    w.x = (uint32_t)to_bf16(x.x * silu(gp[0])) | ((uint32_t)to_bf16(x.y * silu(gp[1])) << 16);
    w.y = (uint32_t)to_bf16(x.z * silu(gp[2])) | ((uint32_t)to_bf16(x.w * silu(gp[3])) << 16);
    *reinterpret_cast<u32x2*>(ga.Y + o) = w;
  };

  if (sm.bad) {  // uniform: zero this tile's outputs (a delayed commit still applies)
    if (!head) {
      if (DLY && dn_s > 0) {  // uniform
        if (kBlockCommit) commit_global(dn_s);
#pragma unroll
        for (int ks = 0; ks < KSL; ++ks) dly_store(ks);
      }
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      for (int t0 = 0; t0 < N && kbase == 0; t0 += 16) {  // one wave per row
        const int t = t0 + l16;
        if (t < N && sok4) {
          const size_t o = (((size_t)b * N + t) * H + h) * dv + srow4;
          if constexpr (GATE)  // the gated form writes the gated zeros bf16(0 * SiLU(gate))
            store_gated(t, o, z);
          else
            *reinterpret_cast<f32x4*>(out + o) = z;
          *reinterpret_cast<f32x4*>(rec.up + ((size_t)bh * N + t) * dv + srow4) = z;
        }
      }
    }
    return;
  }
  // every wave reads the depths, so the choice of solve is uniform
  const bool deep =
      __ballot(lane < N && __popcll(sm.mask[lane < N ? lane : 0]) > kPathMax) != 0ull;

  if (head) {
    if (tile == 0) {  // factor record: this head's k rows (the staged bits)
      constexpr int kC8 = kMaxDim / 8;
      constexpr int RKC = Np * kC8 / 256;
      u32x4 kc[RKC];
#pragma unroll
      for (int x = 0; x < RKC; ++x) {
        const int idx = tid + 256 * x;
        kc[x] = *reinterpret_cast<const u32x4*>(QKs + (Np + idx / kC8) * kQKStride + 8 * (idx % kC8));
      }
#pragma unroll
      for (int x = 0; x < RKC; ++x) {
        const int idx = tid + 256 * x;
        const int t = idx / kC8;
        const int c8 = 8 * (idx % kC8);
        if (t < N && c8 < dk)
          __builtin_nontemporal_store(kc[x], reinterpret_cast<u32x4*>(rec.K + ((size_t)bh * N + t) * dk + c8));
      }
    }
    // 2-3. Gram blocks Q K^T and K K^T, lower-triangle tiles: wave w takes
    // row block pair w / 2 of Q (w even) or of K (w odd), as in
    // tree_verify.hip (with two row blocks, one row block per wave, so all
    // four waves take part); each tile is masked, decayed and scaled in registers
    // into A (FP32) or Attn (split bf16), so no N x N pass follows.  Only the
    // lower-triangle blocks are ever read.
    auto gram_job = [&](auto wc) {
      constexpr int Wc = decltype(wc)::value;
      constexpr int npairs = NQT > 2 ? (NQT + 1) / 2 : NQT;
      if constexpr (Wc < 2 * npairs) {
        constexpr bool isq = Wc % 2 == 0;
        constexpr int ra = NQT - 1 - Wc / 2;
        constexpr int rs = Wc / 2;
        constexpr bool two = NQT > 2 && rs < ra;
        const bf16_t* rows = QKs + (isq ? 0 : Np) * kQKStride;
        bf16x8 fa[KS], fs[two ? KS : 1], kb[2][KS];
        // per-row values of this lane's four rows 4 lg + r of each row block
        uint64_t mra[4], mrs[4];
        float gra[4], grs[4], bra[4], brs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ta = 16 * ra + 4 * lg + r, ts = 16 * rs + 4 * lg + r;
          mra[r] = sm.mask[ta];
          gra[r] = sm.G[ta];
          bra[r] = sm.beta[ta];
          mrs[r] = sm.mask[ts];
          grs[r] = sm.G[ts];
          brs[r] = sm.beta[ts];
        }
        // the tile's entries of A (K K^T: beta_t e^{G_t - G_j} (k_t . k_j) for
        // j a proper ancestor of t) or of Attn (Q K^T: scale e^{G_t - G_j}
        // (q_t . k_j) for j on t's root path), exact zeros elsewhere
        auto put = [&](int rblk, int ct, const f32x4& acc, const uint64_t (&m)[4],
                       const float (&gr)[4], const float (&br)[4]) {
          const int j = 16 * ct + l16;
          const float gj = sm.G[j];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * rblk + 4 * lg + r;
            const bool on = (m[r] >> j) & 1ull;
            const float dec = __expf(gr[r] - gj);
            if constexpr (isq)
              store_split1(Attn + t * kLdS + j, kSplitLoS, on ? scale * dec * acc[r] : 0.f);
            else
              KK[t * kLd + j] = (on && j != t) ? br[r] * dec * acc[r] : 0.f;
          }
        };
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          fa[ks] = lds_bf16x8(rows + (16 * ra + l16) * kQKStride + 32 * ks + koff);
          if constexpr (two) fs[ks] = lds_bf16x8(rows + (16 * rs + l16) * kQKStride + 32 * ks + koff);
        }
        auto kload = [&](int ct, bf16x8 (&dstf)[KS]) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            dstf[ks] = lds_bf16x8(QKs + (Np + 16 * ct + l16) * kQKStride + 32 * ks + koff);
        };
        if constexpr (!two && ra <= 1) {
          // one row block of at most two tiles: both column tiles at once,
          // two independent product chains that hide each other's latency
          constexpr bool pair = ra == 1;
          kload(0, kb[0]);
          if constexpr (pair) kload(1, kb[1]);
          f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            acc0 = mfma16x16x32(fa[ks], kb[0][ks], acc0);
            if constexpr (pair) acc1 = mfma16x16x32(fa[ks], kb[1][ks], acc1);
          }
          mfma_drain(acc0, acc1);
          put(ra, 0, acc0, mra, gra, bra);
          if constexpr (pair) put(ra, 1, acc1, mra, gra, bra);
          return;
        }
        kload(0, kb[0]);
#pragma unroll
        for (int ct = 0; ct <= ra; ++ct) {
          if (ct + 1 <= ra) kload(ct + 1, kb[(ct + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(fa[ks], kb[ct & 1][ks], acc);
          mfma_drain(acc);
          put(ra, ct, acc, mra, gra, bra);
          if (two && ct <= rs) {
            f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              acc2 = mfma16x16x32(fs[two ? ks : 0], kb[ct & 1][ks], acc2);
            mfma_drain(acc2);
            put(rs, ct, acc2, mrs, grs, brs);
          }
        }
      }
    };
    switch (__builtin_amdgcn_readfirstlane(wave)) {
      case 0: gram_job(std::integral_constant<int, 0>{}); break;
      case 1: gram_job(std::integral_constant<int, 1>{}); break;
      case 2: gram_job(std::integral_constant<int, 2>{}); break;
      default: gram_job(std::integral_constant<int, 3>{}); break;
    }
  }
  if (head) ws_sync(&sm.sync, 12);  // A and Attn

  if (head) {
    // rows of T on root paths, one lane per node (wave 0): split bf16, or FP32
    // diagonal blocks for a deep draft
    if (tid < N) {
      const int t = tid;
      const uint64_t m = sm.mask[t];
      const int d = __popcll(m);
      auto put_split = [&](int j, float x) { store_split1(Ts + t * kLdS + j, kSplitLoS, x); };
      auto put_f32 = [&](int j, float x) { Tl[t * kLd + j] = x; };
      if (deep) {
        const uint64_t mb = m & (0xFFFFull << (16 * (t / 16)));
        path_solve_registers(t, mb, __popcll(mb), KK, put_f32);
      } else if (__ballot(d > 8) == 0ull) {
        path_solve_block<8>(t, m, d, KK, put_split);
      } else if (__ballot(d > 12) == 0ull) {
        path_solve_block<12>(t, m, d, KK, put_split);
      } else {
        path_solve_registers(t, m, d, KK, put_split);
      }
    }
  }

  // state waves: contraction (with the committed rows written back), R
  f32x4 yacc[2 * NQT];
  f32x4 yacc2[2][kHalves ? 2 * NQT : 1];  // 16- and 32-row tiles: the sums over the later parts
  f32x4 rv[NQT];
  f32x4 gsl[GATE ? NQT : 1];  // gated form: SiLU(gate) of node 16 i + l16, rows srow4 .. + 3
  if (!head) {
#pragma unroll
    for (int i = 0; i < 2 * NQT; ++i) yacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < (kHalves ? 2 * NQT : 1); ++i) yacc2[0][i] = yacc2[1][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // 4. Y: the K row tiles as K S0^T (rows = nodes, as the B operand of
    // T R), the Q row tiles transposed as S0 Q^T (each lane then holds four
    // consecutive state rows of one node, as O^T needs).  The next k step's
    // A fragments are read while this one multiplies.
    bf16x8 afr[2][2 * NQT];
    auto aload = [&](int ks, bf16x8 (&a)[2 * NQT]) {
#pragma unroll
      for (int i = 0; i < 2 * NQT; ++i)
        a[i] = lds_bf16x8(QKs + (16 * i + l16) * kQKStride + 32 * (kbase + ks) + koff);
    };
    // With a delayed commit, the committed columns of each k step are written
    // back as the step is contracted: the memory system accepts the stores
    // only as fast as it drains them, and the matrix products of the previous
    // steps keep running meanwhile.
    const bool wb = DLY && dn_s > 0;                       // uniform
    const bool lcm = DLY && kBlockCommit && dn_s > 0 && dn_s <= kWsChunk;  // uniform: block by block
    float cuv[kWsChunk / 4] = {};
    const int ngc = (dn_s + 3) >> 2;
    if (DLY && kBlockCommit && dn_s > kWsChunk) commit_global(dn_s);
    if (lcm) {
      make_cuv(dn_s, cuv);
      ws_wait(&sm.csync, NSW);  // every state wave's share of the k rows is in LDS
    }
    // block ks of the (committed) rows: written back, then split into the
    // bf16 hi + lo operands of the contraction
    bf16x8 bhi[2], blo[2];
    auto prep = [&](int ks) {
      if (wb) dly_store(ks);
      const bool okk = sok && 32 * (kbase + ks) + koff < dk;
      split8(mask4(Sraw[ks][0], okk), mask4(Sraw[ks][1], okk), bhi[ks & 1], blo[ks & 1]);
    };
    if (lcm) {
      commit_ks(0, ngc, cuv);
      mfma_drain(Sraw[0][0], Sraw[0][1]);
    }
    prep(0);
    aload(0, afr[0]);
#pragma unroll
    for (int ks = 0; ks < KSL; ++ks) {  // zero-padded past dk: no branch
      if (ks + 1 < KSL) aload(ks + 1, afr[(ks + 1) & 1]);
      if (lcm && ks + 1 < KSL) commit_ks(ks + 1, ngc, cuv);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2 * NQT; ++i) {
        f32x4& acc = (kHalves && ks >= KPART) ? yacc2[kHalves ? ((ks / KPART - 1) & 1) : 0][kHalves ? i : 0] : yacc[i];
        if (i < NQT) {
          acc = mfma16x16x32(bhi[ks & 1], afr[ks & 1][i], acc);
          acc = mfma16x16x32(blo[ks & 1], afr[ks & 1][i], acc);
        } else {
          acc = mfma16x16x32(afr[ks & 1][i], bhi[ks & 1], acc);
          acc = mfma16x16x32(afr[ks & 1][i], blo[ks & 1], acc);
        }
      }
      if (kHalves && ks == 2 * KPART) {  // part 1 is complete: added first, its set reused by part 3
#pragma unroll
        for (int i = 0; i < 2 * NQT; ++i) {
#pragma unroll
          for (int r = 0; r < 4; ++r) yacc[i][r] += yacc2[0][i][r];
          yacc2[0][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      if (ks + 1 < KSL) {
        if (lcm) mfma_drain(Sraw[ks + 1][0], Sraw[ks + 1][1]);
        prep(ks + 1);
      }
    }
    mfma_drain_all(yacc);
    if constexpr (kHalves && kParts == 4) {  // parts 2 and 3, in order
      mfma_drain_all(yacc2[0]);
      mfma_drain_all(yacc2[1]);
#pragma unroll
      for (int i = 0; i < 2 * NQT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[i][r] = (yacc[i][r] + yacc2[1][i][r]) + yacc2[0][i][r];
    } else if constexpr (kHalves) {  // part 1
      mfma_drain_all(yacc2[0]);
#pragma unroll
      for (int i = 0; i < 2 * NQT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[i][r] += yacc2[0][i][r];
    }
    if constexpr (KSPLIT) {  // uniform: the other waves' parts of the sums go to the first, in order
      const int part = kbase / KSL;
      if (part != 0) {
#pragma unroll
        for (int i = 0; i < 2 * NQT; ++i) sm.yx[cj][part - 1][i][lane] = yacc[i];
        ws_arrive(&sm.ysync[cj]);
      } else {
        ws_wait(&sm.ysync[cj], kParts - 1);
#pragma unroll
        for (int p = 0; p < kParts - 1; ++p)
#pragma unroll
          for (int i = 0; i < 2 * NQT; ++i) {
            const f32x4 x = sm.yx[cj][p][i][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) yacc[i][r] += x[r];
          }
      }
    }
    // R = diag(beta) (V - diag(e^G) K S0^T): lane (row srow, lg) holds nodes
    // 16 nb + 4 lg + r
#pragma unroll
    for (int nb = 0; nb < NQT; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * nb + 4 * lg + r;
        const float vv = sok ? widen1(vreg[nb][r]) : 0.f;
        rv[nb][r] = sm.beta[t] * (vv - sm.eG[t] * yacc[NQT + nb][r]);
      }
    // gated form: the gate's SiLU for the epilogue's outputs, formed before
    // the barrier (the same operations as in the epilogue's product)
    if constexpr (GATE) {
#pragma unroll
      for (int i = 0; i < NQT; ++i) {
        const int t = clampi(16 * i + l16, N - 1);
        const float* gp = ga.gate + ((size_t)b * N + t) * ga.ldg + h * dv + clampi(srow4, dv - 4);
        gsl[i] = f32x4{silu(gp[0]), silu(gp[1]), silu(gp[2]), silu(gp[3])};
      }
    }
  }

  if (head && deep) {  // uniform: blocked forward substitution, as in tree_verify.hip
    int tgt = 12;
    ws_sync(&sm.sync, tgt += 4);  // the diagonal blocks are in T
#pragma unroll
    for (int i = 1; i < NQT; ++i) {
      const int j = wave;
      float* blk = Tl + (16 * i) * kLd + 16 * j;
      if (j < i) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        for (int kb = j; kb < i; ++kb)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            x = mfma16x16x4f32(KK[(16 * i + l16) * kLd + 16 * kb + 4 * c + lg],
                               Tl[(16 * kb + 4 * c + lg) * kLd + 16 * j + l16], x);
        mfma_drain(x);
#pragma unroll
        for (int r = 0; r < 4; ++r) blk[(4 * lg + r) * kLd + l16] = x[r];
      }
      ws_sync(&sm.sync, tgt += 4);
      if (j < i) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          y = mfma16x16x4f32(Tl[(16 * i + l16) * kLd + 16 * i + 4 * c + lg],
                             blk[(4 * c + lg) * kLd + l16], y);
        mfma_drain(y);
#pragma unroll
        for (int r = 0; r < 4; ++r) blk[(4 * lg + r) * kLd + l16] = -y[r];
      }
      ws_sync(&sm.sync, tgt += 4);  // block row i is complete before row i + 1 reads it
    }
  }
  __syncthreads();  // T and Attn are complete; the only barrier of both roles after the start
  if (head || kbase != 0) return;  // (split tiles: each group's first state wave finishes it)

  // ---- 5. epilogue (state waves): U' = T R, its transpose for the record,
  // O^T = (Attn U')^T + scale e^G (S0 Q^T); T and Attn are lower triangular,
  // so block row i sums over k blocks 0..i
  auto run = [&](auto deep_c) {
    constexpr bool kDeep = decltype(deep_c)::value;
    constexpr int NPAIR = NQT * (NQT + 1) / 2;
    s16x4 th[NPAIR], tl[NPAIR];
#pragma unroll
    for (int i = 0, x = 0; i < NQT; ++i)
#pragma unroll
      for (int kb = 0; kb <= i; ++kb, ++x) {
        const int row = 16 * i + l16, col = 16 * kb + 4 * lg;
        if constexpr (kDeep) {
          split4(*reinterpret_cast<const f32x4*>(Tl + row * kLd + col), th[x], tl[x]);
        } else {
          th[x] = __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(Ts + row * kLdS + col));
          tl[x] = __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(Ts + kSplitLoS + row * kLdS + col));
        }
      }
    s16x4 rh[NQT], rl[NQT];
#pragma unroll
    for (int kb = 0; kb < NQT; ++kb) split4(rv[kb], rh[kb], rl[kb]);
    f32x4 ua[NQT], ut[NQT];
#pragma unroll
    for (int i = 0, x = 0; i < NQT; ++i) {
      ua[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      ut[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= i; ++kb, ++x) {
        ua[i] = mfma16x16x16(th[x], rh[kb], ua[i]);
        ua[i] = mfma16x16x16(th[x], rl[kb], ua[i]);
        ua[i] = mfma16x16x16(tl[x], rh[kb], ua[i]);
        ut[i] = mfma16x16x16(rh[kb], th[x], ut[i]);
        ut[i] = mfma16x16x16(rl[kb], th[x], ut[i]);
        ut[i] = mfma16x16x16(rh[kb], tl[x], ut[i]);
      }
    }
    s16x4 ah[NPAIR], al[NPAIR];  // Attn fragments, read while U' multiplies
#pragma unroll
    for (int i = 0, x = 0; i < NQT; ++i)
#pragma unroll
      for (int kb = 0; kb <= i; ++kb, ++x) {
        const int o = (16 * i + l16) * kLdS + 16 * kb + 4 * lg;
        ah[x] = __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(Attn + o));
        al[x] = __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(Attn + kSplitLoS + o));
      }
    mfma_drain_all(ua);
    s16x4 uh[NQT], ul[NQT];
#pragma unroll
    for (int kb = 0; kb < NQT; ++kb) split4(ua[kb], uh[kb], ul[kb]);
    f32x4 ot[NQT];
#pragma unroll
    for (int i = 0, x = 0; i < NQT; ++i) {
      const float se = scale * sm.eG[16 * i + l16];
#pragma unroll
      for (int r = 0; r < 4; ++r) ot[i][r] = se * yacc[i][r];
#pragma unroll
      for (int kb = 0; kb <= i; ++kb, ++x) {
        ot[i] = mfma16x16x16(uh[kb], ah[x], ot[i]);
        ot[i] = mfma16x16x16(ul[kb], ah[x], ot[i]);
        ot[i] = mfma16x16x16(uh[kb], al[x], ot[i]);
      }
    }
    mfma_drain_all(ut);
#pragma unroll
    for (int i = 0; i < NQT; ++i) {
      const int t = 16 * i + l16;
      if (t < N && sok4)
        __builtin_nontemporal_store(ut[i], reinterpret_cast<f32x4*>(rec.up + ((size_t)bh * N + t) * dv + srow4));
    }
    mfma_drain_all(ot);
#pragma unroll
    for (int i = 0; i < NQT; ++i) {
      const int t = 16 * i + l16;
      if (t < N && sok4) {
        const size_t o = (((size_t)b * N + t) * H + h) * dv + srow4;
        if constexpr (GATE)
          store_gated_s(o, ot[i], gsl[i]);
        else
          __builtin_nontemporal_store(ot[i], reinterpret_cast<f32x4*>(out + o));
      }
    }
  };
  if (deep)
    run(std::integral_constant<bool, true>{});
  else
    run(std::integral_constant<bool, false>{});
}

template <int NQT, int SW, bool GATE>
hipError_t launch_ws_g(int B, int N, int H, int dk, int dv, float* S0, const int32_t* parents,
                       const bf16_t* q, const bf16_t* k, const bf16_t* v, const float* beta,
                       const float* g, float scale, float* out, const Record<bf16_t>& rec,
                       uint64_t* mask_out, int32_t* dev_status, const void* prev_factors,
                       int Npv, const int32_t* last, int32_t* commit_status, GateArgs ga,
                       hipStream_t stream) {
  const int ntiles = (dv + 16 * SW - 1) / (16 * SW);
  const long grid = (long)B * H * ntiles;
  if (prev_factors) {
    const dim3 block(256 + 64 * ws_state_waves<SW, true>());
    const RecordLayout Lp = record_layout(B, Npv, H, dk, dv, GDN_BF16);
    const Record<bf16_t> prev = record_views<bf16_t>(const_cast<void*>(prev_factors), Lp);
    hipLaunchKernelGGL((tree_ws_kernel<NQT, true, SW, GATE>), dim3((unsigned)grid), block, 0,
                       stream, N, H, dk, dv, ntiles, S0, parents, q, k, v, beta, g, scale, out,
                       rec, mask_out, dev_status, prev, Npv, last, commit_status, ga);
  } else {
    const dim3 block(256 + 64 * ws_state_waves<SW, false>());
    hipLaunchKernelGGL((tree_ws_kernel<NQT, false, SW, GATE>), dim3((unsigned)grid), block, 0,
                       stream, N, H, dk, dv, ntiles, S0, parents, q, k, v, beta, g, scale, out,
                       rec, mask_out, dev_status, Record<bf16_t>{}, 1, nullptr, nullptr, ga);
  }
  return hipGetLastError();
}

template <int NQT>
hipError_t launch_ws_n(int SW, int B, int N, int H, int dk, int dv, float* S0,
                       const int32_t* parents, const bf16_t* q, const bf16_t* k, const bf16_t* v,
                       const float* beta, const float* g, float scale, float* out,
                       const Record<bf16_t>& rec, uint64_t* mask_out, int32_t* dev_status,
                       const void* prev_factors, int Npv, const int32_t* last,
                       int32_t* commit_status, GateArgs ga, hipStream_t stream) {
#define GDN_WS(SWV, G)                                                                        \
  return launch_ws_g<NQT, SWV, G>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out,  \
                                  rec, mask_out, dev_status, prev_factors, Npv, last,          \
                                  commit_status, ga, stream)
  if (ga.gate) {
    if (SW == 1) GDN_WS(1, true);
    if (SW == 2) GDN_WS(2, true);
    GDN_WS(4, true);
  }
  if (SW == 1) GDN_WS(1, false);
  if (SW == 2) GDN_WS(2, false);
  GDN_WS(4, false);
#undef GDN_WS
}

// The split-role form with bf16 inputs, SW state waves of 16 rows each (the
// caller has chosen the tile width 16 SW and checked every size).
hipError_t launch_tree_ws(int SW, int B, int N, int H, int dk, int dv, float* S0,
                          const int32_t* parents, const bf16_t* q, const bf16_t* k,
                          const bf16_t* v, const float* beta, const float* g, float scale,
                          float* out, const Record<bf16_t>& rec, uint64_t* mask_out,
                          int32_t* dev_status, const void* prev_factors, int Npv,
                          const int32_t* last, int32_t* commit_status, GateArgs ga,
                          hipStream_t stream) {
  switch ((N + 15) / 16) {
    case 1:
      return launch_ws_n<1>(SW, B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                            mask_out, dev_status, prev_factors, Npv, last, commit_status, ga,
                            stream);
    case 2:
      return launch_ws_n<2>(SW, B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                            mask_out, dev_status, prev_factors, Npv, last, commit_status, ga,
                            stream);
    case 3:
      return launch_ws_n<3>(SW, B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                            mask_out, dev_status, prev_factors, Npv, last, commit_status, ga,
                            stream);
    default:
      return launch_ws_n<4>(SW, B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                            mask_out, dev_status, prev_factors, Npv, last, commit_status, ga,
                            stream);
  }
}

}  // namespace gdn
