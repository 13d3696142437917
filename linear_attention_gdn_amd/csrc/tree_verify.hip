// Tree-masked factorized verification (gfx950).
//
// SpecLA review, "Core claim" and "What carries the argument" (paper
// Section 4.2): the draft-tree topology is inserted into the delta-rule UT
// factorization as a mask, so every node's output comes from the committed
// state S0 in one pass while updates flow only along ancestor paths.  With
// M the ancestor mask, G_t the path-cumulative log decay, and the pages'
// garbled symbols read as
//     A[t,j]    = beta_t e^{G_t - G_j} (k_t . k_j)      j strict ancestor of t
//     T         = (I + A)^{-1}                          (the "solve_tril" step)
//     Attn[t,j] = e^{G_t - G_j} (q_t . k_j)             j ancestor-or-self of t
// the outputs are
//     U' = T (diag(beta) V - diag(beta e^G) K S0^T)     (factor record)
//     O  = scale (diag(e^G) Q S0^T + Attn U')
// i.e. O = bQ S0^T - Attn (W S0^T) + Attn U with W = T diag(beta e^G) K,
// U = T diag(beta) V, bQ = diag(e^G) Q.  Reassociating
// W S0^T = T diag(beta e^G) (K S0^T) keeps the large contraction on the raw
// bf16 keys instead of an FP32 matrix W.
//
// One kernel, one workgroup (4 waves) per (sequence, head, tile of BV state
// rows).  It serves FP32 q/k/v at every tile width, and bf16 q/k/v when even
// 16-row tiles would give fewer than 128 workgroups (8-row tiles); every
// other bf16 launch takes the split-role kernel of tree_verify_ws.hip, which
// computes the same quantities.  Each workgroup:
//   0. issues one round of loads: Q and K of its head (staged in LDS as bf16,
//      rows padded against bank conflicts), parents / g / beta, and last its
//      S0 tile (straight into MFMA B-fragment registers) and V tile.  Loads
//      complete in issue order, so the staging and step 1 wait only for what
//      precedes them while the state streams in behind steps 1-3;
//   1. validates the parents and builds ancestor bitmasks and the
//      path-cumulative G by pointer jumping (one lane per node, stopping when
//      every path is complete);
//   2. forms the Gram blocks Q K^T and K K^T on bf16 MFMA (lower triangle;
//      each wave owns a pair of row blocks of Q or of K, reads their
//      fragments once and each K column block once for both rows, the next
//      column block's fragments read while the current one multiplies);
//   3. masks and scales them into A and Attn (all threads, only the N x N
//      block the products read, every operand read before any is used), then
//      solves row t of T on t's root path (rows of T vanish off the path), one
//      lane per node with the path's block of A in registers, writing T
//      already split into bf16 hi + lo for step 5.  A draft with a root path
//      deeper than 16 is solved by blocks instead: each lane solves its row
//      of its 16-node diagonal block, then block rows of T follow by blocked
//      forward substitution on FP32 MFMA (T in FP32, split in step 5);
//   4. runs the dense contraction Y = [Q; K] S0_tile^T on bf16 MFMA with the
//      FP32 state split into bf16 hi + lo (bf16 q, k make every product
//      exact; only the 2^-16 split residue is lost);
//   5. forms R = beta (V - e^G Y_k) from the accumulators, then U' = T R and
//      O = scale e^G Y_q + Attn U' as two dense MFMA products.  Their FP32
//      operands are stored in LDS already split into bf16 hi + lo and summed
//      in three passes (hi*hi, hi*lo, lo*hi).  Masked-out entries are exact
//      zeros, so non-ancestors never contribute.
// The per-head steps 1-3 are repeated by each of the head's tiles; they run
// while the state tile is still in flight.  Workgroups are numbered so that
// the tiles of one head run on the same XCD and share its L2 for Q and K.
//
// Delayed commit (review: Referee Report summary, mechanism (ii); Figure 7
// caption, right side): with DLY the kernel also applies the previous draft's
// accepted path to its register-resident state tile before step 4.  The
// path (from the previous record's masks) is known after step 1; its k rows,
// u' of the tile's rows and coefficients e^{G_last - G_i} are loaded then and
// staged in LDS (16 path nodes at a time) while steps 2-3 run, then applied
// in the commit kernel's operation order (so the committed state is bitwise
// gdn_commit_path's) and the tile is written back once.  With tiles of at most
// 16 rows the four waves split the tile's columns for this and exchange the
// committed quarters through LDS.
//
// GATE variants (gdn_layer_verify) multiply the outputs by SiLU of the
// layer's gate in the epilogue and store them as bf16.
#include <type_traits>

#include "tree_common.h"

namespace gdn {

template <int BV>
struct TreeLds {
  static constexpr int kBVT = ((BV + 15) / 16) * 16;            // padded tile width
  static constexpr int kMat = kMatFloats * 4;                    // one N x N matrix region
  static constexpr int kSplitT = kBVT * kLdH * 2 * 2;            // R^T or U'^T, hi + lo
  static constexpr int kRegionA = kQKBytes > 2 * kSplitT ? kQKBytes : 2 * kSplitT;
  static constexpr int kOffKK = kRegionA;        // K K^T -> A (FP32)
  static constexpr int kOffQK = kOffKK + kMat;   // Q K^T -> Attn (bf16 hi + lo)
  static constexpr int kOffT = kOffQK + kMat;    // T (FP32) -> T (bf16 hi + lo)
  static constexpr int kBytes = kOffT + kMat;
};

constexpr int kDlyChunk = 16;  // path nodes staged per round for the delayed commit

template <bool DLY, int BV>
struct DelayLds {  // k rows (FP32), u' of the tile's rows, coefficients, node ids
  static constexpr int kBVT = ((BV + 15) / 16) * 16;
  float k[DLY ? kDlyChunk * kMaxDim : 1];
  float u[DLY ? kDlyChunk * kBVT : 1];
  float c[DLY ? kMaxNodes : 1];
  int node[DLY ? kMaxNodes : 1];
};

template <typename T, int BV, int NQT, bool DLY, bool GATE>
__global__ __launch_bounds__(256) void tree_verify_kernel(
    int N, int H, int dk, int dv, int ntiles, float* __restrict__ S0,
    const int32_t* __restrict__ parents, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const float* __restrict__ beta, const float* __restrict__ g,
    float scale, float* __restrict__ out, Record<T> rec, uint64_t* __restrict__ mask_out,
    int32_t* __restrict__ dev_status, Record<T> prev, int Npv,
    const int32_t* __restrict__ last_acc, int32_t* __restrict__ commit_status, GateArgs ga) {
  using L = TreeLds<BV>;
  constexpr bool kStaged = std::is_same<T, bf16_t>::value;  // Q/K staged in LDS as bf16
  constexpr int NCT = (BV + 15) / 16;                        // MFMA column tiles
  constexpr int WC = NCT < 4 ? NCT : 4;                      // waves along columns
  constexpr int WR = 4 / WC;                                 // waves along rows
  // NQT = number of 16-node blocks (N <= 16 * NQT): every loop bound below is
  // a compile-time constant, so no MFMA sits under a runtime branch.
  constexpr int Np = 16 * NQT;
  constexpr int NK = 32 * ((NQT + 1) / 2);                   // k extent of N x N products
  constexpr int nrt = 2 * NQT;                               // Y row tiles (Q then K)
  constexpr int MAXRT = (nrt + WR - 1) / WR;                 // Y row tiles per wave
  constexpr int MAXNB = (NQT + WR - 1) / WR;                 // node blocks per wave
  constexpr int EPT = Np * NK / 256;                         // Np x NK entries per thread

  __shared__ __attribute__((aligned(16))) char smem[L::kBytes];
  __shared__ uint64_t smask[kMaxNodes];
  __shared__ float sG[kMaxNodes], seG[kMaxNodes], sbeta[kMaxNodes];
  __shared__ int sbad;
  __shared__ __attribute__((aligned(16))) DelayLds<DLY, BV> dly;
  __shared__ int sdly_n;
  __shared__ float sdly_s0;
  bf16_t* QKs = reinterpret_cast<bf16_t*>(smem);
  bf16_t* RTs = reinterpret_cast<bf16_t*>(smem);                 // R^T, split [kBVT][kLdH]
  bf16_t* UTs = reinterpret_cast<bf16_t*>(smem + L::kSplitT);    // U'^T, split
  constexpr int kRTLo = L::kBVT * kLdH;                          // lo offset in R^T / U'^T
  float* KK = reinterpret_cast<float*>(smem + L::kOffKK);        // then A
  float* QK = reinterpret_cast<float*>(smem + L::kOffQK);
  bf16_t* Attn = reinterpret_cast<bf16_t*>(smem + L::kOffQK);    // split, after phase 3
  float* Tl = reinterpret_cast<float*>(smem + L::kOffT);
  bf16_t* Ts = reinterpret_cast<bf16_t*>(smem + L::kOffT);       // split, after phase 4

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int koff = 8 * lg;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int tile = lid % ntiles;
  const int bh = lid / ntiles;
  const int b = bh / H;
  const int h = bh % H;
  const int r0 = tile * BV;
  const int cj = wave % WC;       // this wave's column tile
  const int rb = wave / WC;       // first row tile / node block of this wave
  const int ccol = 16 * cj + l16; // column within the tile (B fragments, D columns)
  const int srow = r0 + ccol;     // state row of this lane's column
  const bool sok = ccol < BV && srow < dv;

  // ---- 0. one round of loads, Q/K first (unconditional, clamped, masked).
  // Consuming a load waits for every load issued before it, so the state
  // tile is issued after what the per-head steps need.
  constexpr int qk_cpr = kMaxDim / 8;                 // chunks per staged row (zero past dk)
  constexpr int qk_total = 2 * Np * qk_cpr;
  constexpr int QKB = (qk_total + 255) / 256;         // 16-byte chunks per thread
  u32x4 qkw[kStaged ? QKB : 1];
  if (kStaged) {
    const bf16_t* qb = reinterpret_cast<const bf16_t*>(static_cast<const void*>(q));
    const bf16_t* kb = reinterpret_cast<const bf16_t*>(static_cast<const void*>(k));
#pragma unroll
    for (int x = 0; x < QKB; ++x) {
      const int idx = clampi(tid + 256 * x, qk_total - 1);
      const int r = idx / qk_cpr;
      const bool isq = r < Np;
      const int t = clampi(isq ? r : r - Np, N - 1);
      const int c8 = clampi(8 * (idx % qk_cpr), dk - 8);
      qkw[x] = *reinterpret_cast<const u32x4*>((isq ? qb : kb) +
                                               (((size_t)b * N + t) * H + h) * dk + c8);
    }
  }
  const int tn = clampi(lane, N - 1);
  const int pl = parents[(size_t)b * N + tn];
  const float gl = g[((size_t)b * N + tn) * H + h];
  const float bl = beta[((size_t)b * N + tn) * H + h];
  // The state tile (straight into MFMA B-fragment order) and V are requested
  // last in this round (load_state below): loads complete in issue order, so
  // the Q/K staging and the topology step wait only for what was issued
  // before them, while the state streams in behind steps 1-3.
  f32x4 Sraw[kMaxDim / 32][2];
  // V for the K row tiles this wave turns into R: its j-th K tile is row tile
  // rt = rb + WR*(iK0 + j) >= NQT, node block rt - NQT (D layout: node
  // 16*nb + 4*lg + r, column ccol).
  const int iK0 = NQT > rb ? (NQT - rb + WR - 1) / WR : 0;
  T vreg[MAXNB][4];
  // GATE: output gate values for the rows this lane stores (node
  // 16 nb + 4 lg + r of its node blocks nb = rb + WR j, column srow), requested
  // once the contraction has consumed the state registers (load_gate below):
  // in the first round of loads they would exceed the register budget and
  // make the compiler wait for the whole state tile before issuing them.
  float gvr[GATE ? MAXNB : 1][4];
  auto load_gate = [&]() {
    if constexpr (GATE) {
      const float* gp = ga.gate + (size_t)b * N * ga.ldg + h * dv + clampi(srow, dv - 1);
#pragma unroll
      for (int j = 0; j < MAXNB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          gvr[j][r] = gp[(size_t)clampi(16 * (rb + WR * j) + 4 * lg + r, N - 1) * ga.ldg];
    }
  };
  auto load_state = [&]() {
    const float* sptr = S0 + ((size_t)bh * dv + clampi(srow, dv - 1)) * dk;
#pragma unroll
    for (int ks = 0; ks < kMaxDim / 32; ++ks) {
      const int kk = clampi(32 * ks + koff, dk - 8);
      Sraw[ks][0] = load4(sptr + kk);
      Sraw[ks][1] = load4(sptr + kk + 4);
    }
#pragma unroll
    for (int j = 0; j < MAXNB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int nb = rb + WR * (iK0 + j) - NQT;
        const int t = clampi(16 * nb + 4 * lg + r, N - 1);
        vreg[j][r] = v[(((size_t)b * N + t) * H + h) * dv + clampi(srow, dv - 1)];
      }
  };

  // delayed commit: the previous draft's last accepted node, and node j's
  // mask and G in lane j of every wave
  int last_v = -1;
  uint64_t pmask_l = 0;
  float pG_l = 0.f;
  if (DLY) {
    last_v = last_acc[b];
    const int tj = clampi(lane, Npv - 1);
    pmask_l = prev.mask[(size_t)b * Npv + tj];
    pG_l = prev.G[(size_t)bh * Npv + tj];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep every load above issued before the state's
  load_state();
  __builtin_amdgcn_sched_barrier(0);

  if (kStaged) {
    static_assert(qk_total % 256 == 0, "every thread stages QKB chunks");
#pragma unroll
    for (int x = 0; x < QKB; ++x) {  // no branch: a load under one is waited for at once
      const int idx = tid + 256 * x;
      const int r = idx / qk_cpr;
      const int t = r < Np ? r : r - Np;
      const int c8 = 8 * (idx % qk_cpr);
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(QKs + r * kQKStride + c8) = (t < N && c8 < dk) ? qkw[x] : z;
    }
  }
  // T starts as zeros in both of its layouts (FP32 rows, or bf16 hi + lo rows)
  for (int idx = tid; idx < L::kMat / 16; idx += 256)
    reinterpret_cast<f32x4*>(Tl)[idx] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- 1. parents -> validation, ancestor-or-self masks and G (pointer jumping)
  if (wave == 0) {
    const int t = lane;
    const int p = t < N ? pl : -1;
    const bool bad = t < N && (p < -1 || p >= t);
    const uint64_t anybad = __ballot(bad);
    uint64_t m = t < N ? (1ull << t) : 0ull;
    float G = t < N ? gl : 0.f;
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
    smask[t] = m;
    sG[t] = G;
    seG[t] = expf(G);
    sbeta[t] = t < N ? bl : 0.f;
    if (t == 0) sbad = anybad != 0ull;
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
    if (DLY) {  // the accepted path, root first, and its coefficients
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
      if (okp && ((pm >> t) & 1ull)) {
        const int pos = __popcll(pm & ((1ull << t) - 1ull));
        dly.node[pos] = t;
        dly.c[pos] = expf(Glast - pG_l);
      }
      if (t == 0) {
        sdly_n = okp ? __popcll(pm) : 0;
        sdly_s0 = expf(Glast);
        if (tile == 0 && h == 0 && commit_status)
          commit_status[b] = (lst == -1 || okp) ? GDN_OK : GDN_ERR_TOPOLOGY;
      }
    }
  }
  __syncthreads();

  // ---- delayed commit, staging: k rows and u' of path nodes [c0, c0 + 16)
  const int dn = DLY ? sdly_n : 0;  // path length (0: nothing to commit)
  constexpr int kTE = std::is_same<T, bf16_t>::value ? 8 : 4;  // elements per 16-byte chunk
  constexpr int DKC = kDlyChunk * kMaxDim / kTE / 256;          // k chunks per thread
  constexpr int DUC = (kDlyChunk * L::kBVT + 255) / 256;        // u' values per thread
  using KChunk = typename std::conditional<std::is_same<T, bf16_t>::value, u32x4, f32x4>::type;
  KChunk dkr[DLY ? DKC : 1];
  float dur[DLY ? DUC : 1];
  auto dly_load = [&](int c0) {
#pragma unroll
    for (int x = 0; x < DKC; ++x) {
      const int idx = tid + 256 * x;                 // chunk of (node j, column)
      const int j = idx / (kMaxDim / kTE);
      const int col = clampi(kTE * (idx % (kMaxDim / kTE)), dk - kTE);
      const int nd = dly.node[clampi(c0 + j, dn > 0 ? dn - 1 : 0)];
      dkr[x] = *reinterpret_cast<const KChunk*>(prev.K + ((size_t)bh * Npv + nd) * dk + col);
    }
#pragma unroll
    for (int x = 0; x < DUC; ++x) {
      const int idx = clampi(tid + 256 * x, kDlyChunk * L::kBVT - 1);
      const int j = idx / L::kBVT;
      const int r = clampi(r0 + idx % L::kBVT, dv - 1);
      const int nd = dly.node[clampi(c0 + j, dn > 0 ? dn - 1 : 0)];
      dur[x] = prev.up[((size_t)bh * Npv + nd) * dv + r];
    }
  };
  auto dly_store = [&]() {
#pragma unroll
    for (int x = 0; x < DKC; ++x) {
      const int idx = tid + 256 * x;
      const int j = idx / (kMaxDim / kTE);
      const int col = kTE * (idx % (kMaxDim / kTE));
      const f32x4 a = widen4(reinterpret_cast<const typename Raw4<T>::type*>(&dkr[x])[0]);
      *reinterpret_cast<f32x4*>(&dly.k[j * kMaxDim + col]) = a;
      if constexpr (kTE == 8) {
        const f32x4 b8 = widen4(reinterpret_cast<const typename Raw4<T>::type*>(&dkr[x])[1]);
        *reinterpret_cast<f32x4*>(&dly.k[j * kMaxDim + col + 4]) = b8;
      }
    }
#pragma unroll
    for (int x = 0; x < DUC; ++x) {
      const int idx = tid + 256 * x;
      if (idx < kDlyChunk * L::kBVT) dly.u[idx] = dur[x];
    }
  };
  // the whole commit on the register tile, then its write-back; `first_staged`
  // says whether chunk 0 is already in LDS.  With 16-row tiles or narrower
  // all four waves hold the same rows (WR == 4), so each updates a quarter of
  // the columns (ks chunks [KQ0, KQ1)), writes it back, and the committed
  // quarters are exchanged through the N x N A block's LDS, free once the
  // solves are done (`xchg`, which then costs two barriers).
  constexpr bool kSplit = WR == 4;
  constexpr int KQN = kSplit ? (kMaxDim / 32) / 4 : kMaxDim / 32;
  const int KQ0 = kSplit ? rb * KQN : 0;
  constexpr int kXLd = kMaxDim + 4;  // row stride (floats) of the exchanged tile
  auto dly_commit = [&](bool first_staged, bool xchg) {
    if (dn == 0) return;  // uniform
    // Stores count in the same vector-memory counter as loads: every state
    // and V register is consumed here, before the first write-back store, so
    // no later wait for those loads also waits for the stores to drain.
#pragma unroll
    for (int ks = 0; ks < kMaxDim / 32; ++ks) asm volatile("" : "+v"(Sraw[ks][0]), "+v"(Sraw[ks][1]));
#pragma unroll
    for (int j = 0; j < MAXNB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(vreg[j][r]));
    const float s0 = sdly_s0;
#pragma unroll
    for (int ks = 0; ks < kMaxDim / 32; ++ks)
      if (!kSplit || (ks >= KQ0 && ks < KQ0 + KQN))
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Sraw[ks][0][e] = Sraw[ks][0][e] * s0;
          Sraw[ks][1][e] = Sraw[ks][1][e] * s0;
        }
    for (int c0 = 0; c0 < dn; c0 += kDlyChunk) {  // uniform
      if (c0 > 0 || !first_staged) {
        __syncthreads();  // every wave is done with the previous chunk
        dly_load(c0);
        dly_store();
        __syncthreads();
      }
      const int nc = __builtin_amdgcn_readfirstlane(dn - c0 < kDlyChunk ? dn - c0 : kDlyChunk);
      // Narrow tiles: columns [32 K0, 32 (K0 + KQN)) of the tile, a compile-time
      // range, so each node's LDS reads issue together with no branch between.
      auto apply_nodes = [&](auto k0c) {
        constexpr int K0 = decltype(k0c)::value;
        for (int jj = 0; jj < nc; ++jj) {  // uniform; node order as in the commit kernel
          const float cu = dly.c[c0 + jj] * dly.u[jj * L::kBVT + (ccol < L::kBVT ? ccol : 0)];
          f32x4 kv[KQN][2];
#pragma unroll
          for (int q = 0; q < KQN; ++q) {
            const float* kr = &dly.k[jj * kMaxDim + 32 * (K0 + q) + koff];
            kv[q][0] = *reinterpret_cast<const f32x4*>(kr);
            kv[q][1] = *reinterpret_cast<const f32x4*>(kr + 4);
          }
#pragma unroll
          for (int q = 0; q < KQN; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              Sraw[K0 + q][0][e] = fmaf(cu, kv[q][0][e], Sraw[K0 + q][0][e]);
              Sraw[K0 + q][1][e] = fmaf(cu, kv[q][1][e], Sraw[K0 + q][1][e]);
            }
        }
      };
      if constexpr (kSplit) {
        switch (__builtin_amdgcn_readfirstlane(rb)) {  // this wave's quarter of the columns
          case 0: apply_nodes(std::integral_constant<int, 0 * KQN>{}); break;
          case 1: apply_nodes(std::integral_constant<int, 1 * KQN>{}); break;
          case 2: apply_nodes(std::integral_constant<int, 2 * KQN>{}); break;
          default: apply_nodes(std::integral_constant<int, 3 * KQN>{}); break;
        }
      } else {
        // wide tiles: every wave reads all of k per node, bounded by LDS
        // bandwidth, where interleaving the reads with the multiply-adds is
        // faster than issuing them together
        for (int jj = 0; jj < nc; ++jj) {
          const float cu = dly.c[c0 + jj] * dly.u[jj * L::kBVT + (ccol < L::kBVT ? ccol : 0)];
#pragma unroll
          for (int ks = 0; ks < kMaxDim / 32; ++ks) {
            const float* kr = &dly.k[jj * kMaxDim + 32 * ks + koff];
            const f32x4 k0 = *reinterpret_cast<const f32x4*>(kr);
            const f32x4 k1 = *reinterpret_cast<const f32x4*>(kr + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              Sraw[ks][0][e] = fmaf(cu, k0[e], Sraw[ks][0][e]);
              Sraw[ks][1][e] = fmaf(cu, k1[e], Sraw[ks][1][e]);
            }
          }
        }
      }
    }
    if ((kSplit || rb == 0) && sok) {  // write-back: each element once
      float* wp = S0 + ((size_t)bh * dv + srow) * dk;
#pragma unroll
      for (int ks = 0; ks < kMaxDim / 32; ++ks) {
        const int col = 32 * ks + koff;
        if ((!kSplit || (ks >= KQ0 && ks < KQ0 + KQN)) && col < dk) {
          *reinterpret_cast<f32x4*>(wp + col) = Sraw[ks][0];
          *reinterpret_cast<f32x4*>(wp + col + 4) = Sraw[ks][1];
        }
      }
    }
    if (kSplit && xchg) {  // every wave needs the whole committed tile for step 4
      float* X = KK;       // 16 rows x kXLd floats fit in the A block's space
      __syncthreads();     // the solves (readers of A) are done
#pragma unroll
      for (int ks = 0; ks < kMaxDim / 32; ++ks)
        if (ks >= KQ0 && ks < KQ0 + KQN) {
          *reinterpret_cast<f32x4*>(X + l16 * kXLd + 32 * ks + koff) = Sraw[ks][0];
          *reinterpret_cast<f32x4*>(X + l16 * kXLd + 32 * ks + koff + 4) = Sraw[ks][1];
        }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < kMaxDim / 32; ++ks) {
        Sraw[ks][0] = *reinterpret_cast<const f32x4*>(X + l16 * kXLd + 32 * ks + koff);
        Sraw[ks][1] = *reinterpret_cast<const f32x4*>(X + l16 * kXLd + 32 * ks + koff + 4);
      }
    }
  };
  static_assert(!kSplit || 16 * kXLd * 4 <= L::kMat, "exchange tile exceeds the A block");
  if (DLY && dn > 0) dly_load(0);  // lands while steps 2-3 run

  const bool bad = sbad != 0;
  if (tile == 0) {  // factor record: copy of k for this head
    if constexpr (kStaged) {  // the staged K rows in LDS hold exactly these bits
      constexpr int kC8 = kMaxDim / 8;              // 16-byte chunks per staged row
      constexpr int RKC = Np * kC8 / 256;           // chunks per thread
      u32x4 kc[RKC];
#pragma unroll
      for (int x = 0; x < RKC; ++x) {  // all reads first, then the stores
        const int idx = tid + 256 * x;
        kc[x] = *reinterpret_cast<const u32x4*>(QKs + (Np + idx / kC8) * kQKStride +
                                                8 * (idx % kC8));
      }
#pragma unroll
      for (int x = 0; x < RKC; ++x) {
        const int idx = tid + 256 * x;
        const int t = idx / kC8;
        const int c8 = 8 * (idx % kC8);
        if (t < N && c8 < dk)
          *reinterpret_cast<u32x4*>(rec.K + ((size_t)bh * N + t) * dk + c8) = kc[x];
      }
    } else {
      const int cpr = dk / 4;
      for (int idx = tid; idx < N * cpr; idx += 256) {
        const int t = idx / cpr;
        const int cc = 4 * (idx % cpr);
        copy4e(reinterpret_cast<float*>(rec.K + ((size_t)bh * N + t) * dk + cc),
               reinterpret_cast<const float*>(k) + (((size_t)b * N + t) * H + h) * dk + cc);
      }
    }
  }
  if (bad) {  // uniform: zero this tile's outputs (a delayed commit still applies)
    if (DLY) dly_commit(false, false);
    const int c = tid % BV;
    for (int t = tid / BV; t < N; t += 256 / BV)
      if (r0 + c < dv) {
        const size_t o = (((size_t)b * N + t) * H + h) * dv + r0 + c;
        if constexpr (GATE)  // the gated form has no O: Y = bf16(0 * SiLU(gate)), as gated zeros
          ga.Y[o] = to_bf16(0.f * silu(ga.gate[((size_t)b * N + t) * ga.ldg + h * dv + r0 + c]));
        else
          out[o] = 0.f;
        rec.up[((size_t)bh * N + t) * dv + r0 + c] = 0.f;
      }
    return;
  }

  // ---- 2. Gram blocks C = [Q; K] K^T on MFMA (tiles with j <= t only)
  if constexpr (kStaged) {
    // Lower-triangle tiles (t-block >= j-block) of Q K^T and K K^T.  Row
    // blocks are paired (NQT-1-p, p) so every pair holds NQT+1 tiles, and
    // wave w takes pair w/2 of Q (w even) or of K (w odd): it reads the A
    // fragments of its two row blocks once and each K column block once,
    // shared by both rows (the next column block's fragments are read while
    // this one multiplies).  The job is a compile-time variant per wave, so
    // no load or MFMA sits under a runtime branch.  Each tile sums over k in
    // the same order as any other schedule, so the Gram values do not depend
    // on it.
    constexpr int KS = kMaxDim / 32;
    auto gram_job = [&](auto wc) {
      constexpr int Wc = decltype(wc)::value;
      constexpr int npairs = (NQT + 1) / 2;
      if constexpr (Wc < 2 * npairs) {
        constexpr bool isq = Wc % 2 == 0;
        constexpr int ra = NQT - 1 - Wc / 2;  // the longer row block of the pair
        constexpr int rs = Wc / 2;            // the shorter one (== ra: a single block)
        constexpr bool two = rs < ra;
        const bf16_t* rows = QKs + (isq ? 0 : Np) * kQKStride;
        float* dst = isq ? QK : KK;
        bf16x8 fa[KS], fs[two ? KS : 1], kb[2][KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {  // columns past dk are zero
          fa[ks] = lds_bf16x8(rows + (16 * ra + l16) * kQKStride + 32 * ks + koff);
          if constexpr (two) fs[ks] = lds_bf16x8(rows + (16 * rs + l16) * kQKStride + 32 * ks + koff);
        }
        auto kload = [&](int ct, bf16x8 (&dstf)[KS]) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            dstf[ks] = lds_bf16x8(QKs + (Np + 16 * ct + l16) * kQKStride + 32 * ks + koff);
        };
        kload(0, kb[0]);
#pragma unroll
        for (int ct = 0; ct <= ra; ++ct) {
          if (ct + 1 <= ra) kload(ct + 1, kb[(ct + 1) & 1]);  // in flight while ct multiplies
          __builtin_amdgcn_sched_barrier(0);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(fa[ks], kb[ct & 1][ks], acc);
          mfma_drain(acc);  // the stores below may sit behind a branch
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(16 * ra + 4 * lg + r) * kLd + 16 * ct + l16] = acc[r];
          if (two && ct <= rs) {  // compile-time after unrolling
            f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              acc2 = mfma16x16x32(fs[two ? ks : 0], kb[ct & 1][ks], acc2);
            mfma_drain(acc2);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              dst[(16 * rs + 4 * lg + r) * kLd + 16 * ct + l16] = acc2[r];
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
  } else {
  for (int tileid = wave; tileid < nrt * NQT; tileid += 4) {
    const int rt = tileid / NQT;
    const int ct = tileid % NQT;
    const bool isq = rt < NQT;
    const int rtl = isq ? rt : rt - NQT;
    if (ct > rtl) continue;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    {
      const int ti = 16 * rtl + l16;
      const int tj = 16 * ct + l16;
      const float* arow = reinterpret_cast<const float*>(isq ? (const void*)q : (const void*)k) +
                          (((size_t)b * N + (ti < N ? ti : 0)) * H + h) * dk;
      const float* brow = reinterpret_cast<const float*>(k) +
                          (((size_t)b * N + (tj < N ? tj : 0)) * H + h) * dk;
      const int nks = (dk + 31) / 32;
      for (int ks = 0; ks < nks; ++ks) {
        const int kk = 32 * ks + koff;
        bf16x8 ah, al, bh8, bl8;
        frag_global(arow + kk, ti < N && kk < dk, ah, al);
        frag_global(brow + kk, tj < N && kk < dk, bh8, bl8);
        acc = mfma16x16x32(ah, bh8, acc);
        acc = mfma16x16x32(ah, bl8, acc);
        acc = mfma16x16x32(al, bh8, acc);
      }
    }
    float* dst = isq ? QK : KK;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(16 * rtl + 4 * lg + r) * kLd + 16 * ct + l16] = acc[r];
  }
  }
  if (DLY && dn > 0) dly_store();  // the path loads issued after step 1
  __syncthreads();

  // ---- 3. A (FP32, in place of K K^T) and Attn (split bf16, in place of
  // Q K^T) over all N x N entries, exact zeros off the masks; then the rows
  // of T on root paths (one lane per node, written split into bf16 hi + lo).
  // Every operand is read unconditionally first (all in bounds: t < Np,
  // j < NK), so the reads issue together instead of one masked round trip
  // per entry.
  float attn[EPT], kkv[EPT], qkv[EPT], gt[EPT], gj[EPT], bt[EPT];
  uint64_t mt[EPT];
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int idx = tid + 256 * x;
    const int t = idx / NK;
    const int j = idx % NK;
    mt[x] = smask[t];
    gt[x] = sG[t];
    gj[x] = sG[j];
    bt[x] = sbeta[t];
    kkv[x] = KK[t * kLd + j];
    qkv[x] = QK[t * kLd + j];
  }
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int idx = tid + 256 * x;
    const int t = idx / NK;
    const int j = idx % NK;
    const bool on = (mt[x] >> j) & 1ull;  // j on t's root path (t >= N: empty mask)
    const float dec = __expf(gt[x] - gj[x]);
    KK[t * kLd + j] = (on && j != t) ? bt[x] * dec * kkv[x] : 0.f;
    attn[x] = on ? scale * dec * qkv[x] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int idx = tid + 256 * x;
    store_split1(Attn + (idx / NK) * kLdH + idx % NK, kSplitLo, attn[x]);
  }
  // A draft with a root path deeper than kPathMax is "deep": its T is solved
  // in FP32 by blocks (below) and split in the epilogue.  Every wave reads
  // the depths (smask is complete since step 1), so the decision is uniform
  // without a barrier.
  const bool deep = __ballot(lane < N && __popcll(smask[lane < N ? lane : 0]) > kPathMax) != 0ull;
  if (tid < N) {
    const int t = tid;
    const uint64_t m = smask[t];
    const int d = __popcll(m);
    // Rows of T go straight into the split bf16 layout the epilogue's
    // products read (T[t][j] = hi + lo).  One variant per wave (all nodes are
    // in wave 0), chosen by its deepest path, so the lanes never run two
    // solves one after the other.
    auto put_split = [&](int j, float x) { store_split1(Ts + t * kLdH + j, kSplitLo, x); };
    auto put_f32 = [&](int j, float x) { Tl[t * kLd + j] = x; };
    if (deep) {
      // diagonal block of t's 16-node block: t's root path restricted to the
      // block is a suffix of it (parents precede children), at most 16 nodes
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
  if (deep) {  // uniform
    // Blocked forward substitution for T = (I + A)^{-1} over 16-node blocks:
    // with the diagonal blocks D_ii = (I + A_ii)^{-1} in place, block row i
    // (i = 1 .. NQT-1, in order) is T_ij = -D_ii sum_{k=j}^{i-1} A_ik T_kj for
    // j < i, wave j taking column block j, on FP32 MFMA.  Entries off the
    // ancestor relation stay exact zeros (each term holds a masked factor).
    __syncthreads();  // the diagonal blocks are in Tl
#pragma unroll
    for (int i = 1; i < NQT; ++i) {
      const int j = wave;
      // X = sum_k A_ik T_kj goes to T's (i, j) block, where D_ii X reads it
      // back as its B operand after a barrier (other lanes wrote it)
      float* blk = Tl + (16 * i) * kLd + 16 * j;
      if (j < i) {  // uniform per wave
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        for (int kb = j; kb < i; ++kb)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            x = mfma16x16x4f32(KK[(16 * i + l16) * kLd + 16 * kb + 4 * c + lg],
                               Tl[(16 * kb + 4 * c + lg) * kLd + 16 * j + l16], x);
#pragma unroll
        for (int r = 0; r < 4; ++r) blk[(4 * lg + r) * kLd + l16] = x[r];
      }
      __syncthreads();
      if (j < i) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          y = mfma16x16x4f32(Tl[(16 * i + l16) * kLd + 16 * i + 4 * c + lg],
                             blk[(4 * c + lg) * kLd + l16], y);
        // every lane's reads of X were issued before these writes, which
        // depend on their results
#pragma unroll
        for (int r = 0; r < 4; ++r) blk[(4 * lg + r) * kLd + l16] = -y[r];
      }
      __syncthreads();  // block row i is complete before row i + 1 reads it
    }
  }

  if (DLY) dly_commit(true, true);

  // ---- 4. Y = [Q; K] S0_tile^T (this wave: column tile cj, row tiles rb + WR*i)
  f32x4 yacc[MAXRT];
#pragma unroll
  for (int i = 0; i < MAXRT; ++i) yacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (kStaged && MAXRT >= 4) {
    // Wide tiles (8 row tiles per wave): the A fragments of the next
    // 32-column chunk are read while this chunk's MFMAs run (two register
    // sets).  Row tiles past nrt read staged rows that exist (the staging area
    // holds 2 * kMaxNodes rows) and are not used.
    constexpr int KS = kMaxDim / 32;
    bf16x8 afr[2][MAXRT];
    auto aload = [&](int ks, bf16x8 (&a)[MAXRT]) {
#pragma unroll
      for (int i = 0; i < MAXRT; ++i)
        a[i] = lds_bf16x8(QKs + (16 * (rb + WR * i) + l16) * kQKStride + 32 * ks + koff);
    };
    aload(0, afr[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {  // zero-padded past dk: no branch
      if (ks + 1 < KS) aload(ks + 1, afr[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 bhi, blo;
      const bool okk = sok && 32 * ks + koff < dk;
      split8(mask4(Sraw[ks][0], okk), mask4(Sraw[ks][1], okk), bhi, blo);
#pragma unroll
      for (int i = 0; i < MAXRT; ++i) {
        const int rt = rb + WR * i;  // rb < WR, so rt < nrt except on the last i
        if (WR * i + WR <= nrt || rt < nrt) {
          yacc[i] = mfma16x16x32(afr[ks & 1][i], bhi, yacc[i]);
          yacc[i] = mfma16x16x32(afr[ks & 1][i], blo, yacc[i]);
        }
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < kMaxDim / 32; ++ks) {  // zero-padded past dk: no branch
      bf16x8 bhi, blo;
      const bool okk = sok && 32 * ks + koff < dk;
      split8(mask4(Sraw[ks][0], okk), mask4(Sraw[ks][1], okk), bhi, blo);
#pragma unroll
      for (int i = 0; i < MAXRT; ++i) {
        const int rt = rb + WR * i;  // rb < WR, so rt < nrt except on the last i
        if (WR * i + WR <= nrt || rt < nrt) {
          if (kStaged) {
            const bf16x8 a8 = lds_bf16x8(QKs + (16 * rt + l16) * kQKStride + 32 * ks + koff);
            yacc[i] = mfma16x16x32(a8, bhi, yacc[i]);
            yacc[i] = mfma16x16x32(a8, blo, yacc[i]);
          } else {
            const bool isq = rt < NQT;
            const int t = 16 * (isq ? rt : rt - NQT) + l16;
            const float* arow = reinterpret_cast<const float*>(isq ? (const void*)q : (const void*)k) +
                                (((size_t)b * N + (t < N ? t : 0)) * H + h) * dk;
            const int kk = 32 * ks + koff;
            bf16x8 ah, al;
            frag_global(arow + kk, t < N && kk < dk, ah, al);
            yacc[i] = mfma16x16x32(ah, bhi, yacc[i]);
            yacc[i] = mfma16x16x32(ah, blo, yacc[i]);
            yacc[i] = mfma16x16x32(al, bhi, yacc[i]);
          }
        }
      }
    }
  }
  mfma_drain_all(yacc);  // the Y accumulators are read after the barrier's branch
  load_gate();      // consumed by the output step, after R and U'
  __syncthreads();  // Q/K reads and the solves are done: region A becomes R^T, U'^T

  // ---- 5. epilogue
  // R = diag(beta) (V - diag(e^G) K S0^T) from the K-row accumulators
  f32x4 rv[MAXNB];
#pragma unroll
  for (int j = 0; j < MAXNB; ++j) rv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto form_r = [&]() {
#pragma unroll
    for (int i = 0; i < MAXRT; ++i) {
      const int rt = rb + WR * i;
      if (rt >= NQT && rt < nrt) {
        const int nb = rt - NQT;
        const int j = i - iK0;  // this wave's j-th K tile: see the vreg loads
#pragma unroll
        for (int jj = 0; jj < MAXNB; ++jj)
          if (jj == j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 16 * nb + 4 * lg + r;
              const float vv = sok ? widen1(vreg[jj][r]) : 0.f;
              rv[jj][r] = sbeta[t] * (vv - seG[t] * yacc[i][r]);
            }
          }
      }
    }
  };
  // the node outputs of block nb (rows 16 nb + 4 lg + r, column srow), from
  // the accumulator of O's block
  auto store_out = [&](int nb, int j, const f32x4& acc) {
    if (sok) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * nb + 4 * lg + r;
        if (t < N) {
          const size_t o = (((size_t)b * N + t) * H + h) * dv + srow;
          if constexpr (GATE)
            ga.Y[o] = to_bf16(acc[r] * silu(gvr[j][r]));  // gdn_gate_merge's arithmetic
          else
            out[o] = acc[r];
        }
      }
    }
  };
  auto store_up = [&](int nb, const f32x4& acc) {
    if (sok) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * nb + 4 * lg + r;
        if (t < N) rec.up[((size_t)bh * N + t) * dv + srow] = acc[r];
      }
    }
  };

  if constexpr (WR == 1) {
    // Every node block of this wave's 16 state rows is in its registers (the
    // Q and K row tiles of all NQT blocks), so U' = T R and O = Attn U' run
    // as chains of 16x16x16 products whose B operands are the previous
    // result's accumulators, split into bf16 hi + lo: R and U' never leave
    // the registers and no barrier separates the steps.  T and Attn are lower
    // triangular (parents precede children), so block row i sums over the
    // k blocks 0..i only.  A operands come from LDS: T split into bf16, or in
    // FP32 after the blocked solve of a deep draft (split here).
    form_r();
    auto run = [&](auto deep_c) {
      constexpr bool kDeep = decltype(deep_c)::value;
      auto tfrag = [&](int i, int kb, s16x4& ah, s16x4& al) {
        const int row = 16 * i + l16, col = 16 * kb + 4 * lg;
        if constexpr (kDeep) {
          split4(*reinterpret_cast<const f32x4*>(Tl + row * kLd + col), ah, al);
        } else {
          ah = __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(Ts + row * kLdH + col));
          al = __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(Ts + kSplitLo + row * kLdH + col));
        }
      };
      auto afrag = [&](int i, int kb, s16x4& ah, s16x4& al) {
        const int o = (16 * i + l16) * kLdH + 16 * kb + 4 * lg;
        ah = __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(Attn + o));
        al = __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(Attn + kSplitLo + o));
      };
      constexpr int NPAIR = NQT * (NQT + 1) / 2;  // lower-triangular blocks (i, kb <= i)
      s16x4 th[NPAIR], tl[NPAIR];
#pragma unroll
      for (int i = 0, x = 0; i < NQT; ++i)
#pragma unroll
        for (int kb = 0; kb <= i; ++kb, ++x) tfrag(i, kb, th[x], tl[x]);
      s16x4 rh[NQT], rl[NQT];
#pragma unroll
      for (int kb = 0; kb < NQT; ++kb) split4(rv[kb], rh[kb], rl[kb]);
      f32x4 ua[NQT];
#pragma unroll
      for (int i = 0, x = 0; i < NQT; ++i) {
        ua[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb <= i; ++kb, ++x) {
          ua[i] = mfma16x16x16(th[x], rh[kb], ua[i]);
          ua[i] = mfma16x16x16(th[x], rl[kb], ua[i]);
          ua[i] = mfma16x16x16(tl[x], rh[kb], ua[i]);
        }
      }
      s16x4 ah[NPAIR], al[NPAIR];  // Attn fragments, read while U' multiplies
#pragma unroll
      for (int i = 0, x = 0; i < NQT; ++i)
#pragma unroll
        for (int kb = 0; kb <= i; ++kb, ++x) afrag(i, kb, ah[x], al[x]);
      mfma_drain_all(ua);  // U' is read below, partly under branches
      s16x4 uh[NQT], ul[NQT];
#pragma unroll
      for (int kb = 0; kb < NQT; ++kb) split4(ua[kb], uh[kb], ul[kb]);
      f32x4 oa[NQT];
#pragma unroll
      for (int i = 0, x = 0; i < NQT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) oa[i][r] = scale * seG[16 * i + 4 * lg + r] * yacc[i][r];
#pragma unroll
        for (int kb = 0; kb <= i; ++kb, ++x) {
          oa[i] = mfma16x16x16(ah[x], uh[kb], oa[i]);
          oa[i] = mfma16x16x16(ah[x], ul[kb], oa[i]);
          oa[i] = mfma16x16x16(al[x], uh[kb], oa[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < NQT; ++i) store_up(i, ua[i]);
      mfma_drain_all(oa);
#pragma unroll
      for (int i = 0; i < NQT; ++i) store_out(i, i, oa[i]);
    };
    if (deep)
      run(std::integral_constant<bool, true>{});
    else
      run(std::integral_constant<bool, false>{});
  } else {
    // Narrow tiles: the waves hold different node blocks of the same state
    // rows, so R and U' pass through LDS (R^T, U'^T split into bf16 hi + lo).
    // T is already split, except after an FP32 solve (deep paths): then its
    // rows go to registers and are split in place after a barrier.
    float trow[EPT];
    if (deep) {
#pragma unroll
      for (int x = 0; x < EPT; ++x) {
        const int idx = tid + 256 * x;
        trow[x] = Tl[(idx / NK) * kLd + idx % NK];
      }
    }
    form_r();
    if (deep) {
      __syncthreads();  // every FP32 row is read before the split rows overwrite it
#pragma unroll
      for (int x = 0; x < EPT; ++x) {
        const int idx = tid + 256 * x;
        store_split1(Ts + (idx / NK) * kLdH + idx % NK, kSplitLo, trow[x]);
      }
    }
#pragma unroll
    for (int j = 0; j < MAXNB; ++j) {
      const int nb = rb + WR * (iK0 + j) - NQT;
      if (nb >= 0 && nb < NQT) store_split4(RTs + ccol * kLdH + 16 * nb + 4 * lg, kRTLo, rv[j]);
    }
    if (NK > Np) {  // zero the k padding [Np, NK) of R^T and U'^T
      constexpr int PAD = NK > Np ? NK - Np : 1;
      for (int idx = tid; idx < L::kBVT * PAD; idx += 256) {
        const int o = (idx / PAD) * kLdH + Np + idx % PAD;
        RTs[o] = 0;
        RTs[kRTLo + o] = 0;
        UTs[o] = 0;
        UTs[kRTLo + o] = 0;
      }
    }
    __syncthreads();
    // U' = T R  (A = T rows, B = R^T rows; three passes)
#pragma unroll
    for (int j = 0; j < MAXNB; ++j) {
      const int nb = rb + WR * j;
      if (nb < NQT) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NK / 32; ++ks) {
          const int ao = (16 * nb + l16) * kLdH + 32 * ks + koff;
          const int bo = ccol * kLdH + 32 * ks + koff;
          const bf16x8 ah = lds_bf16x8(Ts + ao), al = lds_bf16x8(Ts + kSplitLo + ao);
          const bf16x8 bh8 = lds_bf16x8(RTs + bo), bl8 = lds_bf16x8(RTs + kRTLo + bo);
          acc = mfma16x16x32(ah, bh8, acc);
          acc = mfma16x16x32(ah, bl8, acc);
          acc = mfma16x16x32(al, bh8, acc);
        }
        mfma_drain(acc);
        store_split4(UTs + ccol * kLdH + 16 * nb + 4 * lg, kRTLo, acc);
        store_up(nb, acc);
      }
    }
    __syncthreads();
    // O = scale e^G Y_q + Attn U'   (Attn carries the scale).  Node block nb of
    // this wave is Q row tile rt = nb = rb + WR*j, whose Y accumulator is yacc[j].
#pragma unroll
    for (int j = 0; j < MAXNB; ++j) {
      const int nb = rb + WR * j;
      if (nb < NQT) {
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = scale * seG[16 * nb + 4 * lg + r] * yacc[j][r];
#pragma unroll
        for (int ks = 0; ks < NK / 32; ++ks) {
          const int ao = (16 * nb + l16) * kLdH + 32 * ks + koff;
          const int bo = ccol * kLdH + 32 * ks + koff;
          const bf16x8 ah = lds_bf16x8(Attn + ao), al = lds_bf16x8(Attn + kSplitLo + ao);
          const bf16x8 bh8 = lds_bf16x8(UTs + bo), bl8 = lds_bf16x8(UTs + kRTLo + bo);
          acc = mfma16x16x32(ah, bh8, acc);
          acc = mfma16x16x32(ah, bl8, acc);
          acc = mfma16x16x32(al, bh8, acc);
        }
        mfma_drain(acc);
        store_out(nb, j, acc);
      }
    }
  }
}

struct DelayArgs {
  const void* prev_factors;
  int Np;
  const int32_t* last;
  int32_t* commit_status;
  GateArgs gate;
};

template <typename T, int BV, int NQT, bool GATE>
hipError_t launch_bvng(int B, int N, int H, int dk, int dv, float* S0, const int32_t* parents,
                       const T* q, const T* k, const T* v, const float* beta, const float* g,
                       float scale, float* out, const Record<T>& rec, uint64_t* mask_out,
                       int32_t* dev_status, const DelayArgs& da, int dtype, hipStream_t stream) {
  const int ntiles = (dv + BV - 1) / BV;
  const long grid = (long)B * H * ntiles;
  if (da.prev_factors) {
    const RecordLayout Lp = record_layout(B, da.Np, H, dk, dv, dtype);
    const Record<T> prev = record_views<T>(const_cast<void*>(da.prev_factors), Lp);
    hipLaunchKernelGGL((tree_verify_kernel<T, BV, NQT, true, GATE>), dim3((unsigned)grid),
                       dim3(256), 0, stream, N, H, dk, dv, ntiles, S0, parents, q, k, v, beta, g,
                       scale, out, rec, mask_out, dev_status, prev, da.Np, da.last,
                       da.commit_status, da.gate);
  } else {
    hipLaunchKernelGGL((tree_verify_kernel<T, BV, NQT, false, GATE>), dim3((unsigned)grid),
                       dim3(256), 0, stream, N, H, dk, dv, ntiles, S0, parents, q, k, v, beta, g,
                       scale, out, rec, mask_out, dev_status, Record<T>{}, 1, nullptr, nullptr,
                       da.gate);
  }
  return hipGetLastError();
}

template <typename T, int BV, int NQT>
hipError_t launch_bvn(int B, int N, int H, int dk, int dv, float* S0, const int32_t* parents,
                      const T* q, const T* k, const T* v, const float* beta, const float* g,
                      float scale, float* out, const Record<T>& rec, uint64_t* mask_out,
                      int32_t* dev_status, const DelayArgs& da, int dtype, hipStream_t stream) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (da.gate.gate)
      return launch_bvng<T, BV, NQT, true>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale,
                                           out, rec, mask_out, dev_status, da, dtype, stream);
  }
  return launch_bvng<T, BV, NQT, false>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale,
                                        out, rec, mask_out, dev_status, da, dtype, stream);
}

template <typename T, int BV>
hipError_t launch_bv(int B, int N, int H, int dk, int dv, float* S0, const int32_t* parents,
                     const T* q, const T* k, const T* v, const float* beta, const float* g,
                     float scale, float* out, const Record<T>& rec, uint64_t* mask_out,
                     int32_t* dev_status, const DelayArgs& da, int dtype, hipStream_t stream) {
  switch ((N + 15) / 16) {
    case 1:
      return launch_bvn<T, BV, 1>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                                  mask_out, dev_status, da, dtype, stream);
    case 2:
      return launch_bvn<T, BV, 2>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                                  mask_out, dev_status, da, dtype, stream);
    case 3:
      return launch_bvn<T, BV, 3>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                                  mask_out, dev_status, da, dtype, stream);
    default:
      return launch_bvn<T, BV, 4>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                                  mask_out, dev_status, da, dtype, stream);
  }
}

hipError_t launch_tree_ws(int SW, int B, int N, int H, int dk, int dv, float* S0,
                          const int32_t* parents, const bf16_t* q, const bf16_t* k,
                          const bf16_t* v, const float* beta, const float* g, float scale,
                          float* out, const Record<bf16_t>& rec, uint64_t* mask_out,
                          int32_t* dev_status, const void* prev_factors, int Npv,
                          const int32_t* last, int32_t* commit_status, GateArgs ga,
                          hipStream_t stream);

template <typename T>
hipError_t launch_tree_verify_t(int B, int N, int H, int dk, int dv, float* S0,
                                const int32_t* parents, const T* q, const T* k, const T* v,
                                const float* beta, const float* g, float scale, float* out,
                                void* factors, uint64_t* mask_out, int32_t* dev_status,
                                const DelayArgs& da, hipStream_t stream, int dtype) {
  const RecordLayout L = record_layout(B, N, H, dk, dv, dtype);
  Record<T> rec = record_views<T>(factors, L);
  // Tile width: the widest of 64/32/16/8 state rows that still gives one
  // workgroup per compute unit (256), else the narrowest; 16-row tiles need
  // only 128 workgroups.  Every tile repeats its head's per-head steps and the
  // step time of a workgroup is set by their latency, so at batch 1 (8 heads)
  // 128 tiles of 16 rows finish as soon as 256 tiles of 8 and read Q and K
  // half as often (measured: 1-3% faster).
  const long heads = (long)B * H;
  // bf16 inputs with tiles of 16, 32 or 64 rows: the split-role kernel
  // (tree_verify_ws.hip) with one state wave per 16 rows
  if constexpr (std::is_same<T, bf16_t>::value) {
    int sw = 0;
    if (heads * ((dv + 63) / 64) >= 256) sw = 4;
    else if (heads * ((dv + 31) / 32) >= 256) sw = 2;
    else if (heads * ((dv + 15) / 16) >= 128) sw = 1;
    if (sw)
      return launch_tree_ws(sw, B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                            mask_out, dev_status, da.prev_factors, da.Np, da.last,
                            da.commit_status, da.gate, stream);
  }
  if (heads * ((dv + 63) / 64) >= 256)
    return launch_bv<T, 64>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                            mask_out, dev_status, da, dtype, stream);
  if (heads * ((dv + 31) / 32) >= 256)
    return launch_bv<T, 32>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                            mask_out, dev_status, da, dtype, stream);
  if (heads * ((dv + 15) / 16) >= 128)
    return launch_bv<T, 16>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                            mask_out, dev_status, da, dtype, stream);
  return launch_bv<T, 8>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out, rec,
                         mask_out, dev_status, da, dtype, stream);
}

hipError_t launch_tree_verify(int B, int N, int H, int dk, int dv, int dtype, float* S0,
                              const int32_t* parents, const void* q, const void* k,
                              const void* v, const float* beta, const float* g, float scale,
                              float* out, void* factors, void* workspace, uint64_t* mask_out,
                              int32_t* dev_status, const void* prev_factors, int Np,
                              const int32_t* last, int32_t* commit_status, const float* gate,
                              int ldg, void* Y, hipStream_t stream) {
  (void)workspace;
  const DelayArgs da{prev_factors, Np, last, commit_status,
                     GateArgs{gate, ldg, static_cast<bf16_t*>(Y)}};
  if (dtype == GDN_BF16)
    return launch_tree_verify_t<bf16_t>(
        B, N, H, dk, dv, S0, parents, static_cast<const bf16_t*>(q),
        static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), beta, g, scale, out,
        factors, mask_out, dev_status, da, stream, dtype);
  return launch_tree_verify_t<float>(B, N, H, dk, dv, S0, parents, static_cast<const float*>(q),
                                     static_cast<const float*>(k), static_cast<const float*>(v),
                                     beta, g, scale, out, factors, mask_out, dev_status, da,
                                     stream, dtype);
}

}  // namespace gdn
