// Confidence-guided draft pruning (gfx950).
//
// SpecLA review, Figures, Figure 8 caption (and the Axiom & Free-Parameter
// Ledger's tree margin tau_tree and draft budget): before verification the
// candidate tree is cut to the nodes whose confidence lies within tau of the
// best confidence q*, which is ancestor-closed because a node's confidence
// never exceeds its parent's, and a budget T then truncates that selection.
// Here the budget keeps the first T window nodes in the order (q descending,
// index ascending), which keeps every parent before its children, and the
// kept nodes leave in their original (topological) order, renumbered, with
// their parents mapped: a draft the verifiers take as it is.
//
// One workgroup (256 threads) per sequence, M <= 1024 candidates, four per
// thread, all in LDS:
//   1. checks: -1 <= p[t] < t, q[t] not NaN, q[t] <= q[p[t]];
//   2. q* by a block reduction; the threshold q* - tau in FP32;
//   3. the window nodes compacted into a list (a prefix count by ballots),
//      then each window node's rank = the number of window nodes before it
//      in (q descending, index ascending), one list entry per thread, from
//      one pass over the list in LDS (four entries per read);
//   4. kept = window and rank < T; new numbers by a second prefix count.
#include "gdn_common.h"

namespace gdn {

constexpr int kPruneThreads = 256;
constexpr int kPruneMax = 1024;
constexpr int kPrunePer = kPruneMax / kPruneThreads;
static_assert(kPrunePer == 4, "four candidates per thread");

// Exclusive prefix count of per-thread flags over the workgroup in node
// order (thread tid holds nodes 4 tid .. 4 tid + 3): within a wave one ballot
// per flag slot and a popcount of the lanes below, across the four waves one
// LDS round (swave: this scan's own four entries).  Returns the number of set
// flags before this thread's nodes and leaves the total in *total.
__device__ inline int block_flag_scan(const int (&f)[kPrunePer], int* swave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  int before = 0, cnt = 0;
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    const uint64_t m = __ballot(f[i] != 0);
    before += __popcll(m & below);
    cnt += __popcll(m);
  }
  if (lane == 0) swave[wave] = cnt;
  __syncthreads();
  int all = 0;
#pragma unroll
  for (int w = 0; w < kPruneThreads / 64; ++w) {
    const int c = swave[w];
    if (w < wave) before += c;
    all += c;
  }
  *total = all;
  return before;
}

// Maximum over the wave into every lane: DPP within rows of 16, then the
// row and half exchanges on the VALU.
__device__ inline float wave64_max(float x) {
  x = fmaxf(x, dpp_f32<0x128>(x));  // row_ror:8
  x = fmaxf(x, dpp_f32<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]
  unsigned a = __builtin_bit_cast(unsigned, x), c;
  asm("" : "=v"(c) : "0"(a));
  const auto r = __builtin_amdgcn_permlane16_swap(a, c, false, false);
  x = fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
  a = __builtin_bit_cast(unsigned, x);
  asm("" : "=v"(c) : "0"(a));
  const auto r2 = __builtin_amdgcn_permlane32_swap(a, c, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r2[0]), __builtin_bit_cast(float, (unsigned)r2[1]));
}

__global__ __launch_bounds__(kPruneThreads) void prune_kernel(
    int M, int T, float tau, const int32_t* __restrict__ parents,
    const float* __restrict__ conf, int32_t* __restrict__ kept, int32_t* __restrict__ new_parents,
    int32_t* __restrict__ count, int32_t* __restrict__ dev_status) {
  __shared__ float sq[kPruneMax];
  __shared__ int sp[kPruneMax];
  __shared__ int snew[kPruneMax];    // new number of a kept node, -1 otherwise
  __shared__ __attribute__((aligned(16))) int swin[kPruneMax];   // window nodes, ascending
  __shared__ __attribute__((aligned(16))) float swq[kPruneMax];  // their confidences
  __shared__ int swave[kPruneThreads / 64], swave2[kPruneThreads / 64];
  __shared__ int skeep[kPruneMax];   // window nodes: 1 if within the budget
  __shared__ float sred[kPruneThreads / 64];
  __shared__ int sbad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (tid == 0) sbad = 0;
  // thread tid holds nodes kPrunePer * tid .. + kPrunePer - 1
  int p[kPrunePer];
  float q[kPrunePer];
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    const int t = kPrunePer * tid + i;
    const int tc = clampi(t, M - 1);
    p[i] = parents[(size_t)b * M + tc];
    q[i] = conf[(size_t)b * M + tc];
    if (t < M) {
      sq[t] = q[i];
      sp[t] = p[i];
    }
  }
  __syncthreads();
  // 1. preconditions
  bool bad = false;
  float qmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    const int t = kPrunePer * tid + i;
    if (t < M) {
      const bool topo = p[i] >= -1 && p[i] < t;
      bad |= !topo || q[i] != q[i] || (topo && p[i] >= 0 && q[i] > sq[p[i]]);
      qmax = fmaxf(qmax, q[i]);
    }
  }
  if (bad) sbad = 1;
  // 2. q* and the FP32 threshold
  qmax = wave64_max(qmax);
  if (lane == 0) sred[wave] = qmax;
  __syncthreads();
  float qs = sred[0];
#pragma unroll
  for (int w = 1; w < kPruneThreads / 64; ++w) qs = fmaxf(qs, sred[w]);
  const float thr = qs - tau;
  if (sbad) {  // uniform
    if (tid == 0) {
      count[b] = -1;
      if (dev_status) dev_status[b] = GDN_ERR_TOPOLOGY;
    }
    for (int i = tid; i < T; i += kPruneThreads) {
      kept[(size_t)b * T + i] = -1;
      new_parents[(size_t)b * T + i] = -1;
    }
    return;
  }
  // 3. the window, compacted in ascending order, then ranks within it
  int inw[kPrunePer];
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    const int t = kPrunePer * tid + i;
    inw[i] = (t < M && q[i] >= thr) ? 1 : 0;
  }
  int W;
  int off = block_flag_scan(inw, swave, &W);
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    if (inw[i]) {
      swin[off] = kPrunePer * tid + i;
      swq[off] = q[i];
      ++off;
    }
  }
  // pad the list to a multiple of four with entries that rank before no
  // node: confidence -inf, index past every node
  const int W4 = (W + 3) & ~3;
  if (tid < W4 - W) {
    swq[W + tid] = -INFINITY;
    swin[W + tid] = kPruneMax;
  }
  __syncthreads();
  // rank of each window node among the window in (q descending, index
  // ascending), one list entry per thread: one pass over the list, four
  // entries per 16-byte read
  for (int x = tid; x < W; x += kPruneThreads) {
    const float qx = swq[x];
    const int tx = swin[x];
    int rank = 0;
    for (int j = 0; j < W4; j += 4) {
      const f32x4 qv = *reinterpret_cast<const f32x4*>(&swq[j]);
      const int4 tv = *reinterpret_cast<const int4*>(&swin[j]);
      rank += (qv.x > qx || (qv.x == qx && tv.x < tx)) ? 1 : 0;
      rank += (qv.y > qx || (qv.y == qx && tv.y < tx)) ? 1 : 0;
      rank += (qv.z > qx || (qv.z == qx && tv.z < tx)) ? 1 : 0;
      rank += (qv.w > qx || (qv.w == qx && tv.w < tx)) ? 1 : 0;
    }
    skeep[tx] = rank < T ? 1 : 0;
  }
  __syncthreads();
  int keep[kPrunePer];
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) keep[i] = inw[i] ? skeep[kPrunePer * tid + i] : 0;
  // 4. renumbering
  int K;
  int nn = block_flag_scan(keep, swave2, &K);
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    const int t = kPrunePer * tid + i;
    if (t < M) snew[t] = keep[i] ? nn : -1;
    nn += keep[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    const int t = kPrunePer * tid + i;
    if (t < M && keep[i]) {
      const int n = snew[t];
      kept[(size_t)b * T + n] = t;
      new_parents[(size_t)b * T + n] = p[i] >= 0 ? snew[p[i]] : -1;
    }
  }
  for (int i = K + tid; i < T; i += kPruneThreads) {
    kept[(size_t)b * T + i] = -1;
    new_parents[(size_t)b * T + i] = -1;
  }
  if (tid == 0) {
    count[b] = K;
    if (dev_status) dev_status[b] = GDN_OK;
  }
}

hipError_t launch_prune(int B, int M, int T, float tau, const int32_t* parents, const float* conf,
                        int32_t* kept, int32_t* new_parents, int32_t* count, int32_t* dev_status,
                        hipStream_t stream) {
  hipLaunchKernelGGL(prune_kernel, dim3((unsigned)B), dim3(kPruneThreads), 0, stream, M, T, tau,
                     parents, conf, kept, new_parents, count, dev_status);
  return hipGetLastError();
}

}  // namespace gdn
