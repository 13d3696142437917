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
//   3. the window nodes compacted into a list (a block prefix sum), then each
//      window node's rank = the number of window nodes before it in
//      (q descending, index ascending), read from LDS;
//   4. kept = window and rank < T; new numbers by a second prefix sum.
#include "gdn_common.h"

namespace gdn {

constexpr int kPruneThreads = 256;
constexpr int kPruneMax = 1024;
constexpr int kPrunePer = kPruneMax / kPruneThreads;

// Exclusive prefix sum of one count per thread over the workgroup; returns
// this thread's offset and leaves the total in *total (both in every thread).
__device__ inline int block_exclusive_scan(int x, int* swave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) swave[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kPruneThreads / 64; ++w) {
    const int c = swave[w];
    if (w < wave) before += c;
    all += c;
  }
  __syncthreads();  // swave may be reused
  *total = all;
  return before + incl - x;
}

__global__ __launch_bounds__(kPruneThreads) void prune_kernel(
    int M, int T, float tau, const int32_t* __restrict__ parents,
    const float* __restrict__ conf, int32_t* __restrict__ kept, int32_t* __restrict__ new_parents,
    int32_t* __restrict__ count, int32_t* __restrict__ dev_status) {
  __shared__ float sq[kPruneMax];
  __shared__ int sp[kPruneMax];
  __shared__ int snew[kPruneMax];    // new number of a kept node, -1 otherwise
  __shared__ int swin[kPruneMax];    // window nodes, ascending
  __shared__ float swq[kPruneMax];   // their confidences
  __shared__ int swave[kPruneThreads / 64];
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
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, d));
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
  int inw[kPrunePer], nloc = 0;
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    const int t = kPrunePer * tid + i;
    inw[i] = (t < M && q[i] >= thr) ? 1 : 0;
    nloc += inw[i];
  }
  int W;
  int off = block_exclusive_scan(nloc, swave, &W);
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    if (inw[i]) {
      swin[off] = kPrunePer * tid + i;
      swq[off] = q[i];
      ++off;
    }
  }
  __syncthreads();
  int keep[kPrunePer], nk = 0;
#pragma unroll
  for (int i = 0; i < kPrunePer; ++i) {
    const int t = kPrunePer * tid + i;
    keep[i] = 0;
    if (inw[i]) {
      int rank = 0;
      for (int j = 0; j < W; ++j) {  // uniform bound
        const float qj = swq[j];
        const int tj = swin[j];
        rank += (qj > q[i] || (qj == q[i] && tj < t)) ? 1 : 0;
      }
      keep[i] = rank < T ? 1 : 0;
    }
    nk += keep[i];
  }
  // 4. renumbering
  int K;
  int nn = block_exclusive_scan(nk, swave, &K);
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
