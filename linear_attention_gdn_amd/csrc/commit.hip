// Accepted-path commit from the factor record (gfx950).
//
// SpecLA review, "Core claim" and Figure 7 caption (paper Section 5): the
// accepted state is rebuilt from the small per-node factors buffered during
// verification, with no state snapshots and no token replay.  Unrolling
// S_t = alpha_t S_{p(t)} + u'_t k_t^T along the accepted root path p_1..p_n
// gives the rank-n update
//     S_new = e^{G_{p_n}} S0 + sum_i e^{G_{p_n} - G_{p_i}} u'_{p_i} k_{p_i}^T,
// applied here in place while the state streams through once (read + write).
//
// Mapping: CPT = dk/4 threads cover one state row with float4 chunks; the
// 256-thread workgroup processes RG = min(256/CPT, 16) rows at a time and J
// such row groups (rows_per_tile = RG*J <= 64).  Everything that does not
// depend on last_accepted (the state tile, the record's masks, G and u' for
// the tile's rows, and for N <= 16 the k chunks of every node) is loaded in
// one round before the path is known, so the kernel pays one memory round
// trip before it can stream the update.
#include "gdn_common.h"

namespace gdn {

__host__ __device__ inline int commit_row_group(int dk) {
  const int rg = 1024 / dk;  // 256 threads / (dk / 4) chunks per row
  return rg < 16 ? rg : 16;
}

constexpr int kPreloadNodes = 16;

template <typename T, int J, bool PRE>
__global__ __launch_bounds__(256) void commit_kernel(
    int N, int H, int dk, int dv, int ntiles, float* __restrict__ S, Record<T> rec,
    const int32_t* __restrict__ last_accepted, int32_t* __restrict__ path_out,
    int32_t* __restrict__ path_len_out, int32_t* __restrict__ dev_status) {
  __shared__ int plist[kMaxNodes];
  __shared__ uint64_t smask[kMaxNodes];
  __shared__ float sG[kMaxNodes];
  __shared__ float ecoef[kMaxNodes];
  __shared__ float su[kMaxNodes][16 * J];

  const int tid = threadIdx.x;
  const int tile = blockIdx.x % ntiles;
  const int bh = blockIdx.x / ntiles;
  const int b = bh / H;
  const int h = bh % H;
  const int CPT = dk / 4;
  const int RG = commit_row_group(dk);
  const int rows_per_tile = RG * J;
  const int r0 = tile * rows_per_tile;
  const bool reporter = (h == 0 && tile == 0);
  const int cc = tid % CPT;
  const int rg = tid / CPT;
  const bool active = rg < RG;

  // ---- one round of independent loads (unconditional, clamped, masked).
  // Every global load is issued before the first LDS write: consuming any
  // load waits for all loads issued before it.
  const int last = last_accepted[b];
  const int tcl = clampi(tid, N - 1);
  const uint64_t ml = rec.mask[(size_t)b * N + tcl];
  const float gl = rec.G[(size_t)bh * N + tcl];
  constexpr int UB = (kMaxNodes * 16 * J + 255) / 256;  // u' values per thread, at most
  const int utotal = N * rows_per_tile;
  float ub[UB];
#pragma unroll
  for (int x = 0; x < UB; ++x) {
    const int idx = clampi(tid + 256 * x, utotal - 1);
    const int r = clampi(r0 + idx % rows_per_tile, dv - 1);
    ub[x] = rec.up[((size_t)bh * N + idx / rows_per_tile) * dv + r];
  }
  float* Sb = S + (size_t)bh * dv * dk;
  const int ccl = active ? cc : 0;
  f32x4 acc[J];
  bool ok[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int row = r0 + rg + RG * j;
    ok[j] = active && row < dv;
    acc[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (size_t)clampi(row, dv - 1) * dk + 4 * ccl));
  }
  const T* Kb = rec.K + (size_t)bh * N * dk + 4 * ccl;
  typename Raw4<T>::type kpre[PRE ? kPreloadNodes : 1];
  if (PRE) {
#pragma unroll
    for (int t = 0; t < kPreloadNodes; ++t) kpre[t] = raw4(Kb + (size_t)clampi(t, N - 1) * dk);
  }
  if (tid < N) {
    smask[tid] = ml;
    sG[tid] = gl;
  }
#pragma unroll
  for (int x = 0; x < UB; ++x) {
    const int idx = tid + 256 * x;
    if (idx < utotal)
      su[idx / rows_per_tile][idx % rows_per_tile] = r0 + idx % rows_per_tile < dv ? ub[x] : 0.f;
  }
  __syncthreads();

  // ---- the accepted path
  if (last == -1) {
    if (reporter) {
      if (tid < N && path_out) path_out[(size_t)b * N + tid] = -1;
      if (tid == 0) {
        if (path_len_out) path_len_out[b] = 0;
        if (dev_status) dev_status[b] = GDN_OK;
      }
    }
    return;
  }
  const uint64_t valid_bits = N >= 64 ? ~0ull : ((1ull << N) - 1ull);
  const bool in_range = last >= 0 && last < N;
  const uint64_t m = in_range ? (smask[in_range ? last : 0] & valid_bits) : 0ull;
  // Out-of-range index, or a record whose topology was rejected (mask zero,
  // so the node's own bit is missing).
  if (!in_range || ((m >> last) & 1ull) == 0ull) {
    if (reporter) {
      if (tid < N && path_out) path_out[(size_t)b * N + tid] = -1;
      if (tid == 0) {
        if (path_len_out) path_len_out[b] = -1;
        if (dev_status) dev_status[b] = GDN_ERR_TOPOLOGY;
      }
    }
    return;
  }
  const int n = __popcll(m);
  const float Glast = sG[last];
  if (tid < kMaxNodes && ((m >> tid) & 1ull)) {
    plist[__popcll(m & ((1ull << tid) - 1ull))] = tid;
    ecoef[tid] = expf(Glast - sG[tid]);
  }
  __syncthreads();
  if (reporter) {
    if (tid < N && path_out) path_out[(size_t)b * N + tid] = tid < n ? plist[tid] : -1;
    if (tid == 0) {
      if (path_len_out) path_len_out[b] = n;
      if (dev_status) dev_status[b] = GDN_OK;
    }
  }
  if (!active) return;

  // ---- stream: S_new = e^{G_last} S + sum_i coef_i u'_{p_i}[row] k_{p_i}
  const float s0 = expf(Glast);
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = mask4(acc[j], ok[j]) * s0;
  if (PRE) {
#pragma unroll
    for (int t = 0; t < kPreloadNodes; ++t) {
      if ((m >> t) & 1ull) {  // uniform
        const f32x4 kc = widen4(kpre[t]);
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const float c = ecoef[t] * su[t][rg + RG * j];
          acc[j].x = fmaf(c, kc.x, acc[j].x);
          acc[j].y = fmaf(c, kc.y, acc[j].y);
          acc[j].z = fmaf(c, kc.z, acc[j].z);
          acc[j].w = fmaf(c, kc.w, acc[j].w);
        }
      }
    }
  } else {
    for (int i = 0; i < n; ++i) {
      const int p = plist[i];
      const f32x4 kc = load4(Kb + (size_t)p * dk);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const float c = ecoef[p] * su[p][rg + RG * j];
        acc[j].x = fmaf(c, kc.x, acc[j].x);
        acc[j].y = fmaf(c, kc.y, acc[j].y);
        acc[j].z = fmaf(c, kc.z, acc[j].z);
        acc[j].w = fmaf(c, kc.w, acc[j].w);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int row = r0 + rg + RG * j;
    if (ok[j]) __builtin_nontemporal_store(acc[j], reinterpret_cast<f32x4*>(Sb + (size_t)row * dk + 4 * cc));
  }
}

template <typename T, int J>
hipError_t launch_commit_j(int B, int N, int H, int dk, int dv, float* S, const Record<T>& rec,
                           const int32_t* last, int32_t* path_out, int32_t* path_len,
                           int32_t* dev_status, hipStream_t stream) {
  const int RG = commit_row_group(dk);
  const int rows_per_tile = RG * J;
  const int ntiles = (dv + rows_per_tile - 1) / rows_per_tile;
  const long grid = (long)B * H * ntiles;
  if (N <= kPreloadNodes)
    hipLaunchKernelGGL((commit_kernel<T, J, true>), dim3((unsigned)grid), dim3(256), 0, stream,
                       N, H, dk, dv, ntiles, S, rec, last, path_out, path_len, dev_status);
  else
    hipLaunchKernelGGL((commit_kernel<T, J, false>), dim3((unsigned)grid), dim3(256), 0, stream,
                       N, H, dk, dv, ntiles, S, rec, last, path_out, path_len, dev_status);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_commit_t(int B, int N, int H, int dk, int dv, float* S, const void* factors,
                           const RecordLayout& L, const int32_t* last, int32_t* path_out,
                           int32_t* path_len, int32_t* dev_status, hipStream_t stream) {
  Record<T> rec = record_views<T>(const_cast<void*>(factors), L);
  // Enough workgroups to cover the chip: fewer rows per tile for small batches.
  const int RG = commit_row_group(dk);
  const long wg1 = (long)B * H * ((dv + RG - 1) / RG);
  if (wg1 >= 4096)
    return launch_commit_j<T, 4>(B, N, H, dk, dv, S, rec, last, path_out, path_len, dev_status,
                                 stream);
  if (wg1 >= 1024)
    return launch_commit_j<T, 2>(B, N, H, dk, dv, S, rec, last, path_out, path_len, dev_status,
                                 stream);
  return launch_commit_j<T, 1>(B, N, H, dk, dv, S, rec, last, path_out, path_len, dev_status,
                               stream);
}

hipError_t launch_commit(int B, int N, int H, int dk, int dv, int dtype, float* S,
                         const void* factors, const int32_t* last, int32_t* path_out,
                         int32_t* path_len, int32_t* dev_status, hipStream_t stream) {
  const RecordLayout L = record_layout(B, N, H, dk, dv, dtype);
  if (dtype == GDN_BF16)
    return launch_commit_t<bf16_t>(B, N, H, dk, dv, S, factors, L, last, path_out, path_len,
                                   dev_status, stream);
  return launch_commit_t<float>(B, N, H, dk, dv, S, factors, L, last, path_out, path_len,
                                dev_status, stream);
}

}  // namespace gdn
