// Serial chain verification with V-dimension tiling (gfx950).
//
// SpecLA review, "What carries the argument" and Figure 3 caption (paper
// Section 4.1): verifying a chain keeps the recurrent state on chip across
// the candidate tokens, and because the state is too large for on-chip
// memory it is tiled along the value dimension.  Rows of S evolve
// independently under the recurrence, so each workgroup owns a tile of rows
// for the whole chain and never writes S0 back.
//
// One wave64 per workgroup.  16 lanes cover one state row (lane s holds
// columns 64*m + 4*s + e, m < dk/64, e < 4, so each 16-lane group reads
// 256 contiguous bytes per load and dot products reduce across 16 lanes);
// four rows are in flight per wave and RPL row groups per lane.  Everything
// the serial loop needs (k, q as FP32, v for the tile's rows, beta, alpha) is
// staged in LDS with one round of loads that overlaps the state-tile load,
// so the N serial steps touch only registers and LDS.
#include "gdn_common.h"

namespace gdn {

template <typename T, int RPL>
__global__ __launch_bounds__(64) void chain_verify_kernel(
    int N, int H, int dk, int dv, int ntiles, const float* __restrict__ S0,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ g, float scale,
    float* __restrict__ out, Record<T> rec) {
  constexpr int MC = kMaxDim / 64;
  constexpr int ROWS = 4 * RPL;
  // dynamic LDS: k, q as loaded [N][dk], v [N][ROWS], alpha, beta, g [N]
  using R4 = typename Raw4<T>::type;
  extern __shared__ f32x4 lds4[];
  const int cpr = dk / 4;
  R4* sk = reinterpret_cast<R4*>(lds4);
  R4* sq = sk + N * cpr;
  float* sv = reinterpret_cast<float*>(sq + N * cpr);
  float* salpha = sv + N * ROWS;
  float* sbeta = salpha + N;
  float* sG = sbeta + N;

  const int lane = threadIdx.x;
  const int rw = lane >> 4;
  const int s = lane & 15;
  const int tile = blockIdx.x % ntiles;
  const int bh = blockIdx.x / ntiles;
  const int h = bh % H;
  const int b = bh / H;
  const int r0 = tile * ROWS;

  // ---- every global load first (unconditional, clamped), then the LDS writes:
  // a consumer of any load waits for all loads issued before it.
  constexpr int BATCH = 8;
  constexpr int VB = kMaxNodes * ROWS / 64;
  const size_t nhl = ((size_t)b * N + clampi(lane, N - 1)) * H + h;
  const float gl = g[nhl];
  const float bl = beta[nhl];
  T vb[VB];
#pragma unroll
  for (int x = 0; x < VB; ++x) {
    const int idx = clampi(lane + 64 * x, N * ROWS - 1);
    const int r = clampi(r0 + idx % ROWS, dv - 1);
    vb[x] = v[(((size_t)b * N + idx / ROWS) * H + h) * dv + r];
  }
  int row[RPL];
  bool rok[RPL];
  f32x4 Sx[RPL][MC];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    row[i] = r0 + 4 * i + rw;
    rok[i] = row[i] < dv;
    const float* rp = S0 + ((size_t)bh * dv + clampi(row[i], dv - 1)) * dk;
#pragma unroll
    for (int m = 0; m < MC; ++m) Sx[i][m] = load4(rp + clampi(64 * m + 4 * s, dk - 4));
  }
  // k and q rows: the first batch is straight-line code (a loop here would make
  // the compiler drain every outstanding load at its header); larger drafts
  // continue in a loop.
  auto stage = [&](int base) {
    R4 kb[BATCH], qb[BATCH];
#pragma unroll
    for (int x = 0; x < BATCH; ++x) {
      const int idx = clampi(base + 64 * x, N * cpr - 1);
      const size_t off = (((size_t)b * N + idx / cpr) * H + h) * dk + 4 * (idx % cpr);
      kb[x] = raw4(k + off);
      qb[x] = raw4(q + off);
    }
#pragma unroll
    for (int x = 0; x < BATCH; ++x) {
      const int idx = base + 64 * x;
      if (idx < N * cpr) {
        sk[idx] = kb[x];
        sq[idx] = qb[x];
      }
    }
  };
  stage(lane);
  for (int base = lane + 64 * BATCH; base < N * cpr; base += 64 * BATCH) stage(base);
#pragma unroll
  for (int x = 0; x < VB; ++x) {
    const int idx = lane + 64 * x;
    if (idx < N * ROWS) sv[idx] = (r0 + idx % ROWS < dv) ? widen1(vb[x]) : 0.f;
  }
  if (lane < N) {
    salpha[lane] = expf(gl);
    sbeta[lane] = bl;
    sG[lane] = gl;
  }
  float S[RPL][MC][4];
#pragma unroll
  for (int i = 0; i < RPL; ++i)
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const f32x4 x = mask4(Sx[i][m], rok[i] && 64 * m + 4 * s < dk);
      S[i][m][0] = x.x;
      S[i][m][1] = x.y;
      S[i][m][2] = x.z;
      S[i][m][3] = x.w;
    }
  __syncthreads();

  // k_t, q_t (widened) for step t; the next step's are read from LDS while
  // the current step computes.
  auto fetch = [&](int t, float (&kf)[MC][4], float (&qf)[MC][4]) {
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const int cidx = t * cpr + clampi(16 * m + s, cpr - 1);
      const bool okc = 64 * m + 4 * s < dk;
      const f32x4 kx = mask4(widen4(sk[cidx]), okc);
      const f32x4 qx = mask4(widen4(sq[cidx]), okc);
      kf[m][0] = kx.x; kf[m][1] = kx.y; kf[m][2] = kx.z; kf[m][3] = kx.w;
      qf[m][0] = qx.x; qf[m][1] = qx.y; qf[m][2] = qx.z; qf[m][3] = qx.w;
    }
  };
  float kf[MC][4], qf[MC][4];
  fetch(0, kf, qf);
  for (int t = 0; t < N; ++t) {
    float kn[MC][4], qn[MC][4];
    fetch(clampi(t + 1, N - 1), kn, qn);
    const float be = sbeta[t];
    const float al = salpha[t];
    float vt[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) vt[i] = sv[t * ROWS + 4 * i + rw];

    // partial dot products, two accumulators per value for a shorter chain:
    // red[0] = k.q, red[1+2i] = S_i.k, red[2+2i] = S_i.q
    float red[1 + 2 * RPL], red2[1 + 2 * RPL];
#pragma unroll
    for (int x = 0; x < 1 + 2 * RPL; ++x) red[x] = red2[x] = 0.f;
#pragma unroll
    for (int m = 0; m < MC; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float* r = (e & 1) ? red2 : red;
        r[0] = fmaf(kf[m][e], qf[m][e], r[0]);
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
          r[1 + 2 * i] = fmaf(S[i][m][e], kf[m][e], r[1 + 2 * i]);
          r[2 + 2 * i] = fmaf(S[i][m][e], qf[m][e], r[2 + 2 * i]);
        }
      }
#pragma unroll
    for (int x = 0; x < 1 + 2 * RPL; ++x) red[x] = row16_sum(red[x] + red2[x]);
    const float kq = red[0];

#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const float u = be * (vt[i] - al * red[1 + 2 * i]);
      const float o = scale * fmaf(kq, u, al * red[2 + 2 * i]);
#pragma unroll
      for (int m = 0; m < MC; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[i][m][e] = fmaf(u, kf[m][e], al * S[i][m][e]);
      if (s == 0 && rok[i]) {
        const size_t nh = ((size_t)b * N + t) * H + h;
        out[nh * dv + row[i]] = o;
        rec.up[((size_t)bh * N + t) * dv + row[i]] = u;
      }
    }
#pragma unroll
    for (int m = 0; m < MC; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[m][e] = kn[m][e];
        qf[m][e] = qn[m][e];
      }
  }

  // factor record: G (chain prefix sums), k copy, parents, masks
  if (tile == 0) {
    if (lane == 0) {
      float G = 0.f;
      for (int t = 0; t < N; ++t) {
        G += sG[t];
        rec.G[(size_t)bh * N + t] = G;
      }
    }
    for (int idx = lane; idx < N * cpr; idx += 64)  // from the staged rows in LDS
      *reinterpret_cast<R4*>(rec.K + ((size_t)bh * N + idx / cpr) * dk + 4 * (idx % cpr)) = sk[idx];
    if (h == 0 && lane < N) {
      rec.parents[(size_t)b * N + lane] = lane - 1;
      rec.mask[(size_t)b * N + lane] = lane >= 63 ? ~0ull : ((1ull << (lane + 1)) - 1ull);
    }
  }
}

template <typename T>
hipError_t launch_chain_verify_t(int B, int N, int H, int dk, int dv, const float* S0,
                                 const void* q, const void* k, const void* v,
                                 const float* beta, const float* g, float scale, float* out,
                                 void* factors, const RecordLayout& L, hipStream_t stream) {
  Record<T> rec = record_views<T>(factors, L);
  constexpr int RPL = 2;
  const int rows = 4 * RPL;
  const int ntiles = (dv + rows - 1) / rows;
  const long grid = (long)B * H * ntiles;
  const size_t lds = (size_t)N * dk * sizeof(T) * 2 + (size_t)N * rows * 4 + (size_t)N * 4 * 3;
  hipLaunchKernelGGL((chain_verify_kernel<T, RPL>), dim3((unsigned)grid), dim3(64), lds, stream,
                     N, H, dk, dv, ntiles, S0, static_cast<const T*>(q),
                     static_cast<const T*>(k), static_cast<const T*>(v), beta, g, scale, out,
                     rec);
  return hipGetLastError();
}

hipError_t launch_chain_verify(int B, int N, int H, int dk, int dv, int dtype, const float* S0,
                               const void* q, const void* k, const void* v, const float* beta,
                               const float* g, float scale, float* out, void* factors,
                               hipStream_t stream) {
  const RecordLayout L = record_layout(B, N, H, dk, dv, dtype);
  if (dtype == GDN_BF16)
    return launch_chain_verify_t<bf16_t>(B, N, H, dk, dv, S0, q, k, v, beta, g, scale, out,
                                         factors, L, stream);
  return launch_chain_verify_t<float>(B, N, H, dk, dv, S0, q, k, v, beta, g, scale, out,
                                      factors, L, stream);
}

}  // namespace gdn
