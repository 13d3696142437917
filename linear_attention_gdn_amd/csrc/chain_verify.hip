// Serial chain verification with V-dimension tiling (gfx950).
//
// SpecLA review, "What carries the argument" and Figure 3 caption (paper
// Section 4.1): verifying a chain keeps the recurrent state on chip across
// the candidate tokens, and because the state is too large for on-chip
// memory it is tiled along the value dimension.  Rows of S evolve
// independently under the recurrence, so each workgroup owns a tile of rows
// for the whole chain and never writes S0 back.
//
// Per step t and state row r (alpha_t = e^{g_t}):
//     y_k = S_r . k_t,  y_q = S_r . q_t,  u'_t[r] = beta_t (v_t[r] - alpha_t y_k)
//     o_t[r] = scale (alpha_t y_q + (k_t . q_t) u'_t[r])
//     S_r <- alpha_t S_r + u'_t[r] k_t
//
// Mapping: 256 threads = 4 waves; each half-wave (32 lanes) owns one state row
// and lane s of it holds columns 128*m + 4*s + e (m < dk/128, e < 4), so a row
// is read as 512-byte coalesced runs and dot products reduce over 32 lanes
// with DPP row rotations plus one v_permlane16_swap.  A workgroup owns 8 rows,
// one per SIMD pair of half-waves, so all four SIMDs of a CU run the serial
// loop.  Everything the loop needs (k, q as loaded, v of the 8 rows, alpha,
// beta) is staged in LDS by one round of loads that overlaps the state-tile
// load; the loop then touches only registers and LDS, reading the next
// step's k and q while the current step computes.
//
// Delayed commit (review: Referee Report summary, mechanism (ii); Figure 7
// caption, right side): with DLY the same workgroup first applies the
// previous draft's accepted path to its state tile, using the previous factor
// record staged in LDS in the same round of loads, writes the tile back, and
// then verifies the new chain from the updated registers.  The update repeats
// the commit kernel's operations in the same order (scale by e^{G_last}, then
// one fused multiply-add per path node in node order), so the result is
// bitwise that of commit followed by verify.
#include "gdn_common.h"

namespace gdn {

constexpr int kChainRows = 8;  // state rows per workgroup (one per half-wave)

template <typename T, bool DLY>
__global__ __launch_bounds__(256) void chain_verify_kernel(
    int N, int H, int dk, int dv, int ntiles, float* __restrict__ S0,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ g, float scale,
    float* __restrict__ out, Record<T> rec, Record<T> prev, int Np,
    const int32_t* __restrict__ last_acc, int32_t* __restrict__ dev_status) {
  constexpr int MC = kMaxDim / 128;  // float4 chunks per lane
  using R4 = typename Raw4<T>::type;
  // dynamic LDS: k, q as loaded [N][dk], v [N][8], alpha, beta, g [N];
  // with DLY also the previous record's k [Np][dk], u' of the tile's rows
  // [Np][8] and the commit coefficients e^{G_last - G_i} [Np]
  extern __shared__ f32x4 lds4[];
  const int cpr = dk / 4;
  R4* sk = reinterpret_cast<R4*>(lds4);
  R4* sq = sk + N * cpr;
  R4* skp = sq + N * cpr;
  float* sv = reinterpret_cast<float*>(skp + (DLY ? Np * cpr : 0));
  float* salpha = sv + N * kChainRows;
  float* sbeta = salpha + N;
  float* sG = sbeta + N;
  float* sup = sG + N;
  float* sGp = sup + (DLY ? Np * kChainRows : 0);

  const int tid = threadIdx.x;
  const int s = tid & 31;             // lane within the row's half-wave
  const int rl = tid >> 5;            // row within the tile (0..7)
  const int tile = blockIdx.x % ntiles;
  const int bh = blockIdx.x / ntiles;
  const int h = bh % H;
  const int b = bh / H;
  const int r0 = tile * kChainRows;
  const int row = r0 + rl;
  const bool rok = row < dv;

  // ---- every global load first (unconditional, clamped), then the LDS writes
  const size_t nhl = ((size_t)b * N + clampi(tid, N - 1)) * H + h;
  const float gl = g[nhl];
  const float bl = beta[nhl];
  constexpr int VB = kMaxNodes * kChainRows / 256;  // v values per thread, at most
  T vb[VB];
#pragma unroll
  for (int x = 0; x < VB; ++x) {
    const int idx = clampi(tid + 256 * x, N * kChainRows - 1);
    const int r = clampi(r0 + idx % kChainRows, dv - 1);
    vb[x] = v[(((size_t)b * N + idx / kChainRows) * H + h) * dv + r];
  }
  f32x4 Sx[MC];
  {
    const float* rp = S0 + ((size_t)bh * dv + clampi(row, dv - 1)) * dk;
#pragma unroll
    for (int m = 0; m < MC; ++m) Sx[m] = load4(rp + clampi(128 * m + 4 * s, dk - 4));
  }
  // the previous draft's record (delayed commit): masks, G, u' of this tile's
  // rows and the k rows, none of which depends on last_accepted
  constexpr int BATCH = 4;
  int last = -1;
  uint64_t mlp = 0;
  float glp = 0.f;
  float upb[DLY ? VB : 1];
  R4 kpb[DLY ? BATCH : 1];
  auto prevk_off = [&](int idx) {
    idx = clampi(idx, Np * cpr - 1);
    return ((size_t)bh * Np + idx / cpr) * dk + 4 * (idx % cpr);
  };
  int last_v = -1;
  uint64_t pm_r = 0;   // accepted path of the previous draft (bit i: node i)
  float Glast_r = 0.f;
  if (DLY) {
    last_v = last_acc[b];  // a vector load: it joins this round instead of a later scalar one
    const int tcp = clampi(tid & 63, Np - 1);  // every wave holds node j's mask and G in lane j
    mlp = prev.mask[(size_t)b * Np + tcp];
    glp = prev.G[(size_t)bh * Np + tcp];
#pragma unroll
    for (int x = 0; x < VB; ++x) {
      const int idx = clampi(tid + 256 * x, Np * kChainRows - 1);
      const int r = clampi(r0 + idx % kChainRows, dv - 1);
      upb[x] = prev.up[((size_t)bh * Np + idx / kChainRows) * dv + r];
    }
#pragma unroll
    for (int x = 0; x < BATCH; ++x) kpb[x] = raw4(prev.K + prevk_off(tid + 256 * x));
  }
  // k and q rows: the first batch is straight-line code (a loop here would
  // drain every outstanding load at its header); larger drafts loop.
  auto stage = [&](int base) {
    R4 kb[BATCH], qb[BATCH];
#pragma unroll
    for (int x = 0; x < BATCH; ++x) {
      const int idx = clampi(base + 256 * x, N * cpr - 1);
      const size_t off = (((size_t)b * N + idx / cpr) * H + h) * dk + 4 * (idx % cpr);
      kb[x] = raw4(k + off);
      qb[x] = raw4(q + off);
    }
#pragma unroll
    for (int x = 0; x < BATCH; ++x) {
      const int idx = base + 256 * x;
      if (idx < N * cpr) {
        sk[idx] = kb[x];
        sq[idx] = qb[x];
      }
    }
  };
  stage(tid);
  for (int base = tid + 256 * BATCH; base < N * cpr; base += 256 * BATCH) stage(base);
  if (DLY) {
#pragma unroll
    for (int x = 0; x < BATCH; ++x)
      if (tid + 256 * x < Np * cpr) skp[tid + 256 * x] = kpb[x];
    for (int base = tid + 256 * BATCH; base < Np * cpr; base += 256 * BATCH) {
      R4 kb[BATCH];
#pragma unroll
      for (int x = 0; x < BATCH; ++x) kb[x] = raw4(prev.K + prevk_off(base + 256 * x));
#pragma unroll
      for (int x = 0; x < BATCH; ++x)
        if (base + 256 * x < Np * cpr) skp[base + 256 * x] = kb[x];
    }
  }
#pragma unroll
  for (int x = 0; x < VB; ++x) {
    const int idx = tid + 256 * x;
    if (idx < N * kChainRows) sv[idx] = (r0 + idx % kChainRows < dv) ? widen1(vb[x]) : 0.f;
  }
  if (tid < N) {
    salpha[tid] = expf(gl);
    sbeta[tid] = bl;
    sG[tid] = gl;
  }
  if (DLY) {
    // the accepted path and each node's coefficient e^{G_last - G_i}, one lane
    // per node (the same expression the commit kernel evaluates)
    last = __builtin_amdgcn_readfirstlane(last_v);
    const bool in_rng = last >= 0 && last < Np;
    const int lc = in_rng ? last : 0;
    const uint32_t mlo = __builtin_amdgcn_readlane((uint32_t)mlp, lc);
    const uint32_t mhi = __builtin_amdgcn_readlane((uint32_t)(mlp >> 32), lc);
    const uint64_t valid = Np >= 64 ? ~0ull : ((1ull << Np) - 1ull);
    pm_r = in_rng ? ((((uint64_t)mhi << 32) | mlo) & valid) : 0ull;
    Glast_r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, glp), lc));
    if (tid < Np) sGp[tid] = ((pm_r >> tid) & 1ull) ? expf(Glast_r - glp) : 0.f;
#pragma unroll
    for (int x = 0; x < VB; ++x) {
      const int idx = tid + 256 * x;
      if (idx < Np * kChainRows) sup[idx] = (r0 + idx % kChainRows < dv) ? upb[x] : 0.f;
    }
  }
  float S[MC][4];
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const f32x4 x = mask4(Sx[m], rok && 128 * m + 4 * s < dk);
    S[m][0] = x.x;
    S[m][1] = x.y;
    S[m][2] = x.z;
    S[m][3] = x.w;
  }
  __syncthreads();

  if (DLY) {
    // ---- the previous draft's accepted path: S <- e^{G_last} S + sum c_i u'_i k_i^T
    const uint64_t pm = pm_r;
    const bool okp = last >= 0 && last < Np && ((pm >> last) & 1ull);
    if (dev_status && tile == 0 && h == 0 && tid == 0)
      dev_status[b] = (last == -1 || okp) ? GDN_OK : GDN_ERR_TOPOLOGY;
    if (okp) {  // uniform
      const float s0 = expf(Glast_r);
#pragma unroll
      for (int m = 0; m < MC; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[m][e] = S[m][e] * s0;
      for (int i = 0; i <= last; ++i) {
        if (((pm >> i) & 1ull) == 0ull) continue;  // uniform
        const float c = sGp[i] * sup[i * kChainRows + rl];
#pragma unroll
        for (int m = 0; m < MC; ++m) {
          const f32x4 kc = widen4(skp[i * cpr + clampi(32 * m + s, cpr - 1)]);
          S[m][0] = fmaf(c, kc.x, S[m][0]);
          S[m][1] = fmaf(c, kc.y, S[m][1]);
          S[m][2] = fmaf(c, kc.z, S[m][2]);
          S[m][3] = fmaf(c, kc.w, S[m][3]);
        }
      }
      if (rok) {
        float* wp = S0 + ((size_t)bh * dv + row) * dk;
#pragma unroll
        for (int m = 0; m < MC; ++m)
          if (128 * m + 4 * s < dk)
            *reinterpret_cast<f32x4*>(wp + 128 * m + 4 * s) =
                f32x4{S[m][0], S[m][1], S[m][2], S[m][3]};
      }
    }
  }

  // k_t, q_t (widened) for step t; the next step's are read from LDS while
  // the current step computes.
  auto fetch = [&](int t, float (&kf)[MC][4], float (&qf)[MC][4]) {
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const int cidx = t * cpr + clampi(32 * m + s, cpr - 1);
      const bool okc = 128 * m + 4 * s < dk;
      const f32x4 kx = mask4(widen4(sk[cidx]), okc);
      const f32x4 qx = mask4(widen4(sq[cidx]), okc);
      kf[m][0] = kx.x; kf[m][1] = kx.y; kf[m][2] = kx.z; kf[m][3] = kx.w;
      qf[m][0] = qx.x; qf[m][1] = qx.y; qf[m][2] = qx.z; qf[m][3] = qx.w;
    }
  };
  float kf[MC][4], qf[MC][4];
  fetch(0, kf, qf);
  const size_t obase = (size_t)b * N * H * dv + (size_t)h * dv + row;
  const size_t ubase = (size_t)bh * N * dv + row;
  for (int t = 0; t < N; ++t) {
    float kn[MC][4], qn[MC][4];
    fetch(clampi(t + 1, N - 1), kn, qn);
    const float be = sbeta[t];
    const float al = salpha[t];
    const float vt = sv[t * kChainRows + rl];

    float kq = 0.f, yk = 0.f, yq = 0.f, kq2 = 0.f, yk2 = 0.f, yq2 = 0.f;
#pragma unroll
    for (int m = 0; m < MC; ++m)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        kq = fmaf(kf[m][e], qf[m][e], kq);
        yk = fmaf(S[m][e], kf[m][e], yk);
        yq = fmaf(S[m][e], qf[m][e], yq);
        kq2 = fmaf(kf[m][e + 1], qf[m][e + 1], kq2);
        yk2 = fmaf(S[m][e + 1], kf[m][e + 1], yk2);
        yq2 = fmaf(S[m][e + 1], qf[m][e + 1], yq2);
      }
    kq = half32_sum(kq + kq2);
    yk = half32_sum(yk + yk2);
    yq = half32_sum(yq + yq2);

    const float u = be * (vt - al * yk);
    const float o = scale * fmaf(kq, u, al * yq);
#pragma unroll
    for (int m = 0; m < MC; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[m][e] = fmaf(u, kf[m][e], al * S[m][e]);
    if (s == 0 && rok) {
      out[obase + (size_t)t * H * dv] = o;
      rec.up[ubase + (size_t)t * dv] = u;
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
    if (tid == 0) {
      float G = 0.f;
      for (int t = 0; t < N; ++t) {
        G += sG[t];
        rec.G[(size_t)bh * N + t] = G;
      }
    }
    for (int idx = tid; idx < N * cpr; idx += 256)  // from the staged rows in LDS
      *reinterpret_cast<R4*>(rec.K + ((size_t)bh * N + idx / cpr) * dk + 4 * (idx % cpr)) = sk[idx];
    if (h == 0 && tid < N) {
      rec.parents[(size_t)b * N + tid] = tid - 1;
      rec.mask[(size_t)b * N + tid] = tid >= 63 ? ~0ull : ((1ull << (tid + 1)) - 1ull);
    }
  }
}

template <typename T>
hipError_t launch_chain_verify_t(int B, int N, int H, int dk, int dv, float* S0, const void* q,
                                 const void* k, const void* v, const float* beta,
                                 const float* g, float scale, float* out, void* factors,
                                 const RecordLayout& L, const void* prev_factors, int Np,
                                 const int32_t* last, int32_t* dev_status, hipStream_t stream) {
  Record<T> rec = record_views<T>(factors, L);
  const int ntiles = (dv + kChainRows - 1) / kChainRows;
  const long grid = (long)B * H * ntiles;
  size_t lds =
      (size_t)N * dk * sizeof(T) * 2 + (size_t)N * kChainRows * 4 + (size_t)N * 4 * 3;
  if (prev_factors) {
    const RecordLayout Lp = record_layout(B, Np, H, dk, dv, sizeof(T) == 2 ? GDN_BF16 : GDN_F32);
    Record<T> prev = record_views<T>(const_cast<void*>(prev_factors), Lp);
    lds += (size_t)Np * dk * sizeof(T) + (size_t)Np * kChainRows * 4 + (size_t)Np * 4;
    hipLaunchKernelGGL((chain_verify_kernel<T, true>), dim3((unsigned)grid), dim3(256), lds,
                       stream, N, H, dk, dv, ntiles, S0, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), beta, g, scale, out,
                       rec, prev, Np, last, dev_status);
  } else {
    hipLaunchKernelGGL((chain_verify_kernel<T, false>), dim3((unsigned)grid), dim3(256), lds,
                       stream, N, H, dk, dv, ntiles, S0, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), beta, g, scale, out,
                       rec, Record<T>{}, 0, nullptr, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_chain_verify(int B, int N, int H, int dk, int dv, int dtype, float* S0,
                               const void* q, const void* k, const void* v, const float* beta,
                               const float* g, float scale, float* out, void* factors,
                               const void* prev_factors, int Np, const int32_t* last,
                               int32_t* dev_status, hipStream_t stream) {
  const RecordLayout L = record_layout(B, N, H, dk, dv, dtype);
  if (dtype == GDN_BF16)
    return launch_chain_verify_t<bf16_t>(B, N, H, dk, dv, S0, q, k, v, beta, g, scale, out,
                                         factors, L, prev_factors, Np, last, dev_status, stream);
  return launch_chain_verify_t<float>(B, N, H, dk, dv, S0, q, k, v, beta, g, scale, out,
                                      factors, L, prev_factors, Np, last, dev_status, stream);
}

}  // namespace gdn
