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
// with DPP row rotations plus one v_permlane16_swap (or, for y_q, which only
// the storing lane needs, one DPP row broadcast).  A workgroup owns 8 rows,
// one per SIMD pair of half-waves, so all four SIMDs of a CU run the serial
// loop.  Everything the loop needs (k, q, v of the 8 rows, alpha, beta) is
// staged in LDS by one round of loads; the state row is requested last in
// that round and first read after the k.q products, so the staging runs
// while it arrives from HBM.
// The loop is bound by VALU issue (one wave per SIMD), so work that does not
// depend on the row leaves it: k and q are widened to FP32 once while staging
// (drafts of up to 32 nodes), k_t . q_t is computed once per step for the
// whole workgroup before the loop, and column masks exist only for d_k < 256.
// Each step reads the next step's operands from LDS while it computes.
//
// Delayed commit (review: Referee Report summary, mechanism (ii); Figure 7
// caption, right side): with DLY the same workgroup first applies the
// previous draft's accepted path to its state tile, using the previous factor
// record staged in LDS in the same round of loads, writes the tile back, and
// then verifies the new chain from the updated registers.  The update repeats
// the commit kernel's operations in the same order (scale by e^{G_last}, then
// one fused multiply-add per path node in node order), so the result is
// bitwise that of commit followed by verify.
#include <type_traits>

#include "gdn_common.h"

namespace gdn {

constexpr int kChainRows = 8;  // state rows per workgroup (one per half-wave)

// Stored form of staged k/q rows: FP32 (QF) or as loaded.
template <typename T, bool QF>
struct Staged {
  using type = typename std::conditional<QF, f32x4, typename Raw4<T>::type>::type;
};
__device__ inline f32x4 stage_cvt(const f32x4& x, f32x4*) { return x; }
__device__ inline f32x4 stage_cvt(const u32x2& x, f32x4*) { return widen4(x); }
__device__ inline u32x2 stage_cvt(const u32x2& x, u32x2*) { return x; }
// back to the element type (exact: the values came from T)
__device__ inline f32x4 unstage(const f32x4& x, float*) { return x; }
__device__ inline u32x2 unstage(const f32x4& x, bf16_t*) {
  return u32x2{(__float_as_uint(x.x) >> 16) | (__float_as_uint(x.y) & 0xffff0000u),
               (__float_as_uint(x.z) >> 16) | (__float_as_uint(x.w) & 0xffff0000u)};
}
__device__ inline u32x2 unstage(const u32x2& x, bf16_t*) { return x; }

template <typename T, bool DLY, bool QF, bool FULL>
__global__ __launch_bounds__(256) void chain_verify_kernel(
    int N, int H, int dk, int dv, int ntiles, float* __restrict__ S0,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ beta, const float* __restrict__ g, float scale,
    float* __restrict__ out, Record<T> rec, Record<T> prev, int Np,
    const int32_t* __restrict__ last_acc, int32_t* __restrict__ dev_status) {
  constexpr int MC = kMaxDim / 128;  // float4 chunks per lane
  using R4 = typename Raw4<T>::type;
  using SK = typename Staged<T, QF>::type;
  // dynamic LDS: k, q [N][dk] (staged form), v [N][8], alpha, beta, g, k.q [N];
  // with DLY also the previous record's k [Np][dk] (as loaded), u' of the
  // tile's rows [Np][8] and the commit coefficients e^{G_last - G_i} [Np]
  extern __shared__ f32x4 lds4[];
  const int cpr = dk / 4;
  SK* sk = reinterpret_cast<SK*>(lds4);
  SK* sq = sk + N * cpr;
  R4* skp = reinterpret_cast<R4*>(sq + N * cpr);
  float* sv = reinterpret_cast<float*>(skp + (DLY ? Np * cpr : 0));
  float* salpha = sv + N * kChainRows;
  float* sbeta = salpha + N;
  float* sG = sbeta + N;
  float* skq = sG + N;
  float* sup = skq + N;
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
  auto colok = [&](int m) { return FULL || 128 * m + 4 * s < dk; };

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
  // the previous draft's record (delayed commit): masks, G, u' of this tile's
  // rows and the k rows, none of which depends on last_accepted
  constexpr int BATCH = 4;
  int last = -1;
  int last_v = -1;
  uint64_t mlp = 0;
  float glp = 0.f;
  float upb[DLY ? VB : 1];
  R4 kpb[DLY ? BATCH : 1];
  auto prevk_off = [&](int idx) {
    idx = clampi(idx, Np * cpr - 1);
    return ((size_t)bh * Np + idx / cpr) * dk + 4 * (idx % cpr);
  };
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
  auto stage_load = [&](int base, R4 (&kb)[BATCH], R4 (&qb)[BATCH]) {
#pragma unroll
    for (int x = 0; x < BATCH; ++x) {
      const int idx = clampi(base + 256 * x, N * cpr - 1);
      const size_t off = (((size_t)b * N + idx / cpr) * H + h) * dk + 4 * (idx % cpr);
      kb[x] = raw4(k + off);
      qb[x] = raw4(q + off);
    }
  };
  // No branch around the stores (a load used only under one is sunk into it
  // and waited for together with everything issued before): past the end a
  // thread rewrites the clamped chunk with the bits it loaded for it, which
  // are the owner's bits.
  auto stage_store = [&](int base, const R4 (&kb)[BATCH], const R4 (&qb)[BATCH]) {
#pragma unroll
    for (int x = 0; x < BATCH; ++x) {
      const int idx = clampi(base + 256 * x, N * cpr - 1);
      sk[idx] = stage_cvt(kb[x], (SK*)nullptr);
      sq[idx] = stage_cvt(qb[x], (SK*)nullptr);
    }
  };
  R4 kb0[BATCH], qb0[BATCH];
  stage_load(tid, kb0, qb0);
  // The state row is requested last: loads complete in issue order, so the
  // staging below waits only for the loads above, and the state (from HBM)
  // streams in while the staging and the k.q products run.
  f32x4 Sx[MC];
  __builtin_amdgcn_sched_barrier(0);
  {
    const float* rp = S0 + ((size_t)bh * dv + clampi(row, dv - 1)) * dk;
#pragma unroll
    for (int m = 0; m < MC; ++m) Sx[m] = load4(rp + clampi(128 * m + 4 * s, dk - 4));
  }
  __builtin_amdgcn_sched_barrier(0);
  stage_store(tid, kb0, qb0);
  for (int base = tid + 256 * BATCH; base < N * cpr; base += 256 * BATCH) {
    R4 kb[BATCH], qb[BATCH];
    stage_load(base, kb, qb);
    stage_store(base, kb, qb);
  }
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
  __syncthreads();

  // ---- k_t . q_t, the same for every row: half-wave rl takes nodes rl, rl + 8, ...
  auto kchunk = [&](const SK* base, int t, int m) {
    return mask4(widen4(base[t * cpr + (FULL ? 32 * m + s : clampi(32 * m + s, cpr - 1))]),
                 colok(m));
  };
  for (int t = rl; t < N; t += kChainRows) {
    float a = 0.f, a2 = 0.f;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const f32x4 kx = kchunk(sk, t, m);
      const f32x4 qx = kchunk(sq, t, m);
      a = fmaf(kx.x, qx.x, a);
      a2 = fmaf(kx.y, qx.y, a2);
      a = fmaf(kx.z, qx.z, a);
      a2 = fmaf(kx.w, qx.w, a2);
    }
    a = half32_sum(a + a2);
    if (s == 0) skq[t] = a;
  }

  // the state row (first needed here)
  float S[MC][4];
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const f32x4 x = mask4(Sx[m], rok && colok(m));
    S[m][0] = x.x;
    S[m][1] = x.y;
    S[m][2] = x.z;
    S[m][3] = x.w;
  }

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
      // path nodes in increasing order, four at a time: the LDS reads of a
      // group are issued before its multiply-adds
      for (int i0 = 0; i0 <= last; i0 += 4) {
        float c[4];
        f32x4 kc[4][MC];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = clampi(i0 + u, Np - 1);
          c[u] = sGp[i] * sup[i * kChainRows + rl];
#pragma unroll
          for (int m = 0; m < MC; ++m) kc[u][m] = widen4(skp[i * cpr + clampi(32 * m + s, cpr - 1)]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (i0 + u > last || ((pm >> (i0 + u)) & 1ull) == 0ull) continue;  // uniform
#pragma unroll
          for (int m = 0; m < MC; ++m) {
            S[m][0] = fmaf(c[u], kc[u][m].x, S[m][0]);
            S[m][1] = fmaf(c[u], kc[u][m].y, S[m][1]);
            S[m][2] = fmaf(c[u], kc[u][m].z, S[m][2]);
            S[m][3] = fmaf(c[u], kc[u][m].w, S[m][3]);
          }
        }
      }
      if (rok) {
        float* wp = S0 + ((size_t)bh * dv + row) * dk;
#pragma unroll
        for (int m = 0; m < MC; ++m)
          if (colok(m))
            *reinterpret_cast<f32x4*>(wp + 128 * m + 4 * s) =
                f32x4{S[m][0], S[m][1], S[m][2], S[m][3]};
      }
    }
  }
  __syncthreads();  // k.q of every node is in LDS

  // ---- the recurrence.  Operands of step t (k_t, q_t chunks; alpha, beta,
  // v, k.q) are read from LDS during step t - 1; two register sets alternate.
  struct Ops {
    f32x4 kc[MC], qc[MC];
    float al, be, vt, kq;
  };
  auto fetch = [&](int t, Ops& o) {
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      o.kc[m] = kchunk(sk, t, m);
      o.qc[m] = kchunk(sq, t, m);
    }
    o.al = salpha[t];
    o.be = sbeta[t];
    o.vt = sv[t * kChainRows + rl];
    o.kq = skq[t];
  };
  const size_t obase = (size_t)b * N * H * dv + (size_t)h * dv + row;
  const size_t ubase = (size_t)bh * N * dv + row;
  auto run = [&](int t, const Ops& o) {
    float yk = 0.f, yq = 0.f, yk2 = 0.f, yq2 = 0.f;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      yk = fmaf(S[m][0], o.kc[m].x, yk);
      yq = fmaf(S[m][0], o.qc[m].x, yq);
      yk2 = fmaf(S[m][1], o.kc[m].y, yk2);
      yq2 = fmaf(S[m][1], o.qc[m].y, yq2);
      yk = fmaf(S[m][2], o.kc[m].z, yk);
      yq = fmaf(S[m][2], o.qc[m].z, yq);
      yk2 = fmaf(S[m][3], o.kc[m].w, yk2);
      yq2 = fmaf(S[m][3], o.qc[m].w, yq2);
    }
    yk = half32_sum(yk + yk2);
    yq = half32_sum_hi(yq + yq2);  // complete in lanes 16..31 of the half-wave only
    const float u = o.be * (o.vt - o.al * yk);
    const float ov = scale * fmaf(o.kq, u, o.al * yq);
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      S[m][0] = fmaf(u, o.kc[m].x, o.al * S[m][0]);
      S[m][1] = fmaf(u, o.kc[m].y, o.al * S[m][1]);
      S[m][2] = fmaf(u, o.kc[m].z, o.al * S[m][2]);
      S[m][3] = fmaf(u, o.kc[m].w, o.al * S[m][3]);
    }
    if (s == 16 && rok) {
      out[obase + (size_t)t * H * dv] = ov;
      rec.up[ubase + (size_t)t * dv] = u;
    }
  };
  // The prefetched operands pass through an empty asm after the step that
  // overlaps their reads: the values carried around the loop are then not
  // loads, which the optimiser would otherwise re-issue at the top of the
  // next step (folding a phi of loads into a load) and wait for at once.
  auto opaque = [](Ops& o) {
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      asm volatile("" : "+v"(o.kc[m]));
      asm volatile("" : "+v"(o.qc[m]));
    }
    asm volatile("" : "+v"(o.al), "+v"(o.be), "+v"(o.vt), "+v"(o.kq));
  };
  Ops A, Bo;
  fetch(0, A);
  opaque(A);
  for (int t = 0; t < N; t += 2) {
    fetch(clampi(t + 1, N - 1), Bo);
    run(t, A);
    opaque(Bo);
    if (t + 1 < N) {  // uniform
      fetch(clampi(t + 2, N - 1), A);
      run(t + 1, Bo);
      opaque(A);
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
      *reinterpret_cast<R4*>(rec.K + ((size_t)bh * N + idx / cpr) * dk + 4 * (idx % cpr)) =
          unstage(sk[idx], (T*)nullptr);
    if (h == 0 && tid < N) {
      rec.parents[(size_t)b * N + tid] = tid - 1;
      rec.mask[(size_t)b * N + tid] = tid >= 63 ? ~0ull : ((1ull << (tid + 1)) - 1ull);
    }
  }
}

template <typename T, bool DLY, bool QF>
void launch_chain_qf(bool full, long grid, size_t lds, hipStream_t stream, int N, int H, int dk,
                     int dv, int ntiles, float* S0, const T* q, const T* k, const T* v,
                     const float* beta, const float* g, float scale, float* out,
                     const Record<T>& rec, const Record<T>& prev, int Np, const int32_t* last,
                     int32_t* dev_status) {
  if (full)
    hipLaunchKernelGGL((chain_verify_kernel<T, DLY, QF, true>), dim3((unsigned)grid), dim3(256),
                       lds, stream, N, H, dk, dv, ntiles, S0, q, k, v, beta, g, scale, out, rec,
                       prev, Np, last, dev_status);
  else
    hipLaunchKernelGGL((chain_verify_kernel<T, DLY, QF, false>), dim3((unsigned)grid), dim3(256),
                       lds, stream, N, H, dk, dv, ntiles, S0, q, k, v, beta, g, scale, out, rec,
                       prev, Np, last, dev_status);
}

template <typename T>
hipError_t launch_chain_verify_t(int B, int N, int H, int dk, int dv, float* S0, const void* q,
                                 const void* k, const void* v, const float* beta,
                                 const float* g, float scale, float* out, void* factors,
                                 const RecordLayout& L, const void* prev_factors, int Np,
                                 const int32_t* last, int32_t* dev_status, hipStream_t stream) {
  Record<T> rec = record_views<T>(factors, L);
  Record<T> prev{};
  const bool dly = prev_factors != nullptr;
  if (dly) {
    const RecordLayout Lp = record_layout(B, Np, H, dk, dv, sizeof(T) == 2 ? GDN_BF16 : GDN_F32);
    prev = record_views<T>(const_cast<void*>(prev_factors), Lp);
  } else {
    Np = 0;
  }
  // k, q staged as FP32 for drafts of up to 32 nodes (bf16 beyond, to bound LDS)
  const bool qf = sizeof(T) == 4 || N <= 32;
  const bool full = dk == kMaxDim;
  const int ntiles = (dv + kChainRows - 1) / kChainRows;
  const long grid = (long)B * H * ntiles;
  const size_t lds = (size_t)N * dk * (qf ? 4 : sizeof(T)) * 2 + (size_t)N * kChainRows * 4 +
                     (size_t)N * 4 * 4 + (size_t)Np * dk * sizeof(T) +
                     (size_t)Np * kChainRows * 4 + (size_t)Np * 4;
  const T* qq = static_cast<const T*>(q);
  const T* kk = static_cast<const T*>(k);
  const T* vv = static_cast<const T*>(v);
  if (dly) {
    if (qf)
      launch_chain_qf<T, true, true>(full, grid, lds, stream, N, H, dk, dv, ntiles, S0, qq, kk,
                                     vv, beta, g, scale, out, rec, prev, Np, last, dev_status);
    else
      launch_chain_qf<T, true, false>(full, grid, lds, stream, N, H, dk, dv, ntiles, S0, qq, kk,
                                      vv, beta, g, scale, out, rec, prev, Np, last, dev_status);
  } else {
    if (qf)
      launch_chain_qf<T, false, true>(full, grid, lds, stream, N, H, dk, dv, ntiles, S0, qq, kk,
                                      vv, beta, g, scale, out, rec, prev, 0, nullptr, nullptr);
    else
      launch_chain_qf<T, false, false>(full, grid, lds, stream, N, H, dk, dv, ntiles, S0, qq, kk,
                                       vv, beta, g, scale, out, rec, prev, 0, nullptr, nullptr);
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
