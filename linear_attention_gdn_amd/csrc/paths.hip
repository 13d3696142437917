// Serial path kernels (gfx950): the recurrence run node by node along one
// root path per workgroup, with the state rows on chip.  Three uses:
//
//   replay verify  (SpecLA review, Figures, Figure 10 caption; Referee Report
//                  major comment 3): every root-to-leaf path of a draft
//                  replayed from S0; S0 read only.  Every path writes the
//                  outputs of all its nodes: a node's value depends only on
//                  its own root path, computed in the same order by every
//                  workgroup whose path holds it, so the writes agree bitwise.
//   replay commit  (review, Figures, Figure 11 caption): the accepted path's
//                  tokens replayed from S, the rows written back.
//   hybrid chains  (review, "What carries the argument"; Figures, Figure 6
//                  caption): the chain-decomposed verifier.  A node continues
//                  its parent's chain when it is the parent's first child; a
//                  chain's level is one more than that of the chain holding
//                  its head's parent, and one launch runs every chain of a
//                  level (the host plan gives each chain's head and last
//                  node).  A chain under parent p starts from the state after
//                  p, rebuilt from S0 and the factors lower levels buffered,
//                      S_p = e^{G_p} S0 + sum_{j on p's root path} e^{G_p - G_j} u'_j k_j^T,
//                  then runs its nodes serially and writes outputs and the
//                  factor record (u', G, k copy, parents, masks), the same
//                  record the factorized verifier writes.
//
// Per node t of the serial part (alpha_t = e^{g_t}):
//     y_k = S k_t,  u'_t = beta_t (v_t - alpha_t y_k),
//     o_t = scale (alpha_t S q_t + (k_t . q_t) u'_t),  S <- alpha_t S + u'_t k_t^T.
//
// Mapping: 512 threads = 8 waves, wave w owns state row w of the workgroup's
// 8-row tile and lane s its columns 4s .. 4s + 3 (a 1 KiB coalesced row).
// The path's nodes are taken in groups of 8: while a group computes from LDS
// (k and q rows widened to FP32), every thread has the next group's rows in
// flight (one 16-byte load of k and one of q for bf16 inputs), stored to the
// other LDS buffer after the group; a barrier per group.  Per-node scalars
// (g, beta, this row's v) sit in lane i of every wave for path node i and are
// read with readlane; the path itself is walked up the parent array held one
// node per lane, also with readlane.  Two waves per SIMD, as in the chain
// verifier.
#include "gdn_common.h"

namespace gdn {

constexpr int kPathRows = 8;
constexpr int kPathThreads = 512;
constexpr int kGroup = 8;  // path nodes per staging round

enum PathMode { kReplayVerify = 0, kReplayCommit = 1, kHybrid = 2 };

template <typename T, int MODE>
__global__ __launch_bounds__(kPathThreads) void path_kernel(
    int B, int N, int H, int dk, int dv, int ntiles, int P, const int32_t* __restrict__ ends,
    float* __restrict__ S, const int32_t* __restrict__ parents, const T* __restrict__ q,
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ g, float scale, float* __restrict__ out, Record<T> rec,
    int32_t* __restrict__ dev_status) {
  constexpr bool kOut = MODE != kReplayCommit;  // outputs (and q) needed
  __shared__ int snode[kMaxNodes];  // the workgroup's path, root first
  __shared__ __attribute__((aligned(16))) float sk[2][kGroup][kMaxDim];
  __shared__ __attribute__((aligned(16))) float sq[kOut ? 2 : 1][kOut ? kGroup : 1][kMaxDim];
  __shared__ float skq[2][kGroup];  // k . q of each staged node
  const int tid = threadIdx.x;
  const int s = tid & 63;
  const int wave = tid >> 6;
  const int tile = blockIdx.x % ntiles;
  const int bh = blockIdx.x / ntiles;
  const int h = bh % H;
  const int b = bh / H;
  const int slot = blockIdx.y;
  const int row = tile * kPathRows + wave;
  const bool rok = row < dv;
  const int rowc = clampi(row, dv - 1);
  const bool cok = 4 * s < dk;
  const int col = clampi(4 * s, dk - 4);  // global state column (clamped, masked)
  const int lcol = 4 * s;                  // staged column (zero past dk)

  // ---- topology check, this workgroup's end node, status
  const int pj = parents[(size_t)b * N + clampi(s, N - 1)];
  const bool bad = __ballot(s < N && (pj < -1 || pj >= s)) != 0ull;
  int end;
  bool bad_end = false;
  int cend = -1;  // hybrid: the chain's last node
  if (MODE == kHybrid) {
    // P is the level; the plan holds (head, last node) per chain
    end = ends[(((size_t)P * B + b) * N + slot) * 2];
    cend = ends[(((size_t)P * B + b) * N + slot) * 2 + 1];
  } else if (MODE == kReplayVerify) {
    end = ends[(size_t)b * P + slot];
    const int ej = ends[(size_t)b * P + clampi(s, P - 1)];
    bad_end = __ballot(s < P && (ej < -1 || ej >= N)) != 0ull;
  } else {
    end = ends[b];
    bad_end = end < -1 || end >= N;
  }
  const bool first = slot == 0 && tile == 0 && h == 0 && (MODE != kHybrid || P == 0);
  if (first && tid == 0 && dev_status)
    dev_status[b] = (bad || bad_end) ? GDN_ERR_TOPOLOGY : GDN_OK;
  if (bad) {  // uniform
    if (MODE == kHybrid && P == 0 && slot == 0) {  // the sequence's outputs and record rows: zeros
      for (int idx = tid; idx < N * kPathRows; idx += kPathThreads) {
        const int t = idx / kPathRows, r = tile * kPathRows + idx % kPathRows;
        if (r < dv) {
          out[(((size_t)b * N + t) * H + h) * dv + r] = 0.f;
          rec.up[((size_t)bh * N + t) * dv + r] = 0.f;
        }
      }
      if (first && tid < N) {
        rec.parents[(size_t)b * N + tid] = pj;
        rec.mask[(size_t)b * N + tid] = 0ull;
      }
    }
    return;
  }
  if (end < 0 || end >= N) return;  // uniform: an empty or out-of-range slot

  // ---- this workgroup's path as a bit mask, walked up the parent array held
  // one node per lane (readlane: scalar steps, no memory round trips)
  auto walk = [&](int e) {  // uniform e
    uint64_t mm = 0ull;
    for (int t = e; t >= 0; t = __builtin_amdgcn_readlane(pj, t)) mm |= 1ull << t;
    return mm;
  };
  // nodes of m in increasing order (root first); the first npre of them only
  // enter through the hybrid's prefix update
  uint64_t m;
  int npre = 0;
  if (MODE == kHybrid) {
    if (cend < end || cend >= N) return;  // uniform: a plan that does not fit the parents
    m = walk(cend);
    if (!((m >> end) & 1ull)) return;     // uniform: likewise
    npre = __popcll(m & ((1ull << end) - 1ull));
  } else {
    m = walk(end);
  }
  const int np = __popcll(m);
  if (tid < N && ((m >> tid) & 1ull)) snode[__popcll(m & ((1ull << tid) - 1ull))] = tid;

  // ---- hybrid: the record sections one workgroup writes (parents and masks
  // once per sequence, the k copy of the chain's nodes once per head)
  if (MODE == kHybrid && first) {  // uniform: ancestor-or-self masks by pointer jumping
    const int tl = s < N ? s : -1;
    uint64_t mask_l = tl >= 0 ? (1ull << tl) : 0ull;
    int a = tl >= 0 ? pj : -1;
    for (int r = 0; r < 6; ++r) {  // 2^6 = 64 >= path length
      if (__ballot(a >= 0) == 0ull) break;  // uniform
      const int src = a >= 0 ? a : s;
      const uint64_t ma = __shfl(mask_l, src);
      const int aa = __shfl(a, src);
      if (a >= 0) {
        mask_l |= ma;
        a = aa;
      }
    }
    if (tid < N) {
      rec.parents[(size_t)b * N + tid] = pj;
      rec.mask[(size_t)b * N + tid] = mask_l;
    }
  }
  __syncthreads();  // snode complete
  if (MODE == kHybrid && tile == 0) {
    const int cpr = dk / 4;
    for (int idx = tid; idx < (np - npre) * cpr; idx += kPathThreads) {
      const int t = snode[npre + idx / cpr], c = 4 * (idx % cpr);
      *reinterpret_cast<typename Raw4<T>::type*>(rec.K + ((size_t)bh * N + t) * dk + c) =
          raw4(k + (((size_t)b * N + t) * H + h) * dk + c);
    }
  }

  // ---- per-node scalars in lane i (path position i) of every wave: node,
  // alpha, g, beta, this row's v, and whether this workgroup writes its output
  const int t_l = snode[clampi(s, np - 1)];
  const size_t nhi = ((size_t)b * N + t_l) * H + h;
  const float g_l = g[nhi];
  const float b_l = beta[nhi];
  const float v_l = rok ? widen1(v[nhi * dv + rowc]) : 0.f;
  const float a_l = expf(g_l);
  // hybrid prefix: coefficient e^{G_p - G_j} u'_j[row] of prefix position i
  float c_l = 0.f, G = 0.f;
  if (MODE == kHybrid && npre > 0) {  // uniform
    const float Gp = rec.G[(size_t)bh * N + snode[npre - 1]];
    const float Gj = rec.G[(size_t)bh * N + t_l];
    const float uj = rec.up[((size_t)bh * N + t_l) * dv + rowc];
    c_l = expf(Gp - Gj) * uj;
    G = Gp;
  }
  auto lanef = [](float x, int i) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), i));
  };

  // ---- group staging: thread x loads 16 bytes of node (x / units) of the group
  constexpr int EPC = 16 / (int)sizeof(T);              // elements per 16-byte unit
  const int upr = dk / EPC;                              // units per row
  const int ku = tid / upr < kGroup ? tid : -1;          // this thread's unit, or none
  const int kn = ku >= 0 ? ku / upr : 0, kc = ku >= 0 ? (ku % upr) * EPC : 0;
  u32x4 kr = {0u, 0u, 0u, 0u}, qr = {0u, 0u, 0u, 0u};
  auto load_group = [&](int g0) {
    const int t = snode[clampi(g0 + kn, np - 1)];
    const size_t base = (((size_t)b * N + t) * H + h) * dk + kc;
    kr = *reinterpret_cast<const u32x4*>(k + base);
    if (kOut) qr = *reinterpret_cast<const u32x4*>(q + base);
  };
  auto store_group = [&](int buf) {
    if (ku < 0) return;
    if constexpr (sizeof(T) == 2) {
      float* dk_ = &sk[buf][kn][kc];
      *reinterpret_cast<f32x4*>(dk_) = widen4(u32x2{kr.x, kr.y});
      *reinterpret_cast<f32x4*>(dk_ + 4) = widen4(u32x2{kr.z, kr.w});
      if (kOut) {
        float* dq = &sq[buf][kn][kc];
        *reinterpret_cast<f32x4*>(dq) = widen4(u32x2{qr.x, qr.y});
        *reinterpret_cast<f32x4*>(dq + 4) = widen4(u32x2{qr.z, qr.w});
      }
    } else {
      *reinterpret_cast<f32x4*>(&sk[buf][kn][kc]) = __builtin_bit_cast(f32x4, kr);
      if (kOut) *reinterpret_cast<f32x4*>(&sq[buf][kn][kc]) = __builtin_bit_cast(f32x4, qr);
    }
  };

  float* srow = S + ((size_t)bh * dv + rowc) * dk + col;
  const f32x4 s0v = mask4(load4(srow), rok && cok);  // zero past dk: the products vanish
  float Sr[4] = {s0v.x, s0v.y, s0v.z, s0v.w};
  if (MODE == kHybrid && npre > 0) {
    const float sc = expf(G);
#pragma unroll
    for (int e = 0; e < 4; ++e) Sr[e] *= sc;
  }
  const size_t orow = (size_t)h * dv + tile * kPathRows + __builtin_amdgcn_readfirstlane(wave);
  const bool store_lane = s == 63 && rok;

  // operands of one position of the current group, read from LDS a step ahead
  struct Ops {
    f32x4 kx, qx;
    float kq;
  };
  // (columns past dk of both buffers are zero, so no column masks per step)
  auto fetch = [&](int buf, int i, Ops& o) {
    o.kx = *reinterpret_cast<const f32x4*>(&sk[buf][i][lcol]);
    if (kOut) {
      o.qx = *reinterpret_cast<const f32x4*>(&sq[buf][i][lcol]);
      o.kq = skq[buf][i];
    }
  };
  // k . q of the staged group's nodes: wave w takes node w (after a barrier)
  auto kq_group = [&](int buf, int gn) {
    if (kOut && wave < gn) {
      const f32x4 kx = *reinterpret_cast<const f32x4*>(&sk[buf][wave][lcol]);
      const f32x4 qx = *reinterpret_cast<const f32x4*>(&sq[buf][wave][lcol]);
      float a = kx.x * qx.x;
      a = fmaf(kx.y, qx.y, a);
      a = fmaf(kx.z, qx.z, a);
      a = fmaf(kx.w, qx.w, a);
      a = wave64_sum(a);
      if (s == 0) skq[buf][wave] = a;
    }
  };
  // The read-ahead operands pass through an empty asm once the step that
  // overlaps them is done: carried around the loop as plain values, not as
  // loads the optimiser would fold back into the next step (and wait for).
  auto opaque = [](Ops& o) {
    asm volatile("" : "+v"(o.kx));
    if (kOut) {
      asm volatile("" : "+v"(o.qx));
      asm volatile("" : "+v"(o.kq));
    }
  };

  if (dk < kMaxDim) {  // zero the columns past dk once
    for (int idx = tid; idx < 2 * kGroup * (kMaxDim - dk); idx += kPathThreads) {
      const int r = idx / (kMaxDim - dk), c = dk + idx % (kMaxDim - dk);
      sk[r / kGroup][r % kGroup][c] = 0.f;
      if (kOut) sq[r / kGroup][r % kGroup][c] = 0.f;
    }
  }
  load_group(0);
  store_group(0);
  __syncthreads();
  kq_group(0, np < kGroup ? np : kGroup);
  if (kOut) __syncthreads();
  for (int g0 = 0; g0 < np; g0 += kGroup) {  // uniform
    const int buf = (g0 / kGroup) & 1;
    const bool more = g0 + kGroup < np;
    if (more) load_group(g0 + kGroup);  // in flight while this group computes
    const int gn = np - g0 < kGroup ? np - g0 : kGroup;
    Ops cur;
    fetch(buf, 0, cur);
    for (int i = 0; i < gn; ++i) {  // uniform
      Ops nxt;
      fetch(buf, i + 1 < gn ? i + 1 : i, nxt);  // in flight while position i computes
      const int pos = g0 + i;
      if (MODE == kHybrid && pos < npre) {  // prefix: a rank-1 update, no recurrence
        const float c = lanef(c_l, pos);
#pragma unroll
        for (int e = 0; e < 4; ++e) Sr[e] = fmaf(c, cur.kx[e], Sr[e]);
        opaque(nxt);
        cur = nxt;
        continue;
      }
      const float al = lanef(a_l, pos), be = lanef(b_l, pos), vt = lanef(v_l, pos);
      float yk = Sr[0] * cur.kx.x;
      yk = fmaf(Sr[1], cur.kx.y, yk);
      yk = fmaf(Sr[2], cur.kx.z, yk);
      yk = fmaf(Sr[3], cur.kx.w, yk);
      float yq = 0.f;
      if (kOut) {
        yq = Sr[0] * cur.qx.x;
        yq = fmaf(Sr[1], cur.qx.y, yq);
        yq = fmaf(Sr[2], cur.qx.z, yq);
        yq = fmaf(Sr[3], cur.qx.w, yq);
        wave64_sum2_uniform(yk, yq, yk, yq);  // both wave-uniform
      } else {
        yk = wave64_sum_uniform(yk);
      }
      const float u = be * (vt - al * yk);
      if (kOut) {
        const int t = __builtin_amdgcn_readlane(t_l, pos);
        if (store_lane) {
          out[(size_t)(b * N + t) * H * dv + orow] = scale * fmaf(cur.kq, u, al * yq);
          if (MODE == kHybrid) rec.up[((size_t)bh * N + t) * dv + orow - (size_t)h * dv] = u;
        }
        if (MODE == kHybrid) {
          G += lanef(g_l, pos);
          if (tile == 0 && tid == 63) rec.G[(size_t)bh * N + t] = G;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Sr[e] = fmaf(u, cur.kx[e], al * Sr[e]);
      opaque(nxt);
      cur = nxt;
    }
    if (more) store_group(buf ^ 1);
    __syncthreads();
    if (more) {  // uniform
      kq_group(buf ^ 1, np - g0 - kGroup < kGroup ? np - g0 - kGroup : kGroup);
      if (kOut) __syncthreads();
    }
  }
  if (MODE == kReplayCommit && rok && cok)
    *reinterpret_cast<f32x4*>(srow) = f32x4{Sr[0], Sr[1], Sr[2], Sr[3]};
}

template <typename T, int MODE>
hipError_t launch_path_t(dim3 grid, int B, int N, int H, int dk, int dv, int ntiles, int P,
                         const int32_t* ends, float* S, const int32_t* parents, const void* q,
                         const void* k, const void* v, const float* beta, const float* g,
                         float scale, float* out, const Record<T>& rec, int32_t* dev_status,
                         hipStream_t stream) {
  hipLaunchKernelGGL((path_kernel<T, MODE>), grid, dim3(kPathThreads), 0, stream, B, N, H, dk, dv,
                     ntiles, P, ends, S, parents, static_cast<const T*>(q),
                     static_cast<const T*>(k), static_cast<const T*>(v), beta, g, scale, out, rec,
                     dev_status);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_replay_t(bool verify, int B, int N, int H, int dk, int dv, float* S,
                           const int32_t* parents, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, float scale, const int32_t* ends,
                           int P, float* out, int32_t* dev_status, hipStream_t stream) {
  const int ntiles = (dv + kPathRows - 1) / kPathRows;
  const dim3 grid((unsigned)((long)B * H * ntiles), verify ? (unsigned)P : 1u);
  if (verify)
    return launch_path_t<T, kReplayVerify>(grid, B, N, H, dk, dv, ntiles, P, ends, S, parents, q,
                                           k, v, beta, g, scale, out, Record<T>{}, dev_status,
                                           stream);
  return launch_path_t<T, kReplayCommit>(grid, B, N, H, dk, dv, ntiles, 1, ends, S, parents,
                                         nullptr, k, v, beta, g, 1.f, nullptr, Record<T>{},
                                         dev_status, stream);
}

hipError_t launch_replay(bool verify, int B, int N, int H, int dk, int dv, int dtype, float* S,
                         const int32_t* parents, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, float scale, const int32_t* ends,
                         int P, float* out, int32_t* dev_status, hipStream_t stream) {
  if (dtype == GDN_BF16)
    return launch_replay_t<bf16_t>(verify, B, N, H, dk, dv, S, parents, q, k, v, beta, g, scale,
                                   ends, P, out, dev_status, stream);
  return launch_replay_t<float>(verify, B, N, H, dk, dv, S, parents, q, k, v, beta, g, scale,
                                ends, P, out, dev_status, stream);
}

template <typename T>
hipError_t launch_hybrid_t(int B, int N, int H, int dk, int dv, const float* S0,
                           const int32_t* parents, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, float scale, float* out,
                           void* factors, const int32_t* plan, int levels,
                           const int32_t* chains_per_level, int32_t* dev_status,
                           hipStream_t stream) {
  const RecordLayout L = record_layout(B, N, H, dk, dv, sizeof(T) == 2 ? GDN_BF16 : GDN_F32);
  const Record<T> rec = record_views<T>(factors, L);
  const int ntiles = (dv + kPathRows - 1) / kPathRows;
  for (int l = 0; l < levels; ++l) {  // a level runs once every lower level is complete
    const dim3 grid((unsigned)((long)B * H * ntiles), (unsigned)chains_per_level[l]);
    const hipError_t e = launch_path_t<T, kHybrid>(grid, B, N, H, dk, dv, ntiles, l, plan,
                                                   const_cast<float*>(S0), parents, q, k, v,
                                                   beta, g, scale, out, rec, dev_status, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_hybrid(int B, int N, int H, int dk, int dv, int dtype, const float* S0,
                         const int32_t* parents, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, float scale, float* out,
                         void* factors, const int32_t* plan, int levels,
                         const int32_t* chains_per_level, int32_t* dev_status,
                         hipStream_t stream) {
  if (dtype == GDN_BF16)
    return launch_hybrid_t<bf16_t>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out,
                                   factors, plan, levels, chains_per_level, dev_status, stream);
  return launch_hybrid_t<float>(B, N, H, dk, dv, S0, parents, q, k, v, beta, g, scale, out,
                                factors, plan, levels, chains_per_level, dev_status, stream);
}

// ---------------------------------------------------------------------------
// host: the hybrid plan (chains per level) from a parent array in host memory
// ---------------------------------------------------------------------------

// plan[((l * B + b) * N + c) * 2 + {0, 1}] = head and last node of the c-th
// chain of level l in sequence b (-1 past the last); chains_per_level[l] =
// most chains any sequence has at level l; returns the number of levels, or
// -1 for a parent array that fails the topology check.
int hybrid_plan(int B, int N, const int32_t* parents, int32_t* plan, int32_t* chains_per_level) {
  for (long i = 0; i < 2L * N * B * N; ++i) plan[i] = -1;
  for (int l = 0; l < N; ++l) chains_per_level[l] = 0;
  int levels = 0;
  int fc[kMaxNodes], chain_level[kMaxNodes], count[kMaxNodes];
  for (int b = 0; b < B; ++b) {
    const int32_t* p = parents + (size_t)b * N;
    for (int t = 0; t < N; ++t) {
      if (p[t] < -1 || p[t] >= t) return -1;
      fc[t] = -1;
      count[t] = 0;
    }
    for (int t = N - 1; t >= 0; --t)
      if (p[t] >= 0) fc[p[t]] = t;  // ends at the lowest-numbered child
    for (int t = 0; t < N; ++t) {
      const bool is_head = p[t] < 0 || fc[p[t]] != t;
      chain_level[t] = is_head ? (p[t] < 0 ? 0 : chain_level[p[t]] + 1) : chain_level[p[t]];
      if (is_head) {
        const int l = chain_level[t];
        int last = t;
        while (fc[last] >= 0) last = fc[last];
        plan[(((size_t)l * B + b) * N + count[l]) * 2] = t;
        plan[(((size_t)l * B + b) * N + count[l]) * 2 + 1] = last;
        ++count[l];
        if (count[l] > chains_per_level[l]) chains_per_level[l] = count[l];
        if (l + 1 > levels) levels = l + 1;
      }
    }
  }
  return levels;
}

}  // namespace gdn
