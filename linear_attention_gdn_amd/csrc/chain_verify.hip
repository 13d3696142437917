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
// Mapping: 512 threads = 8 waves; each wave owns one state row and lane s
// holds columns 4s .. 4s + 3, so a row is one 1 KiB coalesced read and the
// dot products reduce over the wave with DPP row rotations plus
// v_permlane16_swap and v_permlane32_swap (for y_q, which only the storing
// lane needs, two DPP row broadcasts instead).  A workgroup owns 8 rows and
// puts two waves on every SIMD of its CU: the serial loop is a chain of
// dependent VALU, DPP and LDS operations, and the second wave issues while
// the first waits on one.  Everything the loop needs is staged in LDS by one
// round of loads: k and q of every node (interleaved per node, so one address
// serves both), and per node and row the step scalars {alpha, beta, k.q, v},
// read as one 16-byte word.  The state row is requested last in that round
// and first read after the k.q products, so the staging runs while it arrives
// from HBM.  Work that does not depend on the row leaves the loop: k and q
// are widened to FP32 once while staging (drafts of up to 32 nodes), k_t . q_t
// is computed once per node for the whole workgroup before the loop, and
// column masks exist only for d_k < 256.  Each step reads the next step's
// operands from LDS while it computes; a padding node after the last one
// keeps that read-ahead free of clamps.
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

constexpr int kChainRows = 8;      // state rows per workgroup (one per wave)
constexpr int kChainThreads = 512;  // 8 waves: two per SIMD

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

template <typename T, bool DLY, bool QF, bool FULL, int KB>
__global__ __launch_bounds__(kChainThreads) void chain_verify_kernel(
    uint32_t shape, int H, const T* __restrict__ k, const T* __restrict__ q,
    const float* __restrict__ g, const float* __restrict__ beta, const T* __restrict__ v,
    float* __restrict__ S0, float scale, float* __restrict__ out, Record<T> rec,
    Record<T> prev, int Np, const int32_t* __restrict__ last_acc,
    int32_t* __restrict__ dev_status) {
  // The first 14 argument dwords (shape, H and the six input pointers) arrive
  // preloaded in SGPRs; the rest is fetched from memory, so every load that
  // needs only those goes out before the first one that needs the rest.
  const int N = shape & 0xff;
  const int dk = (shape >> 8) & 0x3ff;
  const int dv = shape >> 18;
  const int ntiles = (dv + kChainRows - 1) / kChainRows;
  static_assert(kMaxDim == 256, "one float4 of each state row per lane");
  constexpr int NT = kChainThreads;
  using R4 = typename Raw4<T>::type;
  using SK = typename Staged<T, QF>::type;
  // 16-byte load units: EPC elements, E4 = EPC / 4 staged chunks of 4 columns
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int E4 = EPC / 4;
  // k . q from registers: with bf16 rows of 256 a node's k and q rows are 64
  // units, one wave (k in lanes 0..31, q in lanes 32..63)
  constexpr bool KQR = FULL && sizeof(T) == 2;
  // dynamic LDS: k and q rows interleaved per node [N + 1][2][dk] (staged
  // form; node N is padding that the loop's read-ahead may touch), the step
  // scalars {alpha, beta, k.q, v[row]} [N + 1][8], G [N]; with DLY also, in
  // accepted-path order, the previous record's k rows widened to FP32
  // [Np][dk] and the commit coefficients e^{G_last - G_p} u'_p[row] [Np][8]
  extern __shared__ f32x4 lds4[];
  const int cpr = dk / 4;
  const int cpu = dk / EPC;  // 16-byte units per row
  f32x4* ssc = lds4;                                            // [N + 1][8]
  SK* skq = reinterpret_cast<SK*>(ssc + (N + 1) * kChainRows);  // [N + 1][2][cpr]
  f32x4* skp = reinterpret_cast<f32x4*>(skq + (N + 1) * 2 * cpr);
  float* sG = reinterpret_cast<float*>(skp + (DLY ? Np * cpr : 0));
  float* scp = sG + N;

  const int tid = threadIdx.x;
  const int s = tid & 63;   // lane: columns 4s .. 4s + 3 of the wave's row
  const int rl = tid >> 6;  // row within the tile (0..7)
  const int tile = blockIdx.x % ntiles;
  const int bh = blockIdx.x / ntiles;
  const int h = bh % H;
  const int b = bh / H;
  const int r0 = tile * kChainRows;
  const int row = r0 + rl;
  const bool rok = row < dv;
  const bool cok = FULL || s < cpr;
  const int sc = FULL ? s : clampi(s, cpr - 1);
  auto kidx = [&](int t) { return 2 * t * cpr + sc; };  // k chunk of node t; q is cpr further
  auto qidx = [&](int t) { return (2 * t + 1) * cpr + sc; };

  // k and q rows in 16-byte units: unit u = node t's unit c of k (c < cpu) or
  // of q (c - cpu)
  const int kq_units = 2 * N * cpu;
  auto kq_load = [&](int u) {
    u = clampi(u, kq_units - 1);
    const int t = u / (2 * cpu), l = u % (2 * cpu);
    const T* src = l < cpu ? k : q;
    const int c = l < cpu ? l : l - cpu;
    return *reinterpret_cast<const u32x4*>(src + (((size_t)b * N + t) * H + h) * dk + c * EPC);
  };
  // k_t . q_t (the same for every row), stored for all 8 rows by lanes 0..7
  auto kq_put = [&](int t, float a) {
    if (s < kChainRows) reinterpret_cast<float*>(&ssc[t * kChainRows + s])[2] = a;
  };
  // No branch around the stores (a load used only under one is sunk into it
  // and waited for together with everything issued before): past the end a
  // thread rewrites the clamped unit with the bits it loaded for it, which
  // are the owner's bits.
  auto kq_store = [&](int u0, const u32x4& x) {
    const int u = clampi(u0, kq_units - 1);
    const int t = u / (2 * cpu), l = u % (2 * cpu);
    const int slot = 2 * t + (l < cpu ? 0 : 1), c = l < cpu ? l : l - cpu;
    SK* dst = skq + slot * cpr + c * E4;
    // q staged as FP32 carries the query scale (applied once here, not per step)
    const float qs = (QF && slot % 2 == 1) ? scale : 1.f;
    if constexpr (sizeof(T) == 4) {
      dst[0] = __builtin_bit_cast(f32x4, x) * qs;
    } else if constexpr (QF) {
      dst[0] = widen4(u32x2{x.x, x.y}) * qs;
      dst[1] = widen4(u32x2{x.z, x.w}) * qs;
    } else {
      dst[0] = stage_cvt(u32x2{x.x, x.y}, (SK*)nullptr);
      dst[1] = stage_cvt(u32x2{x.z, x.w}, (SK*)nullptr);
    }
    if constexpr (KQR) {
      if (u0 - s < kq_units) {  // uniform: the wave holds node t's k (lanes < 32) and q
        // v_permlane32_swap gives every lane both unit c's k and q (symmetric
        // in the halves), so each half forms the whole product
        float a = 0.f, a2 = 0.f;
        u32x4 kk, qq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned own = x[e];
          unsigned cp;
          asm("" : "=v"(cp) : "0"(own));
          const auto r = __builtin_amdgcn_permlane32_swap(own, cp, false, false);
          kk[e] = r[0];
          qq[e] = r[1];
        }
        const f32x4 k0 = widen4(u32x2{kk.x, kk.y}), k1 = widen4(u32x2{kk.z, kk.w});
        const f32x4 q0 = widen4(u32x2{qq.x, qq.y}), q1 = widen4(u32x2{qq.z, qq.w});
        a = k0.x * q0.x;
        a2 = k0.y * q0.y;
        a = fmaf(k0.z, q0.z, a);
        a2 = fmaf(k0.w, q0.w, a2);
        a = fmaf(k1.x, q1.x, a);
        a2 = fmaf(k1.y, q1.y, a2);
        a = fmaf(k1.z, q1.z, a);
        a2 = fmaf(k1.w, q1.w, a2);
        kq_put(t, (QF ? scale : 1.f) * half32_sum(a + a2));
      }
    }
  };

  // ---- every global load first (unconditional, clamped), in the order they
  // are consumed (loads complete in issue order): the first k and q units,
  // then the state row, whose HBM latency the staging overlaps, then what
  // each wave needs for its own row after the barrier (g, beta and v of every
  // node, lane t holding node t), and last the previous record, whose
  // pointers come with the fetched arguments.  Every wave-wide load costs the
  // same issue time whatever its width, and a load under a branch makes the
  // count of outstanding loads uncertain (the compiler then waits for all),
  // so there are few loads and none conditional.
  u32x4 kq0[KB];
#pragma unroll
  for (int x = 0; x < KB; ++x) kq0[x] = kq_load(tid + NT * x);
  f32x4 Sx;
  __builtin_amdgcn_sched_barrier(0);
  Sx = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S0 + ((size_t)bh * dv + clampi(row, dv - 1)) * dk + 4 * sc));
  __builtin_amdgcn_sched_barrier(0);
  const int cs = clampi(s, N - 1);
  const size_t nhl = ((size_t)b * N + cs) * H + h;
  const float gl = g[nhl];
  const float bl = beta[nhl];
  const T vb = v[nhl * dv + clampi(row, dv - 1)];
  // the previous draft's record (delayed commit): k rows, and u' of this row
  // and G of node s in lane s, none of which depends on last_accepted; its
  // pointers pass through an empty asm first, since the compiler would
  // otherwise copy them (and wait for their fetch) before the loads above
  const int kp_units = Np * cpu;
  u32x4 kp0 = u32x4{0u, 0u, 0u, 0u};
  float gnp = 0.f, upb = 0.f;
  uint64_t mlp = 0;
  if (DLY) {
    uint32_t z = 0;
    asm volatile("" : "+s"(z));
    Np += z;
    prev.mask += z;
    prev.G += z;
    prev.up += z;
    prev.K += z;
    last_acc += z;
    kp0 = *reinterpret_cast<const u32x4*>(prev.K + ((size_t)bh * Np) * dk +
                                          (size_t)clampi(tid, kp_units - 1) * EPC);
    const int ns = clampi(s, Np - 1);
    mlp = prev.mask[(size_t)b * Np + ns];
    gnp = prev.G[(size_t)bh * Np + ns];
    upb = prev.up[((size_t)bh * Np + ns) * dv + clampi(row, dv - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- LDS writes read by other waves: k and q (and k . q), and the
  // previous record's path k rows
#pragma unroll
  for (int x = 0; x < KB; ++x) kq_store(tid + NT * x, kq0[x]);
  for (int base = tid + NT * KB; base < kq_units; base += NT) kq_store(base, kq_load(base));

  // the previous draft's accepted path (bit i: node i), its length, G_last and
  // e^{G_last} (wave-uniform: last_accepted by a scalar load, the rest read
  // from lane `last` of the per-node loads)
  int last = -1, npath = 0;
  uint64_t pm = 0;
  float Glast = 0.f, s0 = 1.f;
  if (DLY) {
    last = last_acc[b];
    const bool in_rng = last >= 0 && last < Np;
    const int lc = in_rng ? last : 0;
    const uint32_t mlo = __builtin_amdgcn_readlane((uint32_t)mlp, lc);
    const uint32_t mhi = __builtin_amdgcn_readlane((uint32_t)(mlp >> 32), lc);
    const uint64_t valid = Np >= 64 ? ~0ull : ((1ull << Np) - 1ull);
    pm = in_rng ? ((((uint64_t)mhi << 32) | mlo) & valid) : 0ull;
    npath = __popcll(pm);
    Glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gnp), lc));
    s0 = expf(Glast);
  }
  auto rank = [&](int node) { return __popcll(pm & ((1ull << node) - 1ull)); };
  auto on_path = [&](int node) { return ((pm >> node) & 1ull) != 0ull; };

  if (DLY) {
    // path nodes' k rows, widened, packed in path order
    auto kp_store = [&](int j, const u32x4& x) {
      const int node = j / cpu, c = j % cpu;
      if (j < kp_units && on_path(node)) {
        f32x4* dst = skp + rank(node) * cpr + c * E4;
        if constexpr (sizeof(T) == 4) {
          dst[0] = __builtin_bit_cast(f32x4, x);
        } else {
          dst[0] = widen4(u32x2{x.x, x.y});
          dst[1] = widen4(u32x2{x.z, x.w});
        }
      }
    };
    kp_store(tid, kp0);
    for (int j = tid + NT; j < kp_units; j += NT)
      kp_store(j, *reinterpret_cast<const u32x4*>(prev.K + ((size_t)bh * Np) * dk + (size_t)j * EPC));
  }
  __syncthreads();

  // ---- LDS writes read only by this wave (its row): the step scalars of node
  // s, and with DLY the commit coefficient of path node s for this row (the
  // commit kernel's expression, e^{G_last - G_s} u'_s[row]), in path order
  if (s < N) {
    float* e = reinterpret_cast<float*>(&ssc[s * kChainRows + rl]);
    e[0] = expf(gl);
    e[1] = bl;
    e[3] = rok ? widen1(vb) : 0.f;
    if (rl == 0) sG[s] = gl;
  }
  if (DLY && s < Np && on_path(s))
    scp[rank(s) * kChainRows + rl] = expf(Glast - gnp) * upb;

  if (!KQR) {
    // ---- k_t . q_t from LDS: wave rl takes nodes rl, rl + 8, ...
    for (int t = rl; t < N; t += kChainRows) {
      const f32x4 kx = mask4(widen4(skq[kidx(t)]), cok);
      const f32x4 qx = mask4(widen4(skq[qidx(t)]), cok);
      float a = kx.x * qx.x;
      float a2 = kx.y * qx.y;
      a = fmaf(kx.z, qx.z, a);
      a2 = fmaf(kx.w, qx.w, a2);
      kq_put(t, wave64_sum(a + a2));
    }
  }

  // the state row (first needed here)
  const f32x4 Sm = mask4(Sx, rok && cok);
  float S[4] = {Sm.x, Sm.y, Sm.z, Sm.w};

  if (DLY) {
    // ---- the previous draft's accepted path: S <- e^{G_last} S + sum c_p k_p^T,
    // path nodes in increasing order, four at a time (the LDS reads of a group
    // are issued before its multiply-adds)
    const bool okp = last >= 0 && last < Np && on_path(last);
    if (dev_status && tile == 0 && h == 0 && tid == 0)
      dev_status[b] = (last == -1 || okp) ? GDN_OK : GDN_ERR_TOPOLOGY;
    if (okp) {  // uniform
#pragma unroll
      for (int e = 0; e < 4; ++e) S[e] = S[e] * s0;
      auto apply = [&](int i, auto K) {
        constexpr int KN = decltype(K)::value;
        float c[KN];
        f32x4 kc[KN];
#pragma unroll
        for (int u = 0; u < KN; ++u) {
          c[u] = scp[(i + u) * kChainRows + rl];
          kc[u] = skp[(i + u) * cpr + sc];
        }
#pragma unroll
        for (int u = 0; u < KN; ++u) {
          S[0] = fmaf(c[u], kc[u].x, S[0]);
          S[1] = fmaf(c[u], kc[u].y, S[1]);
          S[2] = fmaf(c[u], kc[u].z, S[2]);
          S[3] = fmaf(c[u], kc[u].w, S[3]);
        }
      };
      int i = 0;
      for (; i + 4 <= npath; i += 4) apply(i, std::integral_constant<int, 4>());
      switch (npath - i) {
        case 3: apply(i, std::integral_constant<int, 3>()); break;
        case 2: apply(i, std::integral_constant<int, 2>()); break;
        case 1: apply(i, std::integral_constant<int, 1>()); break;
        default: break;
      }
      if (rok && cok)
        __builtin_nontemporal_store(f32x4{S[0], S[1], S[2], S[3]}, reinterpret_cast<f32x4*>(S0 + ((size_t)bh * dv + row) * dk + 4 * s));
    }
  }
  if (!KQR) __syncthreads();  // k.q of every node is in LDS

  // ---- the recurrence.  Operands of step t (k_t, q_t chunks and the step
  // scalars) are read from LDS during step t - 1; two register sets
  // alternate.  The read-ahead past the last node lands in the padding node.
  struct Ops {
    f32x4 kc, qc, sc;  // sc = {alpha, beta, k.q, v[row]}
  };
  const SK* kq_lane = skq + sc;
  const f32x4* sc_row = ssc + rl;
  // operands of the next step in order (steps are fetched 0, 1, 2, ...)
  const SK* kq_next = kq_lane;
  const f32x4* sc_next = sc_row;
  auto fetch = [&](Ops& o) {
    o.kc = mask4(widen4(kq_next[0]), cok);
    o.qc = mask4(widen4(kq_next[cpr]), cok);
    o.sc = sc_next[0];
    kq_next += 2 * cpr;
    sc_next += kChainRows;
  };
  // lane 63 holds y_q and stores the step's output and u'; the row is the
  // wave's, so the pointers are wave-uniform (scalar registers, scalar
  // increments)
  const int rlu = __builtin_amdgcn_readfirstlane(rl);
  float* op = out + (size_t)b * N * H * dv + (size_t)h * dv + r0 + rlu;
  float* up = rec.up + (size_t)bh * N * dv + r0 + rlu;
  const size_t ostep = (size_t)H * dv;
  const bool store_lane = s == 63 && rok;
  auto run = [&](const Ops& o) {
    const float al = o.sc.x, be = o.sc.y, kq = o.sc.z, vt = o.sc.w;
    // one multiply-add chain per dot product (the loop is bound by VALU issue,
    // not by this latency)
    float yk = S[0] * o.kc.x;
    float yq = S[0] * o.qc.x;
    yk = fmaf(S[1], o.kc.y, yk);
    yq = fmaf(S[1], o.qc.y, yq);
    yk = fmaf(S[2], o.kc.z, yk);
    yq = fmaf(S[2], o.qc.z, yq);
    yk = fmaf(S[3], o.kc.w, yk);
    yq = fmaf(S[3], o.qc.w, yq);
    wave64_sum2_uniform(yk, yq, yk, yq);  // both wave-uniform
    const float u = be * (vt - al * yk);
    S[0] = fmaf(u, o.kc.x, al * S[0]);
    S[1] = fmaf(u, o.kc.y, al * S[1]);
    S[2] = fmaf(u, o.kc.z, al * S[2]);
    S[3] = fmaf(u, o.kc.w, al * S[3]);
    if (store_lane) {
      const float ov = fmaf(kq, u, al * yq);  // q (and k.q) carry the scale when staged as FP32
      *op = QF ? ov : scale * ov;
      *up = u;
    }
    op += ostep;
    up += dv;
  };
  // The prefetched operands pass through an empty asm after the step that
  // overlaps their reads: the values carried around the loop are then not
  // loads, which the optimiser would otherwise re-issue at the top of the
  // next step (folding a phi of loads into a load) and wait for at once.
  auto opaque = [](Ops& o) {
    asm volatile("" : "+v"(o.kc));
    asm volatile("" : "+v"(o.qc));
    asm volatile("" : "+v"(o.sc));
  };
  Ops A, Bo;
  fetch(A);
  opaque(A);
  for (int t = 0; t < N; t += 2) {
    fetch(Bo);
    run(A);
    opaque(Bo);
    if (t + 1 < N) {  // uniform
      fetch(A);
      run(Bo);
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
    for (int idx = tid; idx < N * cpr; idx += NT)  // from the staged rows in LDS
      *reinterpret_cast<R4*>(rec.K + ((size_t)bh * N + idx / cpr) * dk + 4 * (idx % cpr)) =
          unstage(skq[2 * (idx / cpr) * cpr + idx % cpr], (T*)nullptr);
    if (h == 0 && tid < N) {
      rec.parents[(size_t)b * N + tid] = tid - 1;
      rec.mask[(size_t)b * N + tid] = tid >= 63 ? ~0ull : ((1ull << (tid + 1)) - 1ull);
    }
  }
}

// k, q staged as FP32 for drafts of up to 32 nodes (bf16 beyond, to bound LDS)
bool chain_staged_f32(int N, int dtype) { return dtype == GDN_F32 || N <= 32; }

// Dynamic LDS of one workgroup (the layout at the top of the kernel); Np = 0
// without a previous record.
size_t chain_lds_bytes(int N, int Np, int dk, int dtype) {
  const size_t el = dtype == GDN_BF16 ? 2 : 4;
  const size_t st = chain_staged_f32(N, dtype) ? 4 : el;
  return (size_t)(N + 1) * kChainRows * 16 + (size_t)(N + 1) * 2 * dk * st +
         (size_t)Np * dk * 4 + (size_t)N * 4 + (size_t)Np * kChainRows * 4;
}

template <typename T, bool DLY, bool QF, bool FULL, int KB>
void launch_chain_kb(long grid, size_t lds, hipStream_t stream, uint32_t shape, int H, float* S0,
                     const T* q, const T* k, const T* v, const float* beta, const float* g,
                     float scale, float* out, const Record<T>& rec, const Record<T>& prev,
                     int Np, const int32_t* last, int32_t* dev_status) {
  hipLaunchKernelGGL((chain_verify_kernel<T, DLY, QF, FULL, KB>), dim3((unsigned)grid),
                     dim3(kChainThreads), lds, stream, shape, H, k, q, g, beta, v, S0, scale, out,
                     rec, prev, Np, last, dev_status);
}

// KB: 16-byte k/q units per thread in the first round of loads (one when a
// draft's k and q fit in one unit per thread, else four; more are looped)
template <typename T, bool DLY, bool QF>
void launch_chain_qf(bool full, long grid, size_t lds, hipStream_t stream, int N, int H, int dk,
                     int dv, float* S0, const T* q, const T* k, const T* v, const float* beta,
                     const float* g, float scale, float* out, const Record<T>& rec,
                     const Record<T>& prev, int Np, const int32_t* last, int32_t* dev_status) {
  const uint32_t shape = (uint32_t)N | ((uint32_t)dk << 8) | ((uint32_t)dv << 18);
  const bool one = 2L * N * dk * (long)sizeof(T) <= 16L * kChainThreads;
#define GDN_CHAIN_LAUNCH(FULLV, KBV)                                                           \
  launch_chain_kb<T, DLY, QF, FULLV, KBV>(grid, lds, stream, shape, H, S0, q, k, v, beta, g,   \
                                          scale, out, rec, prev, Np, last, dev_status)
  if (full) {
    if (one) GDN_CHAIN_LAUNCH(true, 1); else GDN_CHAIN_LAUNCH(true, 4);
  } else {
    if (one) GDN_CHAIN_LAUNCH(false, 1); else GDN_CHAIN_LAUNCH(false, 4);
  }
#undef GDN_CHAIN_LAUNCH
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
  const bool qf = chain_staged_f32(N, sizeof(T) == 2 ? GDN_BF16 : GDN_F32);
  const bool full = dk == kMaxDim;
  const int ntiles = (dv + kChainRows - 1) / kChainRows;
  const long grid = (long)B * H * ntiles;
  const size_t lds = chain_lds_bytes(N, Np, dk, sizeof(T) == 2 ? GDN_BF16 : GDN_F32);
  if (lds > (size_t)kMaxLds) return hipErrorInvalidValue;
  const T* qq = static_cast<const T*>(q);
  const T* kk = static_cast<const T*>(k);
  const T* vv = static_cast<const T*>(v);
  if (dly) {
    if (qf)
      launch_chain_qf<T, true, true>(full, grid, lds, stream, N, H, dk, dv, S0, qq, kk,
                                     vv, beta, g, scale, out, rec, prev, Np, last, dev_status);
    else
      launch_chain_qf<T, true, false>(full, grid, lds, stream, N, H, dk, dv, S0, qq, kk,
                                      vv, beta, g, scale, out, rec, prev, Np, last, dev_status);
  } else {
    if (qf)
      launch_chain_qf<T, false, true>(full, grid, lds, stream, N, H, dk, dv, S0, qq, kk,
                                      vv, beta, g, scale, out, rec, prev, 0, nullptr, nullptr);
    else
      launch_chain_qf<T, false, false>(full, grid, lds, stream, N, H, dk, dv, S0, qq, kk,
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
