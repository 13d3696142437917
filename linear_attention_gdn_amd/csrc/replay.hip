// Replay baselines (gfx950): the two mechanisms the factorized verifier and
// the factor-buffer commit replace, as state-resident serial kernels.
//
// SpecLA review, Referee Report major comment 3 and Figures, Figures 10 and
// 11 captions (the desk editor's letter on the verdict page quotes the same
// ratios): tree verification is compared against replaying every
// root-to-leaf path of the draft with a serial recurrence, and the
// accepted-state recovery against replaying the accepted tokens through the
// recurrence.  These kernels are those replays on this GPU, so the two
// ratios can be measured here:
//   replay_verify: one workgroup per (sequence, head, 8 state rows, path):
//     walks the root path of the path's end node and runs
//         y_k = S k_t, u = beta_t (v_t - alpha_t y_k), S <- alpha_t S + u k_t^T,
//         o_t = scale (alpha_t S_old q_t + (k_t . q_t) u)
//     node by node from S0, writing o_t for the nodes the path owns (those on
//     no earlier path of the list); S0 is read only.
//   replay_commit: one workgroup per (sequence, head, 8 state rows): the same
//     recurrence along the accepted path (no outputs), then the rows written
//     back in place.
// Mapping as in the chain kernel: 8 waves per workgroup, wave w owns state row
// w of the tile, lane s columns 4s .. 4s + 3, so a step is two (three)
// wave-wide dot products and a rank-1 update in registers.  The next node's
// k, q and scalars are requested while the current node computes.
#include "gdn_common.h"

namespace gdn {

constexpr int kReplayRows = 8;
constexpr int kReplayThreads = 512;

template <typename T, bool VERIFY>
__global__ __launch_bounds__(kReplayThreads) void replay_kernel(
    int N, int H, int dk, int dv, int ntiles, int P, float* __restrict__ S,
    const int32_t* __restrict__ parents, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const float* __restrict__ beta, const float* __restrict__ g,
    float scale, const int32_t* __restrict__ ends, float* __restrict__ out,
    int32_t* __restrict__ dev_status) {
  __shared__ int spar[kMaxNodes];
  __shared__ uint64_t spath[kMaxNodes];  // VERIFY: path mask of every slot
  const int tid = threadIdx.x;
  const int s = tid & 63;
  const int wave = tid >> 6;
  const int tile = blockIdx.x % ntiles;
  const int bh = blockIdx.x / ntiles;
  const int h = bh % H;
  const int b = bh / H;
  const int slot = blockIdx.y;
  const int row = tile * kReplayRows + wave;
  const bool rok = row < dv;
  const int rowc = clampi(row, dv - 1);
  const bool cok = 4 * s < dk;
  const int col = clampi(4 * s, dk - 4);

  // parents (lane j holds node j) and the topology check of the whole draft
  const int pj = parents[(size_t)b * N + clampi(s, N - 1)];
  const bool bad = __ballot(s < N && (pj < -1 || pj >= s)) != 0ull;
  if (tid < kMaxNodes) spar[tid] = pj;
  const int end = VERIFY ? ends[(size_t)b * P + slot] : ends[b];
  // every end of the sequence in -1..N-1 (lane j: slot j)
  const int ej = VERIFY ? ends[(size_t)b * P + clampi(s, P - 1)] : end;
  const bool bad_end = __ballot(s < P && (ej < -1 || ej >= N)) != 0ull;
  if (dev_status && tile == 0 && h == 0 && slot == 0 && tid == 0)
    dev_status[b] = (bad || bad_end) ? GDN_ERR_TOPOLOGY : GDN_OK;
  __syncthreads();
  // nothing to replay: a rejected topology, an empty or out-of-range path
  if (bad || end < 0 || end >= N) return;  // uniform over the workgroup

  // root path of `end` as a bit mask (ancestors have smaller indices, so the
  // set bits in increasing order are the path root first)
  auto path_of = [&](int e) {
    uint64_t m = 0ull;
    for (int t = e; t >= 0; t = spar[t]) m |= 1ull << t;
    return m;
  };
  const uint64_t m = path_of(end);
  uint64_t own = m;
  if (VERIFY) {
    // a node's output is written by the first slot whose path holds it
    if (tid < P && tid < kMaxNodes) {
      const int e = ends[(size_t)b * P + tid];
      spath[tid] = (e >= 0 && e < N) ? path_of(e) : 0ull;
    }
    __syncthreads();
    uint64_t prior = 0ull;
    for (int j = 0; j < slot && j < kMaxNodes; ++j) prior |= spath[j];  // uniform
    own = m & ~prior;
  }

  float* srow = S + ((size_t)bh * dv + rowc) * dk + col;
  const f32x4 S0 = mask4(load4(srow), rok && cok);
  float Sr[4] = {S0.x, S0.y, S0.z, S0.w};

  // operands of node t: k, q (4 columns per lane), alpha's log, beta, v[row]
  struct Ops {
    typename Raw4<T>::type kr, qr;
    float gl, bl;
    T vr;
  };
  auto fetch = [&](int t, Ops& o) {
    const size_t nh = ((size_t)b * N + t) * H + h;
    o.kr = raw4(k + nh * dk + col);
    if (VERIFY) o.qr = raw4(q + nh * dk + col);
    o.gl = g[nh];
    o.bl = beta[nh];
    o.vr = v[nh * dv + rowc];
  };
  uint64_t rest = m;
  Ops cur;
  fetch(__builtin_ctzll(rest), cur);
  while (rest) {  // uniform
    const int t = __builtin_ctzll(rest);
    rest &= rest - 1ull;
    Ops nxt;
    fetch(rest ? __builtin_ctzll(rest) : t, nxt);  // in flight while node t computes
    const f32x4 kx = mask4(widen4(cur.kr), cok);
    const float al = expf(cur.gl);
    float yk = Sr[0] * kx.x;
    yk = fmaf(Sr[1], kx.y, yk);
    yk = fmaf(Sr[2], kx.z, yk);
    yk = fmaf(Sr[3], kx.w, yk);
    yk = wave64_sum(yk);
    const float u = cur.bl * ((rok ? widen1(cur.vr) : 0.f) - al * yk);
    if (VERIFY && ((own >> t) & 1ull)) {  // uniform
      const f32x4 qx = mask4(widen4(cur.qr), cok);
      float yq = Sr[0] * qx.x;
      float kq = kx.x * qx.x;
      yq = fmaf(Sr[1], qx.y, yq);
      kq = fmaf(kx.y, qx.y, kq);
      yq = fmaf(Sr[2], qx.z, yq);
      kq = fmaf(kx.z, qx.z, kq);
      yq = fmaf(Sr[3], qx.w, yq);
      kq = fmaf(kx.w, qx.w, kq);
      yq = wave64_sum(yq);
      kq = wave64_sum(kq);
      if (s == 0 && rok)
        out[(((size_t)b * N + t) * H + h) * dv + row] = scale * fmaf(kq, u, al * yq);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Sr[e] = fmaf(u, kx[e], al * Sr[e]);
    cur = nxt;
  }
  if (!VERIFY && rok && cok)
    *reinterpret_cast<f32x4*>(srow) = f32x4{Sr[0], Sr[1], Sr[2], Sr[3]};
}

template <typename T>
hipError_t launch_replay_t(bool verify, int B, int N, int H, int dk, int dv, float* S,
                           const int32_t* parents, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, float scale, const int32_t* ends,
                           int P, float* out, int32_t* dev_status, hipStream_t stream) {
  const int ntiles = (dv + kReplayRows - 1) / kReplayRows;
  const dim3 grid((unsigned)((long)B * H * ntiles), verify ? (unsigned)P : 1u);
  const T* qq = static_cast<const T*>(q);
  const T* kk = static_cast<const T*>(k);
  const T* vv = static_cast<const T*>(v);
  if (verify)
    hipLaunchKernelGGL((replay_kernel<T, true>), grid, dim3(kReplayThreads), 0, stream, N, H, dk,
                       dv, ntiles, P, S, parents, qq, kk, vv, beta, g, scale, ends, out,
                       dev_status);
  else
    hipLaunchKernelGGL((replay_kernel<T, false>), grid, dim3(kReplayThreads), 0, stream, N, H,
                       dk, dv, ntiles, 1, S, parents, qq, kk, vv, beta, g, scale, ends, nullptr,
                       dev_status);
  return hipGetLastError();
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

}  // namespace gdn
