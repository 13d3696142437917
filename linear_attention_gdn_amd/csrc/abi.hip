// extern "C" entry points of libgdnspec: argument validation, error text and
// dispatch to the gfx950 kernels.  Every check here runs on the host before
// anything is enqueued; nothing is allocated.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "gdn_common.h"
#include "../../include/gdnlayer.h"
#include "../../include/gdnnext.h"

namespace gdn {
size_t chain_lds_bytes(int N, int Np, int dk, int dtype);
hipError_t launch_chain_verify(int B, int N, int H, int dk, int dv, int dtype, float* S0,
                               const void* q, const void* k, const void* v, const float* beta,
                               const float* g, float scale, float* out, void* factors,
                               const void* prev_factors, int Np, const int32_t* last,
                               int32_t* dev_status, hipStream_t stream);
hipError_t launch_tree_verify(int B, int N, int H, int dk, int dv, int dtype, float* S0,
                              const int32_t* parents, const void* q, const void* k,
                              const void* v, const float* beta, const float* g, float scale,
                              float* out, void* factors, void* workspace, uint64_t* mask_out,
                              int32_t* dev_status, const void* prev_factors, int Np,
                              const int32_t* last, int32_t* commit_status, const float* gate,
                              int ldg, void* Y, hipStream_t stream);
hipError_t launch_commit(int B, int N, int H, int dk, int dv, int dtype, float* S,
                         const void* factors, const int32_t* last, int32_t* path_out,
                         int32_t* path_len, int32_t* dev_status, hipStream_t stream);
hipError_t launch_linear(int M, int Nc, int K, const void* A, const void* W, int layout,
                         const float* R, float* C, void* Cb, hipStream_t stream);
hipError_t launch_pack_weights(int Nc, int K, const void* W, void* Wp, hipStream_t stream);
hipError_t launch_layer_prep(int B, int N, int H, int dk, int dv, int D, const float* P,
                             const void* x, const void* W_ab, const int32_t* parents,
                             const float* conv_w, const float* hist, float gate_shift, void* q,
                             void* k, void* v, float* beta, float* g, const float* P_prev,
                             int Np, const int32_t* parents_prev, const int32_t* last_prev,
                             float* hist_out, int32_t* dev_status, hipStream_t stream);
hipError_t launch_gate_merge(int M, int Cw, const float* o, const float* gate, int ldg, void* Y,
                             hipStream_t stream);
hipError_t launch_conv_commit(int B, int N, int Cc, const float* P, int ldP,
                              const int32_t* parents, const int32_t* last, float* hist,
                              int32_t* dev_status, hipStream_t stream);
hipError_t launch_decode_step(int B, int H, int dk, int dv, int dtype, float* S, const void* q,
                              const void* k, const void* v, const float* beta, const float* g,
                              float scale, float* out, hipStream_t stream);
hipError_t launch_hybrid(int B, int N, int H, int dk, int dv, int dtype, const float* S0,
                         const int32_t* parents, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, float scale, float* out,
                         void* factors, const int32_t* plan, int levels,
                         const int32_t* chains_per_level, int32_t* dev_status,
                         hipStream_t stream);
int hybrid_plan(int B, int N, const int32_t* parents, int32_t* plan, int32_t* chains_per_level);
hipError_t launch_prune(int B, int M, int T, float tau, const int32_t* parents, const float* conf,
                        int32_t* kept, int32_t* new_parents, int32_t* count, int32_t* dev_status,
                        hipStream_t stream);
hipError_t launch_replay(bool verify, int B, int N, int H, int dk, int dv, int dtype, float* S,
                         const int32_t* parents, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, float scale, const int32_t* ends,
                         int P, float* out, int32_t* dev_status, hipStream_t stream);
}  // namespace gdn

namespace {

thread_local std::string g_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return status;
}

int ok() {
  g_error.clear();
  return GDN_OK;
}

bool sizes_ok(int B, int N, int H, int dk, int dv) {
  return B >= 0 && N >= 0 && N <= gdn::kMaxNodes && H >= 1 && dk >= 8 && dk <= gdn::kMaxDim &&
         dk % 8 == 0 && dv >= 4 && dv <= gdn::kMaxDim && dv % 4 == 0 &&
         (long long)B * H * N * gdn::kMaxDim < (1ll << 40);
}

int check_sizes(const char* fn, int B, int N, int H, int dk, int dv) {
  if (!sizes_ok(B, N, H, dk, dv))
    return fail(GDN_ERR_SHAPE,
                "%s: unsupported sizes B=%d N=%d H=%d dk=%d dv=%d (need B>=0, 0<=N<=64, H>=1, "
                "8<=dk<=256 with dk%%8==0, 4<=dv<=256 with dv%%4==0)",
                fn, B, N, H, dk, dv);
  return GDN_OK;
}

int check_dtype(const char* fn, int dtype) {
  if (dtype != GDN_BF16 && dtype != GDN_F32)
    return fail(GDN_ERR_ARG, "%s: qkv_dtype %d is neither GDN_BF16 (0) nor GDN_F32 (1)", fn,
                dtype);
  return GDN_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, bool required) {
  if (!p) {
    if (required) return fail(GDN_ERR_ARG, "%s: %s is NULL", fn, name);
    return GDN_OK;
  }
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(GDN_ERR_ARG, "%s: %s is not 16-byte aligned", fn, name);
  return GDN_OK;
}

int check_ptr4(const char* fn, const char* name, const void* p, bool required) {
  if (!p) {
    if (required) return fail(GDN_ERR_ARG, "%s: %s is NULL", fn, name);
    return GDN_OK;
  }
  if (reinterpret_cast<uintptr_t>(p) % 4 != 0)
    return fail(GDN_ERR_ARG, "%s: %s is not 4-byte aligned", fn, name);
  return GDN_OK;
}

// One chain workgroup stages the draft (and the previous record) in LDS.
int check_chain_lds(const char* fn, int N, int N_prev, int dk, int dtype) {
  const size_t need = gdn::chain_lds_bytes(N, N_prev, dk, dtype);
  if (need > (size_t)gdn::kMaxLds)
    return fail(GDN_ERR_UNSUPPORTED,
                "%s: N=%d, N_prev=%d, dk=%d with %s inputs needs %zu bytes of LDS per workgroup "
                "(limit %d); use bf16 inputs or smaller drafts",
                fn, N, N_prev, dk, dtype == GDN_BF16 ? "bf16" : "fp32", need, gdn::kMaxLds);
  return GDN_OK;
}

int hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess)
    return fail(GDN_ERR_HIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
  return ok();
}

#define GDN_TRY(expr)          \
  do {                         \
    const int _rc = (expr);    \
    if (_rc != GDN_OK) return _rc; \
  } while (0)

}  // namespace

extern "C" {

int gdn_version(void) { return (0 << 16) | 1; }

const char* gdn_last_error(void) { return g_error.c_str(); }

size_t gdn_factor_bytes(int B, int N, int H, int dk, int dv, int qkv_dtype) {
  if (!sizes_ok(B, N, H, dk, dv) || (qkv_dtype != GDN_BF16 && qkv_dtype != GDN_F32)) return 0;
  return gdn::record_layout(B, N, H, dk, dv, qkv_dtype).total;
}

int gdn_factor_layout(int B, int N, int H, int dk, int dv, int qkv_dtype, size_t offsets[5]) {
  GDN_TRY(check_sizes("gdn_factor_layout", B, N, H, dk, dv));
  GDN_TRY(check_dtype("gdn_factor_layout", qkv_dtype));
  if (!offsets) return fail(GDN_ERR_ARG, "gdn_factor_layout: offsets is NULL");
  const gdn::RecordLayout L = gdn::record_layout(B, N, H, dk, dv, qkv_dtype);
  for (int i = 0; i < 5; ++i) offsets[i] = L.off[i];
  return ok();
}

size_t gdn_workspace_bytes(int B, int N, int H, int dk, int dv) {
  (void)B; (void)N; (void)H; (void)dk; (void)dv;
  return 0;  // the fused tree kernel keeps all per-head factors in LDS
}

int gdn_tree_verify(int B, int N, int H, int dk, int dv, int qkv_dtype, const float* S0,
                    const int32_t* parents, const void* q, const void* k, const void* v,
                    const float* beta, const float* g, float scale, float* out, void* factors,
                    void* workspace, uint64_t* mask_out, int32_t* dev_status, void* stream) {
  const char* fn = "gdn_tree_verify";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  GDN_TRY(check_dtype(fn, qkv_dtype));
  if (!std::isfinite(scale)) return fail(GDN_ERR_ARG, "%s: scale is not finite", fn);
  if (B == 0 || N == 0) return ok();
  GDN_TRY(check_ptr(fn, "S0", S0, true));
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  GDN_TRY(check_ptr(fn, "out", out, true));
  GDN_TRY(check_ptr(fn, "factors", factors, true));
  GDN_TRY(check_ptr(fn, "workspace", workspace, false));
  GDN_TRY(check_ptr(fn, "mask_out", mask_out, false));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  return hip_status(fn, gdn::launch_tree_verify(B, N, H, dk, dv, qkv_dtype,
                                                const_cast<float*>(S0), parents, q, k, v, beta,
                                                g, scale, out, factors, workspace, mask_out,
                                                dev_status, nullptr, 0, nullptr, nullptr,
                                                nullptr, 0, nullptr,
                                                static_cast<hipStream_t>(stream)));
}

int gdn_tree_verify_delayed(int B, int N_prev, int N, int H, int dk, int dv, int qkv_dtype,
                            float* S, const void* prev_factors, const int32_t* last_accepted,
                            int32_t* commit_status, const int32_t* parents, const void* q,
                            const void* k, const void* v, const float* beta, const float* g,
                            float scale, float* out, void* factors, void* workspace,
                            uint64_t* mask_out, int32_t* dev_status, void* stream) {
  const char* fn = "gdn_tree_verify_delayed";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  if (N_prev < 1 || N_prev > gdn::kMaxNodes)
    return fail(GDN_ERR_SHAPE, "%s: N_prev=%d outside 1..64", fn, N_prev);
  GDN_TRY(check_dtype(fn, qkv_dtype));
  if (!std::isfinite(scale)) return fail(GDN_ERR_ARG, "%s: scale is not finite", fn);
  if (B == 0) return ok();
  if (N == 0)
    return fail(GDN_ERR_SHAPE, "%s: N=0; use gdn_commit_path to commit without verifying", fn);
  GDN_TRY(check_ptr(fn, "S", S, true));
  GDN_TRY(check_ptr(fn, "prev_factors", prev_factors, true));
  GDN_TRY(check_ptr4(fn, "last_accepted", last_accepted, true));
  GDN_TRY(check_ptr4(fn, "commit_status", commit_status, false));
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  GDN_TRY(check_ptr(fn, "out", out, true));
  GDN_TRY(check_ptr(fn, "factors", factors, true));
  GDN_TRY(check_ptr(fn, "workspace", workspace, false));
  GDN_TRY(check_ptr(fn, "mask_out", mask_out, false));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  const char* a0 = static_cast<const char*>(prev_factors);
  const char* b0 = static_cast<const char*>(factors);
  const size_t na = gdn::record_layout(B, N_prev, H, dk, dv, qkv_dtype).total;
  const size_t nb = gdn::record_layout(B, N, H, dk, dv, qkv_dtype).total;
  if (a0 < b0 + nb && b0 < a0 + na)
    return fail(GDN_ERR_ARG, "%s: factors and prev_factors overlap", fn);
  return hip_status(fn, gdn::launch_tree_verify(B, N, H, dk, dv, qkv_dtype, S, parents, q, k, v,
                                                beta, g, scale, out, factors, workspace,
                                                mask_out, dev_status, prev_factors, N_prev,
                                                last_accepted, commit_status, nullptr, 0,
                                                nullptr, static_cast<hipStream_t>(stream)));
}

int gdn_chain_verify(int B, int N, int H, int dk, int dv, int qkv_dtype, const float* S0,
                     const void* q, const void* k, const void* v, const float* beta,
                     const float* g, float scale, float* out, void* factors, void* stream) {
  const char* fn = "gdn_chain_verify";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  GDN_TRY(check_dtype(fn, qkv_dtype));
  if (!std::isfinite(scale)) return fail(GDN_ERR_ARG, "%s: scale is not finite", fn);
  if (B == 0 || N == 0) return ok();
  GDN_TRY(check_ptr(fn, "S0", S0, true));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  GDN_TRY(check_ptr(fn, "out", out, true));
  GDN_TRY(check_ptr(fn, "factors", factors, true));
  GDN_TRY(check_chain_lds(fn, N, 0, dk, qkv_dtype));
  return hip_status(fn, gdn::launch_chain_verify(B, N, H, dk, dv, qkv_dtype,
                                                 const_cast<float*>(S0), q, k, v, beta, g,
                                                 scale, out, factors, nullptr, 0, nullptr,
                                                 nullptr, static_cast<hipStream_t>(stream)));
}

int gdn_chain_verify_delayed(int B, int N_prev, int N, int H, int dk, int dv, int qkv_dtype,
                             float* S, const void* prev_factors, const int32_t* last_accepted,
                             int32_t* dev_status, const void* q, const void* k, const void* v,
                             const float* beta, const float* g, float scale, float* out,
                             void* factors, void* stream) {
  const char* fn = "gdn_chain_verify_delayed";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  if (N_prev < 1 || N_prev > gdn::kMaxNodes)
    return fail(GDN_ERR_SHAPE, "%s: N_prev=%d outside 1..64", fn, N_prev);
  GDN_TRY(check_dtype(fn, qkv_dtype));
  if (!std::isfinite(scale)) return fail(GDN_ERR_ARG, "%s: scale is not finite", fn);
  if (B == 0) return ok();
  if (N == 0)
    return fail(GDN_ERR_SHAPE, "%s: N=0; use gdn_commit_path to commit without verifying", fn);
  GDN_TRY(check_ptr(fn, "S", S, true));
  GDN_TRY(check_ptr(fn, "prev_factors", prev_factors, true));
  GDN_TRY(check_ptr4(fn, "last_accepted", last_accepted, true));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  GDN_TRY(check_ptr(fn, "out", out, true));
  GDN_TRY(check_ptr(fn, "factors", factors, true));
  const char* a0 = static_cast<const char*>(prev_factors);
  const char* b0 = static_cast<const char*>(factors);
  const size_t na = gdn::record_layout(B, N_prev, H, dk, dv, qkv_dtype).total;
  const size_t nb = gdn::record_layout(B, N, H, dk, dv, qkv_dtype).total;
  if (a0 < b0 + nb && b0 < a0 + na)
    return fail(GDN_ERR_ARG, "%s: factors and prev_factors overlap", fn);
  GDN_TRY(check_chain_lds(fn, N, N_prev, dk, qkv_dtype));
  return hip_status(fn, gdn::launch_chain_verify(B, N, H, dk, dv, qkv_dtype, S, q, k, v, beta, g,
                                                 scale, out, factors, prev_factors, N_prev,
                                                 last_accepted, dev_status,
                                                 static_cast<hipStream_t>(stream)));
}

int gdn_commit_path(int B, int N, int H, int dk, int dv, int qkv_dtype, float* S,
                    const void* factors, const int32_t* last_accepted, int32_t* path_out,
                    int32_t* path_len_out, int32_t* dev_status, void* stream) {
  const char* fn = "gdn_commit_path";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  GDN_TRY(check_dtype(fn, qkv_dtype));
  if (B == 0) return ok();
  GDN_TRY(check_ptr4(fn, "last_accepted", last_accepted, true));
  GDN_TRY(check_ptr4(fn, "path_len_out", path_len_out, false));
  GDN_TRY(check_ptr4(fn, "path_out", path_out, false));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  if (N == 0) return ok();  // only last_accepted = -1 is possible: nothing to apply
  GDN_TRY(check_ptr(fn, "S", S, true));
  GDN_TRY(check_ptr(fn, "factors", factors, true));
  return hip_status(fn, gdn::launch_commit(B, N, H, dk, dv, qkv_dtype, S, factors,
                                           last_accepted, path_out, path_len_out, dev_status,
                                           static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// layer scaffold (gdnlayer.h)
// ---------------------------------------------------------------------------

static int linear_sizes_ok(const char* fn, int M, int Nc, int K) {
  if (M < 0 || M > 64 || Nc < 0 || Nc % 16 != 0 || K < 256 || K > 65536 || K % 256 != 0)
    return fail(GDN_ERR_SHAPE,
                "%s: unsupported sizes M=%d Nc=%d K=%d (need 0<=M<=64, Nc%%16==0, "
                "256<=K<=65536 with K%%256==0)",
                fn, M, Nc, K);
  return GDN_OK;
}

int gdn_linear(int M, int Nc, int K, const void* A, const void* W, int w_layout, const float* R,
               float* C, void* C_bf16, void* stream) {
  const char* fn = "gdn_linear";
  GDN_TRY(linear_sizes_ok(fn, M, Nc, K));
  if (w_layout != GDN_W_ROWS && w_layout != GDN_W_PACKED)
    return fail(GDN_ERR_ARG, "%s: w_layout %d is neither GDN_W_ROWS (0) nor GDN_W_PACKED (1)",
                fn, w_layout);
  if (!C && !C_bf16) return fail(GDN_ERR_ARG, "%s: C and C_bf16 are both NULL", fn);
  if (M == 0 || Nc == 0) return ok();
  GDN_TRY(check_ptr(fn, "A", A, true));
  GDN_TRY(check_ptr(fn, "W", W, true));
  GDN_TRY(check_ptr(fn, "R", R, false));
  GDN_TRY(check_ptr(fn, "C", C, false));
  GDN_TRY(check_ptr(fn, "C_bf16", C_bf16, false));
  return hip_status(fn, gdn::launch_linear(M, Nc, K, A, W, w_layout, R, C, C_bf16,
                                           static_cast<hipStream_t>(stream)));
}

int gdn_pack_weights(int Nc, int K, const void* W, void* W_packed, void* stream) {
  const char* fn = "gdn_pack_weights";
  GDN_TRY(linear_sizes_ok(fn, 1, Nc, K));
  if (Nc == 0) return ok();
  GDN_TRY(check_ptr(fn, "W", W, true));
  GDN_TRY(check_ptr(fn, "W_packed", W_packed, true));
  const char* w0 = static_cast<const char*>(W);
  const char* p0 = static_cast<const char*>(W_packed);
  const size_t n = (size_t)Nc * K * 2;
  if (w0 < p0 + n && p0 < w0 + n) return fail(GDN_ERR_ARG, "%s: W and W_packed overlap", fn);
  return hip_status(fn, gdn::launch_pack_weights(Nc, K, W, W_packed,
                                                 static_cast<hipStream_t>(stream)));
}

int gdn_layer_prep(int B, int N, int H, int dk, int dv, int D, const float* P, const void* x,
                   const void* W_ab, const int32_t* parents, const float* conv_w,
                   const float* hist, float gate_shift, void* q, void* k, void* v, float* beta,
                   float* g, void* stream) {
  const char* fn = "gdn_layer_prep";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  if (D < 8 || D > 65536 || D % 8 != 0)
    return fail(GDN_ERR_SHAPE, "%s: unsupported hidden width D=%d (need 8<=D<=65536, D%%8==0)",
                fn, D);
  if (!std::isfinite(gate_shift)) return fail(GDN_ERR_ARG, "%s: gate_shift is not finite", fn);
  if (B == 0 || N == 0) return ok();
  GDN_TRY(check_ptr(fn, "P", P, true));
  GDN_TRY(check_ptr(fn, "x", x, true));
  GDN_TRY(check_ptr(fn, "W_ab", W_ab, true));
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr(fn, "conv_w", conv_w, true));
  GDN_TRY(check_ptr(fn, "hist", hist, true));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  return hip_status(fn, gdn::launch_layer_prep(B, N, H, dk, dv, D, P, x, W_ab, parents, conv_w,
                                               hist, gate_shift, q, k, v, beta, g, nullptr, 0,
                                               nullptr, nullptr, nullptr, nullptr,
                                               static_cast<hipStream_t>(stream)));
}

int gdn_layer_prep_delayed(int B, int N_prev, int N, int H, int dk, int dv, int D,
                           const float* P, const void* x, const void* W_ab,
                           const int32_t* parents, const float* conv_w, const float* hist,
                           float gate_shift, void* q, void* k, void* v, float* beta, float* g,
                           const float* P_prev, const int32_t* parents_prev,
                           const int32_t* last_prev, float* hist_out, int32_t* dev_status,
                           void* stream) {
  const char* fn = "gdn_layer_prep_delayed";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  if (N_prev < 1 || N_prev > gdn::kMaxNodes)
    return fail(GDN_ERR_SHAPE, "%s: N_prev=%d outside 1..64", fn, N_prev);
  if (D < 8 || D > 65536 || D % 8 != 0)
    return fail(GDN_ERR_SHAPE, "%s: unsupported hidden width D=%d (need 8<=D<=65536, D%%8==0)",
                fn, D);
  if (!std::isfinite(gate_shift)) return fail(GDN_ERR_ARG, "%s: gate_shift is not finite", fn);
  if (B == 0) return ok();
  if (N == 0) return fail(GDN_ERR_SHAPE, "%s: N=0; use gdn_conv_commit alone", fn);
  GDN_TRY(check_ptr(fn, "P", P, true));
  GDN_TRY(check_ptr(fn, "x", x, true));
  GDN_TRY(check_ptr(fn, "W_ab", W_ab, true));
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr(fn, "conv_w", conv_w, true));
  GDN_TRY(check_ptr(fn, "hist", hist, true));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  GDN_TRY(check_ptr(fn, "P_prev", P_prev, true));
  GDN_TRY(check_ptr4(fn, "parents_prev", parents_prev, true));
  GDN_TRY(check_ptr4(fn, "last_prev", last_prev, true));
  GDN_TRY(check_ptr(fn, "hist_out", hist_out, true));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  const size_t hb = (size_t)B * 3 * H * (2 * dk + dv) * sizeof(float);
  const char* h0 = reinterpret_cast<const char*>(hist);
  const char* h1 = reinterpret_cast<const char*>(hist_out);
  if (h0 < h1 + hb && h1 < h0 + hb)
    return fail(GDN_ERR_ARG, "%s: hist and hist_out overlap", fn);
  return hip_status(fn, gdn::launch_layer_prep(B, N, H, dk, dv, D, P, x, W_ab, parents, conv_w,
                                               hist, gate_shift, q, k, v, beta, g, P_prev,
                                               N_prev, parents_prev, last_prev, hist_out,
                                               dev_status, static_cast<hipStream_t>(stream)));
}

int gdn_gate_merge(int M, int Cw, const float* o, const float* gate, int ldg, void* Y,
                   void* stream) {
  const char* fn = "gdn_gate_merge";
  if (M < 0 || Cw < 0 || Cw % 4 != 0 || ldg < Cw || ldg % 4 != 0 ||
      (long long)M * ldg >= (1ll << 40))
    return fail(GDN_ERR_SHAPE, "%s: unsupported sizes M=%d Cw=%d ldg=%d (need Cw%%4==0, "
                "ldg>=Cw, ldg%%4==0)", fn, M, Cw, ldg);
  if (M == 0 || Cw == 0) return ok();
  GDN_TRY(check_ptr(fn, "o", o, true));
  GDN_TRY(check_ptr(fn, "gate", gate, true));
  GDN_TRY(check_ptr(fn, "Y", Y, true));
  return hip_status(fn, gdn::launch_gate_merge(M, Cw, o, gate, ldg, Y,
                                               static_cast<hipStream_t>(stream)));
}

int gdn_layer_verify(int B, int N_prev, int N, int H, int dk, int dv, float* S,
                     const void* prev_factors, const int32_t* last_accepted,
                     int32_t* commit_status, const int32_t* parents, const void* q,
                     const void* k, const void* v, const float* beta, const float* g,
                     float scale, const float* gate, int ldg, void* Y, void* factors,
                     int32_t* dev_status, void* stream) {
  const char* fn = "gdn_layer_verify";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  const bool dly = prev_factors != nullptr;
  if (dly && (N_prev < 1 || N_prev > gdn::kMaxNodes))
    return fail(GDN_ERR_SHAPE, "%s: N_prev=%d outside 1..64", fn, N_prev);
  if (!std::isfinite(scale)) return fail(GDN_ERR_ARG, "%s: scale is not finite", fn);
  if (ldg < H * dv) return fail(GDN_ERR_SHAPE, "%s: ldg=%d below H*dv=%d", fn, ldg, H * dv);
  if (B == 0 || N == 0) return ok();
  GDN_TRY(check_ptr(fn, "S", S, true));
  if (dly) GDN_TRY(check_ptr4(fn, "last_accepted", last_accepted, true));
  GDN_TRY(check_ptr4(fn, "commit_status", commit_status, false));
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  GDN_TRY(check_ptr4(fn, "gate", gate, true));
  GDN_TRY(check_ptr(fn, "Y", Y, true));
  GDN_TRY(check_ptr(fn, "factors", factors, true));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  if (dly) {
    const char* a0 = static_cast<const char*>(prev_factors);
    const char* b0 = static_cast<const char*>(factors);
    const size_t na = gdn::record_layout(B, N_prev, H, dk, dv, GDN_BF16).total;
    const size_t nb = gdn::record_layout(B, N, H, dk, dv, GDN_BF16).total;
    if (a0 < b0 + nb && b0 < a0 + na)
      return fail(GDN_ERR_ARG, "%s: factors and prev_factors overlap", fn);
  }
  return hip_status(fn, gdn::launch_tree_verify(B, N, H, dk, dv, GDN_BF16, S, parents, q, k, v,
                                                beta, g, scale, nullptr, factors, nullptr,
                                                nullptr, dev_status, prev_factors,
                                                dly ? N_prev : 0, last_accepted, commit_status,
                                                gate, ldg, Y, static_cast<hipStream_t>(stream)));
}

int gdn_conv_commit(int B, int N, int Cc, const float* P, int ldP, const int32_t* parents,
                    const int32_t* last_accepted, float* hist, int32_t* dev_status,
                    void* stream) {
  const char* fn = "gdn_conv_commit";
  if (B < 0 || N < 0 || N > gdn::kMaxNodes || Cc < 4 || Cc % 4 != 0 || ldP < Cc ||
      ldP % 4 != 0 || B > 65535)
    return fail(GDN_ERR_SHAPE, "%s: unsupported sizes B=%d N=%d Cc=%d ldP=%d (need "
                "0<=B<=65535, 0<=N<=64, Cc%%4==0, ldP>=Cc, ldP%%4==0)", fn, B, N, Cc, ldP);
  if (B == 0) return ok();
  GDN_TRY(check_ptr4(fn, "last_accepted", last_accepted, true));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  if (N == 0) return ok();  // only last_accepted = -1 is possible: nothing to apply
  GDN_TRY(check_ptr(fn, "P", P, true));
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr(fn, "hist", hist, true));
  return hip_status(fn, gdn::launch_conv_commit(B, N, Cc, P, ldP, parents, last_accepted, hist,
                                                dev_status, static_cast<hipStream_t>(stream)));
}

int gdn_decode_step(int B, int H, int dk, int dv, int qkv_dtype, float* S, const void* q,
                    const void* k, const void* v, const float* beta, const float* g,
                    float scale, float* out, void* stream) {
  const char* fn = "gdn_decode_step";
  GDN_TRY(check_sizes(fn, B, 1, H, dk, dv));
  GDN_TRY(check_dtype(fn, qkv_dtype));
  if (!std::isfinite(scale)) return fail(GDN_ERR_ARG, "%s: scale is not finite", fn);
  if (B == 0) return ok();
  GDN_TRY(check_ptr(fn, "S", S, true));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  GDN_TRY(check_ptr4(fn, "out", out, true));
  return hip_status(fn, gdn::launch_decode_step(B, H, dk, dv, qkv_dtype, S, q, k, v, beta, g,
                                                scale, out, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// replay baselines (gdnnext.h)
// ---------------------------------------------------------------------------

int gdn_replay_verify(int B, int N, int H, int dk, int dv, int qkv_dtype, const float* S0,
                      const int32_t* parents, const void* q, const void* k, const void* v,
                      const float* beta, const float* g, float scale, const int32_t* ends,
                      int P, float* out, int32_t* dev_status, void* stream) {
  const char* fn = "gdn_replay_verify";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  GDN_TRY(check_dtype(fn, qkv_dtype));
  if (P < 1 || P > gdn::kMaxNodes)
    return fail(GDN_ERR_SHAPE, "%s: P=%d path slots outside 1..64", fn, P);
  if (!std::isfinite(scale)) return fail(GDN_ERR_ARG, "%s: scale is not finite", fn);
  if (B == 0 || N == 0) return ok();
  GDN_TRY(check_ptr(fn, "S0", S0, true));
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  GDN_TRY(check_ptr4(fn, "ends", ends, true));
  GDN_TRY(check_ptr4(fn, "out", out, true));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  return hip_status(fn, gdn::launch_replay(true, B, N, H, dk, dv, qkv_dtype,
                                           const_cast<float*>(S0), parents, q, k, v, beta, g,
                                           scale, ends, P, out, dev_status,
                                           static_cast<hipStream_t>(stream)));
}

int gdn_replay_commit(int B, int N, int H, int dk, int dv, int qkv_dtype, float* S,
                      const int32_t* parents, const void* k, const void* v, const float* beta,
                      const float* g, const int32_t* last_accepted, int32_t* dev_status,
                      void* stream) {
  const char* fn = "gdn_replay_commit";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  GDN_TRY(check_dtype(fn, qkv_dtype));
  if (B == 0) return ok();
  GDN_TRY(check_ptr4(fn, "last_accepted", last_accepted, true));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  if (N == 0) return ok();  // only last_accepted = -1 is possible: nothing to apply
  GDN_TRY(check_ptr(fn, "S", S, true));
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  return hip_status(fn, gdn::launch_replay(false, B, N, H, dk, dv, qkv_dtype, S, parents, nullptr,
                                           k, v, beta, g, 1.0f, last_accepted, 1, nullptr,
                                           dev_status, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// chain-decomposed hybrid verifier (gdnnext.h)
// ---------------------------------------------------------------------------

size_t gdn_hybrid_plan_entries(int B, int N) {
  if (B < 1 || N < 1 || N > gdn::kMaxNodes) return 0;
  return 2 * (size_t)N * B * N;
}

int gdn_hybrid_plan(int B, int N, const int32_t* parents, int32_t* plan,
                    int32_t* chains_per_level, int32_t* levels) {
  const char* fn = "gdn_hybrid_plan";
  if (B < 1 || N < 1 || N > gdn::kMaxNodes || (long long)B * N * N >= (1ll << 31))
    return fail(GDN_ERR_SHAPE, "%s: unsupported sizes B=%d N=%d (need B>=1, 1<=N<=64)", fn, B,
                N);
  if (!parents || !plan || !chains_per_level || !levels)
    return fail(GDN_ERR_ARG, "%s: NULL argument", fn);
  const int L = gdn::hybrid_plan(B, N, parents, plan, chains_per_level);
  if (L < 0)
    return fail(GDN_ERR_TOPOLOGY, "%s: parents fail the topology check (-1 <= p[t] < t)", fn);
  *levels = L;
  return ok();
}

int gdn_hybrid_verify(int B, int N, int H, int dk, int dv, int qkv_dtype, const float* S0,
                      const int32_t* parents, const void* q, const void* k, const void* v,
                      const float* beta, const float* g, float scale, float* out,
                      void* factors, const int32_t* plan, int levels,
                      const int32_t* chains_per_level, int32_t* dev_status, void* stream) {
  const char* fn = "gdn_hybrid_verify";
  GDN_TRY(check_sizes(fn, B, N, H, dk, dv));
  GDN_TRY(check_dtype(fn, qkv_dtype));
  if (!std::isfinite(scale)) return fail(GDN_ERR_ARG, "%s: scale is not finite", fn);
  if (B == 0 || N == 0) return ok();
  if (levels < 1 || levels > N)
    return fail(GDN_ERR_SHAPE, "%s: levels=%d outside 1..N=%d", fn, levels, N);
  if (!chains_per_level) return fail(GDN_ERR_ARG, "%s: chains_per_level is NULL", fn);
  for (int l = 0; l < levels; ++l)
    if (chains_per_level[l] < 1 || chains_per_level[l] > N)
      return fail(GDN_ERR_SHAPE, "%s: level %d has %d chains (need 1..N)", fn, l,
                  chains_per_level[l]);
  GDN_TRY(check_ptr(fn, "S0", S0, true));
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr(fn, "q", q, true));
  GDN_TRY(check_ptr(fn, "k", k, true));
  GDN_TRY(check_ptr(fn, "v", v, true));
  GDN_TRY(check_ptr4(fn, "beta", beta, true));
  GDN_TRY(check_ptr4(fn, "g", g, true));
  GDN_TRY(check_ptr4(fn, "out", out, true));
  GDN_TRY(check_ptr(fn, "factors", factors, true));
  GDN_TRY(check_ptr4(fn, "plan", plan, true));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  return hip_status(fn, gdn::launch_hybrid(B, N, H, dk, dv, qkv_dtype, S0, parents, q, k, v, beta,
                                           g, scale, out, factors, plan, levels,
                                           chains_per_level, dev_status,
                                           static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------------------
// confidence-guided pruning (gdnnext.h)
// ---------------------------------------------------------------------------

int gdn_prune_draft(int B, int M, int T, float tau, const int32_t* parents, const float* conf,
                    int32_t* kept, int32_t* new_parents, int32_t* count, int32_t* dev_status,
                    void* stream) {
  const char* fn = "gdn_prune_draft";
  if (B < 0 || B > 65535 || M < 1 || M > 1024 || T < 1 || T > gdn::kMaxNodes)
    return fail(GDN_ERR_SHAPE, "%s: unsupported sizes B=%d M=%d T=%d (need 0<=B<=65535, "
                "1<=M<=1024, 1<=T<=64)", fn, B, M, T);
  if (!std::isfinite(tau) || tau < 0.f)
    return fail(GDN_ERR_ARG, "%s: tau must be finite and >= 0", fn);
  if (B == 0) return ok();
  GDN_TRY(check_ptr4(fn, "parents", parents, true));
  GDN_TRY(check_ptr4(fn, "conf", conf, true));
  GDN_TRY(check_ptr4(fn, "kept", kept, true));
  GDN_TRY(check_ptr4(fn, "new_parents", new_parents, true));
  GDN_TRY(check_ptr4(fn, "count", count, true));
  GDN_TRY(check_ptr4(fn, "dev_status", dev_status, false));
  return hip_status(fn, gdn::launch_prune(B, M, T, tau, parents, conf, kept, new_parents, count,
                                          dev_status, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
