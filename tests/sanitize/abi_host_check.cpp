// Host-side checks of libgdnspec's argument validation and host planning,
// meant to run under AddressSanitizer and UndefinedBehaviorSanitizer on a
// machine without a GPU.  The library sources are compiled for the host only
// (no device code), so any call that got past validation would reach the HIP
// runtime and come back as GDN_ERR_HIP: every rejected call here must return
// its own status instead, i.e. fail before any launch.
//
// Device pointers are fake addresses that are never mapped: a host-side read
// of one crashes the program.  Host arrays (the hybrid plan's) are allocated
// at their exact sizes, so a read or write past them is reported by ASan.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/gdnlayer.h"
#include "../../include/gdnnext.h"
#include "../../include/gdnspec.h"

namespace {

int g_fail = 0;
int g_checks = 0;

void check(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, gdn_last_error());
    ++g_fail;
  }
}
#define CHECK(x) check((x), #x, __LINE__)
#define EXPECT_RC(call, code) check((call) == (code), #call " == " #code, __LINE__)

// never dereferenced on the host
void* dev(uintptr_t a) { return reinterpret_cast<void*>(a); }
float* devf(uintptr_t a) { return reinterpret_cast<float*>(a); }
int32_t* devi(uintptr_t a) { return reinterpret_cast<int32_t*>(a); }
uint64_t* devu(uintptr_t a) { return reinterpret_cast<uint64_t*>(a); }

const uintptr_t P = 1ull << 40;  // 16-byte aligned fake device address
const uintptr_t ODD = P + 8;     // 4- and 8-byte aligned, not 16
const uintptr_t ODD4 = P + 2;    // not 4-byte aligned

void verify_core_entry_points() {
  const int B = 1, N = 8, H = 8, dk = 256, dv = 256;
  // sizes
  const int bad[][5] = {{1, 65, 8, 256, 256}, {1, 8, 8, 12, 256}, {1, 8, 8, 256, 6},
                        {1, 8, 0, 256, 256},  {-1, 8, 8, 256, 256}, {1, 8, 8, 264, 256},
                        {1, 8, 8, 256, 260},  {1, -1, 8, 256, 256}};
  for (auto& s : bad) {
    CHECK(gdn_factor_bytes(s[0], s[1], s[2], s[3], s[4], GDN_BF16) == 0);
    EXPECT_RC(gdn_tree_verify(s[0], s[1], s[2], s[3], s[4], GDN_BF16, devf(P), devi(P), dev(P),
                              dev(P), dev(P), devf(P), devf(P), 1.f, devf(P), dev(P), nullptr,
                              nullptr, nullptr, nullptr),
              GDN_ERR_SHAPE);
    CHECK(std::strstr(gdn_last_error(), "unsupported sizes") != nullptr);
    EXPECT_RC(gdn_chain_verify(s[0], s[1], s[2], s[3], s[4], GDN_BF16, devf(P), dev(P), dev(P),
                               dev(P), devf(P), devf(P), 1.f, devf(P), dev(P), nullptr),
              GDN_ERR_SHAPE);
    EXPECT_RC(gdn_commit_path(s[0], s[1], s[2], s[3], s[4], GDN_BF16, devf(P), dev(P), devi(P),
                              nullptr, nullptr, nullptr, nullptr),
              GDN_ERR_SHAPE);
    EXPECT_RC(gdn_replay_verify(s[0], s[1], s[2], s[3], s[4], GDN_BF16, devf(P), devi(P), dev(P),
                                dev(P), dev(P), devf(P), devf(P), 1.f, devi(P), 1, devf(P),
                                nullptr, nullptr),
              GDN_ERR_SHAPE);
    EXPECT_RC(gdn_replay_commit(s[0], s[1], s[2], s[3], s[4], GDN_BF16, devf(P), devi(P), dev(P),
                                dev(P), devf(P), devf(P), devi(P), nullptr, nullptr),
              GDN_ERR_SHAPE);
  }
  // dtype, scale, pointers
  EXPECT_RC(gdn_tree_verify(B, N, H, dk, dv, 7, devf(P), devi(P), dev(P), dev(P), dev(P),
                            devf(P), devf(P), 1.f, devf(P), dev(P), nullptr, nullptr, nullptr,
                            nullptr),
            GDN_ERR_ARG);
  CHECK(std::strstr(gdn_last_error(), "qkv_dtype") != nullptr);
  EXPECT_RC(gdn_tree_verify(B, N, H, dk, dv, GDN_BF16, nullptr, devi(P), dev(P), dev(P), dev(P),
                            devf(P), devf(P), 1.f, devf(P), dev(P), nullptr, nullptr, nullptr,
                            nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_tree_verify(B, N, H, dk, dv, GDN_BF16, devf(ODD), devi(P), dev(P), dev(P),
                            dev(P), devf(P), devf(P), 1.f, devf(P), dev(P), nullptr, nullptr,
                            nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_tree_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(ODD4), dev(P), dev(P),
                            dev(P), devf(P), devf(P), 1.f, devf(P), dev(P), nullptr, nullptr,
                            nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_tree_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P), dev(P),
                            devf(P), devf(P), NAN, devf(P), dev(P), nullptr, nullptr, nullptr,
                            nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_chain_verify(B, N, H, dk, dv, GDN_BF16, devf(P), dev(P), nullptr, dev(P),
                             devf(P), devf(P), 1.f, devf(P), dev(P), nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_chain_verify(B, N, H, dk, dv, GDN_BF16, devf(P), dev(P), dev(P), dev(P),
                             devf(P), devf(P), INFINITY, devf(P), dev(P), nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_commit_path(B, N, H, dk, dv, GDN_BF16, devf(P), nullptr, devi(P), nullptr,
                            nullptr, nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_commit_path(B, N, H, dk, dv, GDN_BF16, devf(P), dev(P), devi(ODD4), nullptr,
                            nullptr, nullptr, nullptr),
            GDN_ERR_ARG);
  // delayed forms: N_prev range, overlapping records
  EXPECT_RC(gdn_tree_verify_delayed(B, 0, N, H, dk, dv, GDN_BF16, devf(P), dev(P), devi(P),
                                    nullptr, devi(P), dev(P), dev(P), dev(P), devf(P), devf(P),
                                    1.f, devf(P), dev(P), nullptr, nullptr, nullptr, nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_tree_verify_delayed(B, 8, N, H, dk, dv, GDN_BF16, devf(P), dev(P), devi(P),
                                    nullptr, devi(P), dev(P), dev(P), dev(P), devf(P), devf(P),
                                    1.f, devf(P), dev(P), nullptr, nullptr, nullptr, nullptr),
            GDN_ERR_ARG);  // factors == prev_factors
  EXPECT_RC(gdn_chain_verify_delayed(B, 65, N, H, dk, dv, GDN_BF16, devf(P), dev(P), devi(P),
                                     nullptr, dev(P), dev(P), dev(P), devf(P), devf(P), 1.f,
                                     devf(P), dev(1ull << 41), nullptr),
            GDN_ERR_SHAPE);
  // FP32 drafts whose LDS staging does not fit are refused before any launch
  EXPECT_RC(gdn_chain_verify_delayed(B, 64, 64, H, dk, dv, GDN_F32, devf(P), dev(P), devi(P),
                                     nullptr, dev(P), dev(P), dev(P), devf(P), devf(P), 1.f,
                                     devf(P), dev(1ull << 41), nullptr),
            GDN_ERR_UNSUPPORTED);
  // empty batches are valid and launch nothing
  EXPECT_RC(gdn_tree_verify(0, N, H, dk, dv, GDN_BF16, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, nullptr, 1.f, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr),
            GDN_OK);
  EXPECT_RC(gdn_commit_path(0, N, H, dk, dv, GDN_BF16, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, nullptr),
            GDN_OK);
  // the record layout: five 256-byte aligned sections in order, then the total
  for (int code : {GDN_BF16, GDN_F32}) {
    const size_t es = code == GDN_BF16 ? 2 : 4;
    for (int n : {1, 7, 8, 33, 64}) {
      const int b = 3, h = 2, k = 24, v = 40;
      size_t off[5];
      EXPECT_RC(gdn_factor_layout(b, n, h, k, v, code, off), GDN_OK);
      const size_t sz[5] = {(size_t)b * h * n * v * 4, (size_t)b * h * n * 4,
                            (size_t)b * h * n * k * es, (size_t)b * n * 4, (size_t)b * n * 8};
      CHECK(off[0] == 0);
      for (int i = 0; i < 5; ++i) {
        const size_t next = i < 4 ? off[i + 1] : gdn_factor_bytes(b, n, h, k, v, code);
        CHECK(off[i] % 256 == 0);
        CHECK(off[i] + sz[i] <= next && next < off[i] + sz[i] + 256);
      }
    }
  }
  CHECK(gdn_workspace_bytes(8, 64, 8, 256, 256) == 0);
}

void verify_layer_entry_points() {
  EXPECT_RC(gdn_linear(65, 16, 256, dev(P), dev(P), GDN_W_ROWS, nullptr, devf(P), nullptr,
                       nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_linear(32, 16, 300, dev(P), dev(P), GDN_W_ROWS, nullptr, devf(P), nullptr,
                       nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_linear(32, 16, 256, dev(P), dev(P), 5, nullptr, devf(P), nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_linear(32, 16, 256, dev(P), dev(P), GDN_W_ROWS, nullptr, nullptr, nullptr,
                       nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_linear(32, 16, 256, nullptr, dev(P), GDN_W_ROWS, nullptr, devf(P), nullptr,
                       nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_linear(0, 16, 256, nullptr, nullptr, GDN_W_ROWS, nullptr, devf(P), nullptr,
                       nullptr),
            GDN_OK);
  EXPECT_RC(gdn_pack_weights(16, 256, dev(P), dev(P + 4096), nullptr), GDN_ERR_ARG);  // overlap
  EXPECT_RC(gdn_pack_weights(15, 256, dev(P), dev(P << 1), nullptr), GDN_ERR_SHAPE);
  const int B = 1, N = 32, H = 8, dk = 256, dv = 256, D = 2048;
  EXPECT_RC(gdn_layer_prep(B, N, H, dk, dv, 12, devf(P), dev(P), dev(P), devi(P), devf(P),
                           devf(P), 0.f, dev(P), dev(P), dev(P), devf(P), devf(P), nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_layer_prep(B, N, H, dk, dv, D, devf(P), dev(P), dev(P), devi(P), devf(P),
                           devf(P), NAN, dev(P), dev(P), dev(P), devf(P), devf(P), nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_layer_prep(B, N, H, dk, dv, D, devf(P), dev(P), nullptr, devi(P), devf(P),
                           devf(P), 0.f, dev(P), dev(P), dev(P), devf(P), devf(P), nullptr),
            GDN_ERR_ARG);
  // the delayed prep: history buffers may not overlap, N_prev in range, N > 0
  const uintptr_t H0 = P, H1 = P + 64;
  EXPECT_RC(gdn_layer_prep_delayed(B, 32, N, H, dk, dv, D, devf(P), dev(P), dev(P), devi(P),
                                   devf(P), devf(H0), 0.f, dev(P), dev(P), dev(P), devf(P),
                                   devf(P), devf(P), devi(P), devi(P), devf(H1), nullptr,
                                   nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_layer_prep_delayed(B, 0, N, H, dk, dv, D, devf(P), dev(P), dev(P), devi(P),
                                   devf(P), devf(P), 0.f, dev(P), dev(P), dev(P), devf(P),
                                   devf(P), devf(P), devi(P), devi(P), devf(P << 1), nullptr,
                                   nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_layer_prep_delayed(B, 32, 0, H, dk, dv, D, devf(P), dev(P), dev(P), devi(P),
                                   devf(P), devf(P), 0.f, dev(P), dev(P), dev(P), devf(P),
                                   devf(P), devf(P), devi(P), devi(P), devf(P << 1), nullptr,
                                   nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_gate_merge(4, 6, devf(P), devf(P), 8, dev(P), nullptr), GDN_ERR_SHAPE);
  EXPECT_RC(gdn_gate_merge(4, 8, devf(P), devf(P), 4, dev(P), nullptr), GDN_ERR_SHAPE);
  EXPECT_RC(gdn_gate_merge(4, 8, devf(P), nullptr, 8, dev(P), nullptr), GDN_ERR_ARG);
  EXPECT_RC(gdn_layer_verify(B, 32, N, H, dk, dv, devf(P), dev(P), devi(P), nullptr, devi(P),
                             dev(P), dev(P), dev(P), devf(P), devf(P), 1.f, devf(P), H * dv - 4,
                             dev(P), dev(P << 1), nullptr, nullptr),
            GDN_ERR_SHAPE);  // ldg below H*dv
  EXPECT_RC(gdn_layer_verify(B, 32, N, H, dk, dv, devf(P), dev(P), devi(P), nullptr, devi(P),
                             dev(P), dev(P), dev(P), devf(P), devf(P), 1.f, devf(P), H * dv,
                             dev(P), dev(P), nullptr, nullptr),
            GDN_ERR_ARG);  // factors == prev_factors
  EXPECT_RC(gdn_conv_commit(B, 65, 16, devf(P), 16, devi(P), devi(P), devf(P), nullptr, nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_conv_commit(B, N, 16, devf(P), 12, devi(P), devi(P), devf(P), nullptr, nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_conv_commit(B, N, 16, devf(P), 16, devi(P), nullptr, devf(P), nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_decode_step(B, H, dk, dv, 3, devf(P), dev(P), dev(P), dev(P), devf(P), devf(P),
                            1.f, devf(P), nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_decode_step(B, H, dk, dv, GDN_BF16, devf(P), dev(P), dev(P), dev(P), devf(P),
                            devf(P), 1.f, nullptr, nullptr),
            GDN_ERR_ARG);
}

void verify_next_entry_points() {
  const int B = 2, N = 16, H = 8, dk = 256, dv = 256;
  EXPECT_RC(gdn_replay_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P),
                              dev(P), devf(P), devf(P), 1.f, devi(P), 0, devf(P), nullptr,
                              nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_replay_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P),
                              dev(P), devf(P), devf(P), 1.f, devi(P), 65, devf(P), nullptr,
                              nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_replay_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P),
                              dev(P), devf(P), devf(P), 1.f, nullptr, 4, devf(P), nullptr,
                              nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_replay_commit(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P),
                              devf(P), devf(P), nullptr, nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_replay_commit(B, N, H, dk, dv, 2, devf(P), devi(P), dev(P), dev(P), devf(P),
                              devf(P), devi(P), nullptr, nullptr),
            GDN_ERR_ARG);
  // hybrid verify: the host arrays of the plan are read only up to `levels`
  std::vector<int32_t> cpl = {1, 3, 2};
  EXPECT_RC(gdn_hybrid_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P),
                              dev(P), devf(P), devf(P), 1.f, devf(P), dev(P), devi(P), 0,
                              cpl.data(), nullptr, nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_hybrid_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P),
                              dev(P), devf(P), devf(P), 1.f, devf(P), dev(P), devi(P), N + 1,
                              cpl.data(), nullptr, nullptr),
            GDN_ERR_SHAPE);
  cpl[1] = 0;
  EXPECT_RC(gdn_hybrid_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P),
                              dev(P), devf(P), devf(P), 1.f, devf(P), dev(P), devi(P), 3,
                              cpl.data(), nullptr, nullptr),
            GDN_ERR_SHAPE);
  cpl[1] = 3;
  EXPECT_RC(gdn_hybrid_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P),
                              dev(P), devf(P), devf(P), 1.f, devf(P), dev(P), devi(P), 3,
                              nullptr, nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_hybrid_verify(B, N, H, dk, dv, GDN_BF16, devf(P), devi(P), dev(P), dev(P),
                              dev(P), devf(P), devf(P), 1.f, devf(P), dev(P), nullptr, 3,
                              cpl.data(), nullptr, nullptr),
            GDN_ERR_ARG);
  // pruning
  EXPECT_RC(gdn_prune_draft(B, 1025, 16, 3.f, devi(P), devf(P), devi(P), devi(P), devi(P),
                            nullptr, nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_prune_draft(B, 341, 65, 3.f, devi(P), devf(P), devi(P), devi(P), devi(P),
                            nullptr, nullptr),
            GDN_ERR_SHAPE);
  EXPECT_RC(gdn_prune_draft(B, 341, 16, -1.f, devi(P), devf(P), devi(P), devi(P), devi(P),
                            nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_prune_draft(B, 341, 16, NAN, devi(P), devf(P), devi(P), devi(P), devi(P),
                            nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_prune_draft(B, 341, 16, 3.f, devi(P), devf(P), nullptr, devi(P), devi(P),
                            nullptr, nullptr),
            GDN_ERR_ARG);
  EXPECT_RC(gdn_prune_draft(0, 341, 16, 3.f, nullptr, nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr),
            GDN_OK);
}

// ---- the hybrid plan on the host, checked against its definition
std::vector<int32_t> random_tree(std::mt19937& rng, int N, int kind) {
  std::vector<int32_t> p(N, -1);
  for (int t = 1; t < N; ++t) {
    switch (kind) {
      case 0: p[t] = t - 1; break;                                            // chain
      case 1: p[t] = 0; break;                                                // star
      case 2: p[t] = (t - 1) / 2; break;                                      // binary
      case 3: p[t] = (int)(rng() % (unsigned)t); break;                       // uniform recursive
      case 4: p[t] = (rng() % 4 == 0) ? -1 : (int)(rng() % (unsigned)t); break;  // forest
      default: p[t] = (rng() % 4) ? t - 1 : std::max(0, t - 2 - (int)(rng() % 6)); break;
    }
  }
  return p;
}

void check_plan(int B, int N, const std::vector<int32_t>& par) {
  const size_t entries = gdn_hybrid_plan_entries(B, N);
  CHECK(entries == 2ull * N * B * N);
  // exact-size heap blocks, so ASan sees any access past them
  int32_t* plan = static_cast<int32_t*>(std::malloc(entries * sizeof(int32_t)));
  int32_t* cpl = static_cast<int32_t*>(std::malloc(N * sizeof(int32_t)));
  int32_t* pp = static_cast<int32_t*>(std::malloc(par.size() * sizeof(int32_t)));
  std::memcpy(pp, par.data(), par.size() * sizeof(int32_t));
  int32_t levels = -7;
  EXPECT_RC(gdn_hybrid_plan(B, N, pp, plan, cpl, &levels), GDN_OK);
  CHECK(levels >= 1 && levels <= N);
  for (int b = 0; b < B; ++b) {
    const int32_t* p = pp + (size_t)b * N;
    // lowest-numbered child of every node
    std::vector<int> first(N, -1);
    for (int t = N - 1; t >= 0; --t)
      if (p[t] >= 0) first[p[t]] = t;
    std::vector<int> seen(N, 0), chain_level(N, -1);
    for (int l = 0; l < levels; ++l) {
      int count = 0;
      for (int c = 0; c < N; ++c) {
        const int32_t* e = plan + (((size_t)l * B + b) * N + c) * 2;
        if (e[0] < 0) {
          CHECK(e[0] == -1 && e[1] == -1);
          continue;
        }
        CHECK(c == count);  // chains packed at the front
        ++count;
        const int head = e[0], last = e[1];
        CHECK(head >= 0 && head < N && last >= head && last < N);
        if (!(head >= 0 && head < N && last >= head && last < N)) continue;
        // a chain is a head that is no first child, then first children down to last
        CHECK(p[head] < 0 || first[p[head]] != head);
        CHECK(p[head] < 0 ? l == 0 : (chain_level[p[head]] == l - 1));
        int u = head, guard = 0;
        while (true) {
          CHECK(seen[u] == 0);
          seen[u] = 1;
          chain_level[u] = l;
          if (u == last || ++guard > N) break;
          u = first[u];
          if (u < 0) break;
        }
        CHECK(u == last);
        CHECK(first[last] < 0);  // a chain runs until the node has no child
      }
      CHECK(count <= cpl[l]);
    }
    for (int t = 0; t < N; ++t) CHECK(seen[t] == 1);
  }
  for (int l = 0; l < levels; ++l) {
    int most = 0;
    for (int b = 0; b < B; ++b) {
      int count = 0;
      for (int c = 0; c < N; ++c) count += plan[(((size_t)l * B + b) * N + c) * 2] >= 0;
      most = std::max(most, count);
    }
    CHECK(cpl[l] == most && most >= 1);
  }
  for (int l = levels; l < N; ++l) CHECK(cpl[l] == 0);
  std::free(plan);
  std::free(cpl);
  std::free(pp);
}

void verify_hybrid_plan() {
  std::mt19937 rng(1234);
  for (int kind = 0; kind < 6; ++kind)
    for (int N : {1, 2, 3, 8, 17, 32, 63, 64})
      for (int B : {1, 3}) {
        std::vector<int32_t> par;
        for (int b = 0; b < B; ++b) {
          auto t = random_tree(rng, N, kind);
          par.insert(par.end(), t.begin(), t.end());
        }
        check_plan(B, N, par);
      }
  // rejected topologies and sizes
  std::vector<int32_t> plan(gdn_hybrid_plan_entries(1, 4)), cpl(4);
  int32_t levels = 0;
  const int32_t bad1[4] = {-1, 0, 2, 1};   // p[2] = 2
  const int32_t bad2[4] = {-1, 0, -2, 1};  // p[2] = -2
  const int32_t bad3[4] = {0, 0, 1, 2};    // p[0] = 0
  for (const int32_t* bad : {bad1, bad2, bad3})
    EXPECT_RC(gdn_hybrid_plan(1, 4, bad, plan.data(), cpl.data(), &levels), GDN_ERR_TOPOLOGY);
  const int32_t good[4] = {-1, 0, 1, 2};
  EXPECT_RC(gdn_hybrid_plan(1, 65, good, plan.data(), cpl.data(), &levels), GDN_ERR_SHAPE);
  EXPECT_RC(gdn_hybrid_plan(0, 4, good, plan.data(), cpl.data(), &levels), GDN_ERR_SHAPE);
  EXPECT_RC(gdn_hybrid_plan(1, 4, good, nullptr, cpl.data(), &levels), GDN_ERR_ARG);
  CHECK(gdn_hybrid_plan_entries(1, 65) == 0 && gdn_hybrid_plan_entries(0, 4) == 0);
}

}  // namespace

int main() {
  CHECK(gdn_version() >= 1);
  verify_core_entry_points();
  verify_layer_entry_points();
  verify_next_entry_points();
  verify_hybrid_plan();
  std::printf("%d checks, %d failed\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
