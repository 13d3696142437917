/* Checks of the C oracle (oracle/gdn_oracle.c) meant to run under
 * AddressSanitizer and UndefinedBehaviorSanitizer: small random drafts with
 * every buffer allocated at its exact size, on one thread and on several.
 * Besides memory safety it checks properties that hold exactly in the
 * oracle's own arithmetic:
 *   - a chain draft verified per path equals token-by-token decode, bitwise;
 *   - the commit of a chain's last node equals the decode's final state;
 *   - a zero-length commit returns S0 bitwise;
 *   - the masks and depths agree with walking the parents;
 *   - non-topological parents are rejected, empty batches accepted. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdno_set_threads(int n);
int gdno_masks(int B, int N, const int32_t* parents, uint64_t* mask, int32_t* depth);
int gdno_tree_verify(int B, int N, int H, int dk, int dv, const double* S0,
                     const int32_t* parents, const double* q, const double* k,
                     const double* v, const double* beta, const double* g, double scale,
                     double* out, double* uprime, double* G);
int gdno_commit(int B, int N, int H, int dk, int dv, const double* S0, const int32_t* parents,
                const double* k, const double* v, const double* beta, const double* g,
                const int32_t* last_accepted, double* S_new, int32_t* path_out,
                int32_t* path_len);
int gdno_sequential_decode(int B, int N, int H, int dk, int dv, const double* S0,
                           const double* q, const double* k, const double* v,
                           const double* beta, const double* g, double scale, double* out,
                           double* S_final);

static int g_fail = 0, g_checks = 0;
#define CHECK(x)                                                   \
  do {                                                             \
    ++g_checks;                                                    \
    if (!(x)) {                                                    \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #x);       \
      ++g_fail;                                                    \
    }                                                              \
  } while (0)

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return (double)((g_rng * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}

static double* dalloc(size_t n) {
  double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = urand();
  return p;
}

static void run_case(int B, int N, int H, int dk, int dv, int threads) {
  gdno_set_threads(threads);
  const size_t nh = (size_t)B * N * H;
  double* S0 = dalloc((size_t)B * H * dv * dk);
  double* q = dalloc(nh * dk);
  double* k = dalloc(nh * dk);
  double* v = dalloc(nh * dv);
  double* beta = dalloc(nh);
  double* g = dalloc(nh);
  for (size_t i = 0; i < nh; ++i) {
    beta[i] = 0.5 + 0.5 * beta[i] * 0.9;
    g[i] = -0.5 - 0.5 * fabs(g[i]);
  }
  int32_t* chain = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * N);
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < N; ++t) chain[(size_t)b * N + t] = t - 1;

  /* chain verify == sequential decode, bitwise; commit of the last node ==
   * the decode's final state, bitwise */
  double* out = dalloc(nh * dv);
  double* up = dalloc(nh * dv);
  double* G = dalloc(nh);
  double* out_seq = dalloc(nh * dv);
  double* S_seq = dalloc((size_t)B * H * dv * dk);
  double* S_new = dalloc((size_t)B * H * dv * dk);
  int32_t* last = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B ? B : 1));
  int32_t* path = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B * N ? B * N : 1));
  int32_t* plen = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B ? B : 1));
  CHECK(gdno_tree_verify(B, N, H, dk, dv, S0, chain, q, k, v, beta, g, 0.5, out, up, G) == 0);
  CHECK(gdno_sequential_decode(B, N, H, dk, dv, S0, q, k, v, beta, g, 0.5, out_seq, S_seq) == 0);
  CHECK(memcmp(out, out_seq, sizeof(double) * nh * dv) == 0);
  for (int b = 0; b < B; ++b) last[b] = N - 1;
  CHECK(gdno_commit(B, N, H, dk, dv, S0, chain, k, v, beta, g, last, S_new, path, plen) == 0);
  if (N > 0) CHECK(memcmp(S_new, S_seq, sizeof(double) * (size_t)B * H * dv * dk) == 0);
  for (int b = 0; b < B; ++b) CHECK(plen[b] == N);

  /* zero-length commit returns S0 */
  for (int b = 0; b < B; ++b) last[b] = -1;
  CHECK(gdno_commit(B, N, H, dk, dv, S0, chain, k, v, beta, g, last, S_new, path, plen) == 0);
  CHECK(memcmp(S_new, S0, sizeof(double) * (size_t)B * H * dv * dk) == 0);

  /* a random tree: masks and depths against the parent walk; verify runs */
  int32_t* tree = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B * N ? B * N : 1));
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < N; ++t)
      tree[(size_t)b * N + t] = t == 0 ? -1 : (int32_t)((urand() + 1.0) * 0.5 * t);
  uint64_t* mask = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)(B * N ? B * N : 1));
  int32_t* depth = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B * N ? B * N : 1));
  CHECK(gdno_masks(B, N, tree, mask, depth) == 0);
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < N; ++t) {
      const int32_t p = tree[(size_t)b * N + t];
      const uint64_t want = (p >= 0 ? mask[(size_t)b * N + p] : 0) | ((uint64_t)1 << t);
      CHECK(mask[(size_t)b * N + t] == want);
      CHECK(depth[(size_t)b * N + t] == (p >= 0 ? depth[(size_t)b * N + p] : 0) + 1);
    }
  CHECK(gdno_tree_verify(B, N, H, dk, dv, S0, tree, q, k, v, beta, g, 0.5, out, up, G) == 0);
  for (int b = 0; b < B; ++b) last[b] = N - 1;
  CHECK(gdno_commit(B, N, H, dk, dv, S0, tree, k, v, beta, g, last, S_new, path, plen) == 0);
  for (int b = 0; b < B; ++b)
    if (N > 0) CHECK(plen[b] == depth[(size_t)b * N + N - 1]);

  /* rejected parents */
  if (B >= 1 && N >= 2) {
    tree[1] = 1;
    CHECK(gdno_masks(B, N, tree, mask, depth) != 0);
    CHECK(gdno_tree_verify(B, N, H, dk, dv, S0, tree, q, k, v, beta, g, 0.5, out, up, G) != 0);
    tree[1] = -2;
    CHECK(gdno_commit(B, N, H, dk, dv, S0, tree, k, v, beta, g, last, S_new, path, plen) != 0);
    tree[1] = 0;
    last[0] = N;
    CHECK(gdno_commit(B, N, H, dk, dv, S0, tree, k, v, beta, g, last, S_new, path, plen) != 0);
  }

  free(S0); free(q); free(k); free(v); free(beta); free(g); free(chain); free(out); free(up);
  free(G); free(out_seq); free(S_seq); free(S_new); free(last); free(path); free(plen);
  free(tree); free(mask); free(depth);
}

int main(void) {
  const int shapes[][5] = {{1, 1, 1, 4, 4},  {2, 7, 2, 8, 12}, {3, 13, 1, 16, 8},
                           {1, 64, 2, 8, 8}, {2, 33, 3, 5, 7}, {0, 8, 2, 8, 8},
                           {2, 0, 2, 8, 8}};
  for (int threads = 1; threads <= 4; threads += 3)
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
      run_case(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4], threads);
  printf("%d checks, %d failed\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
