/*
 * CPU oracle for tree-masked Gated DeltaNet verification and accepted-path commit.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; it exists so tests, the smoke check and the benchmark's CPU
 * baseline can compare the GPU library against a plain definition.  It shares
 * no code with the GPU library.
 *
 * What it computes (plain definition, float64 throughout):
 *   The Gated DeltaNet recurrence that the SpecLA review pages name (the
 *   review's "Circularity Check" refers to the paper's Equations 1-3; its
 *   axiom ledger lists the per-token factors (k, v, alpha, beta)):
 *
 *       S_t = alpha_t * S_{p(t)} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *       o_t = scale * S_t q_t
 *
 *   with S in R^{dv x dk} (rows along d_k), alpha_t = exp(g_t), and p(t) the
 *   node's parent in the draft tree.  Every node's output is obtained by
 *   replaying the recurrence from the committed state S0 along its own
 *   root-to-node path, separately for each node (no sharing between paths):
 *   this is the "sequential token-by-token GDN recurrence" that the review's
 *   falsifier ("What would settle it") asks the factorized verifier to match.
 *
 *   The commit replays the accepted root-to-node path from S0 (review "Core
 *   claim": only the accepted path is applied to the state); a zero-length
 *   path (last_accepted = -1) returns S0 unchanged.
 *
 *   Side outputs used to check the GPU factor record:
 *     uprime[t] = beta_t (v_t - alpha_t S_{p(t)} k_t)  (the vector written
 *                 into the state by node t: S_t = alpha_t S_{p(t)} + u'_t k_t^T)
 *     G[t]      = sum of g_j over the root-to-node path of t, root first.
 *
 * Layouts (C order): S0 [B][H][dv][dk]; q,k [B][N][H][dk]; v [B][N][H][dv];
 * beta,g [B][N][H]; parents [B][N]; out [B][N][H][dv]; uprime [B][H][N][dv];
 * G [B][H][N]; S_new [B][H][dv][dk]; path [B][N]; path_len [B].
 *
 * Return value: 0 on success, -3 for a parent array that is not topological
 * (-1 <= p[t] < t), -1 for bad sizes / last_accepted out of range.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int check_parents(int B, int N, const int32_t* parents) {
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < N; ++t) {
      int p = parents[(size_t)b * N + t];
      if (p < -1 || p >= t) return -3;
    }
  return 0;
}

/* Root-first path of node t; returns its length. */
static int walk_path(const int32_t* par, int t, int* path) {
  int m = 0;
  for (int u = t; u >= 0; u = par[u]) path[m++] = u;
  for (int i = 0; i < m / 2; ++i) {
    int x = path[i];
    path[i] = path[m - 1 - i];
    path[m - 1 - i] = x;
  }
  return m;
}

/* One recurrence step on the dense state (dv x dk), returning u' in u. */
static void gdn_step(double* S, int dk, int dv, const double* kj, const double* vj,
                     double beta, double alpha, double* u) {
  for (int r = 0; r < dv; ++r) {
    const double* Sr = S + (size_t)r * dk;
    double y = 0.0;
    for (int c = 0; c < dk; ++c) y += Sr[c] * kj[c];
    u[r] = beta * (vj[r] - alpha * y);
  }
  for (int r = 0; r < dv; ++r) {
    double* Sr = S + (size_t)r * dk;
    for (int c = 0; c < dk; ++c) Sr[c] = alpha * Sr[c] + u[r] * kj[c];
  }
}

int gdno_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* Ancestor-or-self bitmask and depth of every node, by walking parents. */
int gdno_masks(int B, int N, const int32_t* parents, uint64_t* mask, int32_t* depth) {
  if (B < 0 || N < 0 || N > 64) return -1;
  int rc = check_parents(B, N, parents);
  if (rc) return rc;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < N; ++t) {
      uint64_t m = 0;
      int d = 0;
      for (int u = t; u >= 0; u = parents[(size_t)b * N + u]) {
        m |= (uint64_t)1 << u;
        ++d;
      }
      mask[(size_t)b * N + t] = m;
      depth[(size_t)b * N + t] = d;
    }
  return 0;
}

/* Per-node outputs by per-path replay from S0. */
int gdno_tree_verify(int B, int N, int H, int dk, int dv, const double* S0,
                     const int32_t* parents, const double* q, const double* k,
                     const double* v, const double* beta, const double* g, double scale,
                     double* out, double* uprime, double* G) {
  if (B < 0 || N < 0 || H < 1 || dk < 1 || dv < 1) return -1;
  int rc = check_parents(B, N, parents);
  if (rc) return rc;
  const long units = (long)B * H * N;
  int failed = 0;
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    int* path = (int*)malloc(sizeof(int) * (size_t)(N > 0 ? N : 1));
    if (!S || !u || !path) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long w = 0; w < units; ++w) {
        const int t = (int)(w % N);
        const int h = (int)((w / N) % H);
        const int b = (int)(w / ((long)N * H));
        const int32_t* par = parents + (size_t)b * N;
        const int m = walk_path(par, t, path);
        memcpy(S, S0 + ((size_t)b * H + h) * dv * dk, sizeof(double) * (size_t)dv * dk);
        double Gt = 0.0;
        for (int i = 0; i < m; ++i) {
          const int j = path[i];
          const size_t nh = ((size_t)b * N + j) * H + h;
          Gt += g[nh];
          gdn_step(S, dk, dv, k + nh * dk, v + nh * dv, beta[nh], exp(g[nh]), u);
        }
        const size_t th = ((size_t)b * N + t) * H + h;
        const double* qt = q + th * dk;
        double* o = out + th * dv;
        for (int r = 0; r < dv; ++r) {
          const double* Sr = S + (size_t)r * dk;
          double acc = 0.0;
          for (int c = 0; c < dk; ++c) acc += Sr[c] * qt[c];
          o[r] = scale * acc;
        }
        if (uprime) memcpy(uprime + (((size_t)b * H + h) * N + t) * dv, u, sizeof(double) * dv);
        if (G) G[((size_t)b * H + h) * N + t] = Gt;
      }
    }
    free(S);
    free(u);
    free(path);
  }
  return failed ? -1 : 0;
}

/* Replay the accepted path of each sequence from S0 into S_new. */
int gdno_commit(int B, int N, int H, int dk, int dv, const double* S0,
                const int32_t* parents, const double* k, const double* v,
                const double* beta, const double* g, const int32_t* last_accepted,
                double* S_new, int32_t* path_out, int32_t* path_len) {
  if (B < 0 || N < 0 || H < 1 || dk < 1 || dv < 1) return -1;
  int rc = check_parents(B, N, parents);
  if (rc) return rc;
  for (int b = 0; b < B; ++b)
    if (last_accepted[b] < -1 || last_accepted[b] >= N) return -1;
  const long units = (long)B * H;
  int failed = 0;
#pragma omp parallel
  {
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    int* path = (int*)malloc(sizeof(int) * (size_t)(N > 0 ? N : 1));
    if (!u || !path) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long w = 0; w < units; ++w) {
        const int h = (int)(w % H);
        const int b = (int)(w / H);
        const int last = last_accepted[b];
        double* S = S_new + ((size_t)b * H + h) * dv * dk;
        memcpy(S, S0 + ((size_t)b * H + h) * dv * dk, sizeof(double) * (size_t)dv * dk);
        const int m = last >= 0 ? walk_path(parents + (size_t)b * N, last, path) : 0;
        for (int i = 0; i < m; ++i) {
          const size_t nh = ((size_t)b * N + path[i]) * H + h;
          gdn_step(S, dk, dv, k + nh * dk, v + nh * dv, beta[nh], exp(g[nh]), u);
        }
        if (h == 0) {
          if (path_len) path_len[b] = m;
          if (path_out)
            for (int i = 0; i < N; ++i) path_out[(size_t)b * N + i] = i < m ? path[i] : -1;
        }
      }
    }
    free(u);
    free(path);
  }
  return failed ? -1 : 0;
}

/* Plain token-by-token decode of a linear sequence of N tokens, carrying one
 * running state per (b, h): the autoregressive schedule the verifier replaces.
 * Writes every token's output and the final state. */
int gdno_sequential_decode(int B, int N, int H, int dk, int dv, const double* S0,
                           const double* q, const double* k, const double* v,
                           const double* beta, const double* g, double scale,
                           double* out, double* S_final) {
  if (B < 0 || N < 0 || H < 1 || dk < 1 || dv < 1) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double* u = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!u) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long w = 0; w < (long)B * H; ++w) {
        const int h = (int)(w % H);
        const int b = (int)(w / H);
        double* S = S_final + ((size_t)b * H + h) * dv * dk;
        memcpy(S, S0 + ((size_t)b * H + h) * dv * dk, sizeof(double) * (size_t)dv * dk);
        for (int t = 0; t < N; ++t) {
          const size_t nh = ((size_t)b * N + t) * H + h;
          gdn_step(S, dk, dv, k + nh * dk, v + nh * dv, beta[nh], exp(g[nh]), u);
          double* o = out + nh * dv;
          for (int r = 0; r < dv; ++r) {
            const double* Sr = S + (size_t)r * dk;
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += Sr[c] * q[nh * dk + c];
            o[r] = scale * acc;
          }
        }
      }
    }
    free(u);
  }
  return failed ? -1 : 0;
}
