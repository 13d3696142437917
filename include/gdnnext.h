/*
 * gdnnext.h: the verifier's companions beyond the verify/commit core of
 * gdnspec.h, on the same conventions (sizes, layouts, dtypes, status codes,
 * the caller's HIP stream, nothing allocated, host-checkable faults returned
 * before any launch).
 *
 * Sources: the Pith review of "SpecLA: Efficient Speculative Decoding for
 * Linear-Attention Models" (arXiv 2607.16673), in its HTML page (sections as
 * named there) and its JSON verdict page.
 *
 *   gdn_replay_verify, gdn_replay_commit  the replay mechanisms the paper
 *       measures its kernels against (review, Referee Report major comment 3;
 *       Figures, Figure 10 and Figure 11 captions).
 *   gdn_hybrid_plan, gdn_hybrid_verify     the chain-decomposed hybrid
 *       verifier (review, "What carries the argument"; Figures, Figure 6
 *       caption).
 *   gdn_prune_draft                        confidence-guided pruning of a
 *       candidate tree before verification (review, Figures, Figure 8
 *       caption).
 */
#ifndef GDNNEXT_H
#define GDNNEXT_H

#include <stddef.h>
#include <stdint.h>

#include "gdnspec.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gdn_replay_verify: root-to-leaf replay, the baseline of tree verification
 * (review, Figures, Figure 10 caption: tree verification against replaying
 * the draft's root-to-leaf paths; Referee Report major comment 3).  For each
 * sequence b and path slot p with end node e = ends[b][p] (-1: empty slot),
 * the gated delta rule is replayed from S0 along the root path of e, node by
 * node (S_t = alpha_t S_p (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 * o_t = scale S_t q_t), by a serial state-resident kernel, one launch for all
 * slots.  Every slot writes the outputs of all nodes on its path: a node's
 * value depends only on its own root path, replayed in the same order by
 * every slot that holds it, so those writes carry the same bits.  With the
 * leaves as ends every node is written and the outputs are gdn_tree_verify's
 * (up to rounding).  S0 is not modified; no factor record is written.
 *   B, N, H, dk, dv, qkv_dtype, S0, parents, q, k, v, beta, g, scale, out:
 *            as gdn_tree_verify (out rows of nodes on no path are left as they were)
 *   ends     int32 [B][P] device: path end nodes, -1 for an empty slot
 *   P        1 <= P <= 64 slots per sequence
 *   dev_status optional int32 [B]: GDN_OK, or GDN_ERR_TOPOLOGY when parents
 *            fails the topology check (-1 <= p[t] < t) or an end lies outside
 *            -1..N-1; that sequence is then not replayed (or, for one bad end,
 *            that slot only)
 * Errors: GDN_ERR_SHAPE (sizes as gdn_tree_verify, P), GDN_ERR_ARG (NULL or
 * misaligned pointers, non-finite scale).
 */
int gdn_replay_verify(int B, int N, int H, int dk, int dv, int qkv_dtype, const float* S0,
                      const int32_t* parents, const void* q, const void* k, const void* v,
                      const float* beta, const float* g, float scale, const int32_t* ends,
                      int P, float* out, int32_t* dev_status, void* stream);

/*
 * gdn_replay_commit: token replay, the baseline of the factor-buffer commit
 * (review, Figures, Figure 11 caption: accepted-state recovery against token
 * replay).  For each sequence, the accepted path root..last_accepted[b] is
 * replayed from S through the recurrence, token by token, with the state rows
 * held on chip, and S is overwritten with the result (last_accepted[b] = -1:
 * S[b] untouched).  Unlike gdn_commit_path it needs the draft's k, v, beta, g
 * (not a factor record) and recomputes S k_t for every token.
 *   S        FP32 [B][H][dv][dk] device, updated in place
 *   parents, k, v, beta, g: as gdn_tree_verify
 *   last_accepted int32 [B] device
 *   dev_status optional int32 [B]: GDN_OK, or GDN_ERR_TOPOLOGY (bad parents
 *            or last_accepted outside -1..N-1; S[b] then untouched)
 * Errors: as gdn_replay_verify.
 */
int gdn_replay_commit(int B, int N, int H, int dk, int dv, int qkv_dtype, float* S,
                      const int32_t* parents, const void* k, const void* v, const float* beta,
                      const float* g, const int32_t* last_accepted, int32_t* dev_status,
                      void* stream);

/*
 * gdn_hybrid_plan_entries: int32 entries of a hybrid plan, 2 * N * B * N.
 */
size_t gdn_hybrid_plan_entries(int B, int N);

/*
 * gdn_hybrid_plan: on the host, cut each draft tree into chains and order
 * them into dependency levels, for gdn_hybrid_verify (review, "What carries
 * the argument": serial kernels inside dependency-respecting chains,
 * parallel across ready chains).  A node continues its parent's chain when it
 * is the parent's lowest-numbered child; every other node (and every root)
 * heads a chain.  A chain's level is 0 for a root's chain, else one more than
 * the level of the chain holding its head's parent.
 *   parents  int32 [B][N], host memory (the same values the device copy holds)
 *   plan     int32 [N][B][N][2], host, written: plan[((l*B + b)*N + c)*2 + 0 / 1]
 *            = head / last node of the c-th chain of level l of sequence b,
 *            -1 past the last chain
 *   chains_per_level int32 [N], host, written: the most chains any sequence
 *            has at level l (0 past the last level)
 *   levels   int32, host, written: the number of levels (1 <= levels <= N)
 * Errors: GDN_ERR_SHAPE (B < 1, N outside 1..64), GDN_ERR_ARG (NULL),
 * GDN_ERR_TOPOLOGY (some p[t] < -1 or p[t] >= t; nothing usable is written).
 * Runs on the calling thread; no device work.
 */
int gdn_hybrid_plan(int B, int N, const int32_t* parents, int32_t* plan,
                    int32_t* chains_per_level, int32_t* levels);

/*
 * gdn_hybrid_verify: tree verification by chains (review, "What carries the
 * argument"; Figures, Figure 6 caption).  One launch per level of the plan;
 * each runs every chain of that level for every (sequence, head, 8 state
 * rows) in parallel.  A chain with head c under parent p first rebuilds the
 * state after p from the committed state and the factors that lower levels
 * buffered, S_p = e^{G_p} S0 + sum_{j on p's root path} e^{G_p - G_j} u'_j k_j^T,
 * then runs the recurrence serially along the chain with the state rows on
 * chip.  Outputs and the factor record equal gdn_tree_verify's (up to
 * rounding), so gdn_commit_path applies the record unchanged.
 *   B, N, H, dk, dv, qkv_dtype, S0, parents, q, k, v, beta, g, scale, out,
 *   factors: as gdn_tree_verify (S0 read only)
 *   plan     int32 [N][B][N][2] device: gdn_hybrid_plan's plan for the same
 *            parents (a chain that does not fit them is skipped)
 *   levels, chains_per_level: gdn_hybrid_plan's outputs (host memory)
 *   dev_status optional int32 [B]: GDN_OK, or GDN_ERR_TOPOLOGY when the device
 *            parents fail the topology check (that sequence's outputs and
 *            record rows are zeroed)
 * Errors: as gdn_tree_verify, plus GDN_ERR_SHAPE for levels outside 1..N or a
 * level with no chain or more than N.
 */
int gdn_hybrid_verify(int B, int N, int H, int dk, int dv, int qkv_dtype, const float* S0,
                      const int32_t* parents, const void* q, const void* k, const void* v,
                      const float* beta, const float* g, float scale, float* out,
                      void* factors, const int32_t* plan, int levels,
                      const int32_t* chains_per_level, int32_t* dev_status, void* stream);

/*
 * gdn_prune_draft: confidence-guided pruning of a candidate draft tree
 * (review, Figures, Figure 8 caption; Axiom & Free-Parameter Ledger: tree
 * margin tau_tree, draft budget).  Per sequence b, with q[t] the confidence of
 * candidate t (a path score that never increases from a node to its
 * children, such as the cumulative log-probability) and q* = max_t q[t]:
 *   window  = {t : q[t] >= q* - tau}, the threshold formed in FP32, which is
 *             ancestor-closed because q never increases along a path;
 *   kept    = the first T window nodes in the order (q descending, index
 *             ascending): every parent precedes its children, so the kept set
 *             is ancestor-closed too;
 *   outputs = the kept nodes in their original order, renumbered 0..n-1.
 *   B        sequences; M candidates per sequence, 1 <= M <= 1024
 *   T        budget, 1 <= T <= 64 (a draft the verifiers take)
 *   tau      tree margin, finite, >= 0
 *   parents  int32 [B][M] device, topological: -1 <= parents[t] < t
 *   conf     FP32 [B][M] device: q, no NaN, q[t] <= q[parents[t]]
 *   kept     int32 [B][T] device, written: kept[b][i] = the original index of
 *            new node i, -1 past the count
 *   new_parents int32 [B][T] device, written: the parent of new node i in the
 *            new numbering (-1 for a root), -1 past the count
 *   count    int32 [B] device, written: the number of kept nodes, or -1 when
 *            the candidates break a precondition (kept, new_parents all -1)
 *   dev_status optional int32 [B]: GDN_OK, or GDN_ERR_TOPOLOGY for broken
 *            preconditions
 * Integer outputs: they depend on q only through FP32 comparisons.
 * Errors: GDN_ERR_SHAPE (B < 0, M, T), GDN_ERR_ARG (NULL or misaligned
 * pointers, tau not finite or negative).
 */
int gdn_prune_draft(int B, int M, int T, float tau, const int32_t* parents, const float* conf,
                    int32_t* kept, int32_t* new_parents, int32_t* count, int32_t* dev_status,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDNNEXT_H */
