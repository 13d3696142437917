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
 * slots.  Node t's output is written by the first slot (lowest p) whose path
 * holds t, so with the leaves as ends every node is written once and the
 * outputs are gdn_tree_verify's (up to rounding).  S0 is not modified; no
 * factor record is written.
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

#ifdef __cplusplus
}
#endif

#endif /* GDNNEXT_H */
