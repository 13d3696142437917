/*
 * gdnspec.h - C ABI of libgdnspec: speculative-decoding verification and
 * accepted-path commit for Gated DeltaNet (GDN) layers on AMD Instinct MI355X
 * (gfx950).
 *
 * Operations (source: "SpecLA: Efficient Speculative Decoding for
 * Linear-Attention Models", pith.science review pages):
 *
 *   gdn_tree_verify   review "Core claim" / "What carries the argument"
 *                     (paper Section 4.2): every draft-tree node's output from
 *                     the committed state S0, with state updates flowing only
 *                     along ancestor paths (tree-masked factorized form).
 *   gdn_chain_verify  review "What carries the argument" and Figure 3 caption
 *                     (paper Section 4.1): a linear draft chain verified by a
 *                     serial recurrence that keeps V-dimension tiles of the
 *                     state on chip.
 *   gdn_commit_path   review "Core claim" and Figure 7 caption (paper
 *                     Section 5): rebuild the accepted state from the per-node
 *                     factors buffered during verification, without snapshots
 *                     or token replay.
 *
 * The recurrence, per head, with S in R^{dv x dk}, alpha_t = exp(g_t):
 *     S_t = alpha_t S_{p(t)} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t                   (readout after the update)
 * where p(t) is node t's parent (S_{-1} = S0).  Writing
 *     u'_t = beta_t (v_t - alpha_t S_{p(t)} k_t)  gives  S_t = alpha_t S_{p(t)} + u'_t k_t^T.
 *
 * Conventions shared by every call
 *   - B sequences, N draft nodes (1 <= N <= 64), H heads, key width dk and
 *     value width dv: 8 <= dk <= 256 with dk % 8 == 0; 4 <= dv <= 256 with
 *     dv % 4 == 0.  B = 0 or N = 0 is a valid no-op.
 *   - All arrays are C-contiguous device memory unless stated; every base
 *     pointer must be 16-byte aligned.  The caller owns and allocates all
 *     memory; the library allocates nothing and keeps no state between calls
 *     except the thread-local error text.
 *   - State S: float32 [B][H][dv][dk] (state rows run along dk).
 *   - q, k: [B][N][H][dk]; v: [B][N][H][dv]; element type GDN_BF16 (bfloat16
 *     bits) or GDN_F32, the same for all three.
 *   - beta, g: float32 [B][N][H]; beta in [0, 1], g = log(alpha) <= 0.
 *   - out: float32 [B][N][H][dv].
 *   - parents: int32 [B][N], topologically numbered: -1 <= parents[t] < t
 *     (node 0 is a root; other -1 entries start further roots).
 *   - stream: a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues work on it and returns; results are valid once the
 *     stream has reached that point.  A commit must be ordered after the
 *     verify that wrote its factor record (same stream or an event).
 *
 * Return values are gdn_status_t.  Host-checkable faults (null required
 * pointer, misalignment, unsupported size or dtype) return before anything is
 * enqueued.  Faults only visible on the device (a parent array that is not
 * topological, last_accepted out of range) are reported per sequence through
 * the optional dev_status arrays; the affected sequence's outputs are zeros
 * and its commit leaves S untouched.  A HIP launch failure returns
 * GDN_ERR_HIP.  gdn_last_error() describes the last non-OK status of the
 * calling thread.  No C++ exception crosses this interface.
 */
#ifndef GDNSPEC_H
#define GDNSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_ARG = -1,         /* null/misaligned pointer, bad dtype or scale */
  GDN_ERR_SHAPE = -2,       /* size outside the supported range */
  GDN_ERR_TOPOLOGY = -3,    /* (device status) parents not topological, bad last_accepted */
  GDN_ERR_UNSUPPORTED = -4, /* combination not implemented */
  GDN_ERR_HIP = -5          /* HIP runtime error while enqueuing */
} gdn_status_t;

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype_t;

/* Library version, (major << 16) | minor. */
int gdn_version(void);

/* Text for the calling thread's last non-OK status ("" if none). */
const char* gdn_last_error(void);

/*
 * Factor record: what verification buffers per node so that a later commit
 * can rebuild the accepted state (review "Core claim": buffer the small
 * per-token factors produced during verification).  Self-contained: q, k, v
 * may be freed before the commit.  Sections, each starting on a 256-byte
 * boundary, in this order:
 *   0  u'       float32 [B][H][N][dv]   per-node state write u'_t
 *   1  G        float32 [B][H][N]       path-cumulative log decay
 *                                       G_t = sum of g_j over the root-to-t path
 *   2  K        [B][H][N][dk]           copy of k (element type of q/k/v)
 *   3  parents  int32  [B][N]           copy of the parent array
 *   4  mask     uint64 [B][N]           ancestor-or-self bitmask (bit j of
 *                                       mask[t] set iff j is on t's root path);
 *                                       all zero for a sequence whose
 *                                       topology was rejected
 * gdn_factor_bytes returns the total size (0 for invalid sizes);
 * gdn_factor_layout writes the 5 section byte offsets.
 */
size_t gdn_factor_bytes(int B, int N, int H, int dk, int dv, int qkv_dtype);
int gdn_factor_layout(int B, int N, int H, int dk, int dv, int qkv_dtype, size_t offsets[5]);

/* Device scratch gdn_tree_verify needs (caller-allocated, 256-byte aligned,
 * no initialisation required).  This version needs none and returns 0; the
 * workspace argument is reserved and may be NULL. */
size_t gdn_workspace_bytes(int B, int N, int H, int dk, int dv);

/*
 * gdn_tree_verify - tree-masked factorized verification (review "Core claim";
 * paper Section 4.2).  For each (sequence, head), with M the ancestor mask
 * of the draft tree, G the path-cumulative log decays and the garbled
 * symbols of the pages read as A[t,j] = beta_t e^{G_t-G_j} (k_t . k_j) on
 * strict ancestors j, T = (I + A)^{-1}, Attn[t,j] = e^{G_t-G_j} (q_t . k_j)
 * on ancestors-or-self j:
 *     U' = T diag(beta) V - T diag(beta e^G) K S0^T
 *     O  = scale * (diag(e^G) Q S0^T + Attn U')
 * which equals the recurrence above replayed separately along every
 * root-to-node path from S0.
 *   S0        [B][H][dv][dk] float32, read only
 *   parents   [B][N] int32
 *   q, k, v   see conventions; qkv_dtype says their element type
 *   beta, g   [B][N][H] float32
 *   scale     query scale (1.0f: none)
 *   out       [B][N][H][dv] float32, written
 *   factors   gdn_factor_bytes(...) bytes, written (record for the commit)
 *   workspace gdn_workspace_bytes(...) bytes (reserved; may be NULL when 0)
 *   mask_out  optional [B][N] uint64 ancestor-or-self masks, or NULL
 *   dev_status optional [B] int32: GDN_OK or GDN_ERR_TOPOLOGY per sequence
 */
int gdn_tree_verify(int B, int N, int H, int dk, int dv, int qkv_dtype, const float* S0,
                    const int32_t* parents, const void* q, const void* k, const void* v,
                    const float* beta, const float* g, float scale, float* out,
                    void* factors, void* workspace, uint64_t* mask_out,
                    int32_t* dev_status, void* stream);

/*
 * gdn_chain_verify - serial verification of a linear chain (parent of node t
 * is t - 1) with V-dimension tiling (review "What carries the argument";
 * Figure 3 caption; paper Section 4.1).  Each workgroup keeps a tile of state
 * rows in registers and runs the recurrence over the N nodes; S0 is never
 * written.  Same arguments and outputs as gdn_tree_verify (the record's
 * parents are t - 1 and its masks the prefixes); no workspace is needed.
 */
int gdn_chain_verify(int B, int N, int H, int dk, int dv, int qkv_dtype, const float* S0,
                     const void* q, const void* k, const void* v, const float* beta,
                     const float* g, float scale, float* out, void* factors, void* stream);

/*
 * gdn_commit_path - accepted-state recovery from the factor record (review
 * "Core claim", Figure 7 caption; paper Section 5).  For each sequence b with
 * last = last_accepted[b] and root-first accepted path p_1..p_n (the nodes
 * of mask[last]):
 *     S <- e^{G_last} S + sum_i e^{G_last - G_{p_i}} u'_{p_i} k_{p_i}^T
 * in place.  last = -1 is a zero-length commit: S is left bitwise unchanged.
 *   S             [B][H][dv][dk] float32, in place: must hold the S0 the
 *                 verify that wrote `factors` started from
 *   factors       record written by gdn_tree_verify / gdn_chain_verify with
 *                 the same B, N, H, dk, dv and qkv_dtype
 *   last_accepted [B] int32 device array, -1 <= last < N
 *   path_out      optional [B][N] int32: accepted path root first, -1 padded
 *   path_len_out  optional [B] int32: n (0 for a zero-length commit, -1 on
 *                 a rejected sequence)
 *   dev_status    optional [B] int32: GDN_OK, or GDN_ERR_TOPOLOGY when
 *                 last_accepted is out of range or the record's topology was
 *                 rejected (S untouched)
 */
int gdn_commit_path(int B, int N, int H, int dk, int dv, int qkv_dtype, float* S,
                    const void* factors, const int32_t* last_accepted, int32_t* path_out,
                    int32_t* path_len_out, int32_t* dev_status, void* stream);

/*
 * gdn_chain_verify_delayed - the delayed commit fused into the next
 * verification (review: Referee Report summary, mechanism (ii); Figures,
 * Figure 7 caption, right side; paper Section 5): the accepted-factor buffer
 * of the previous draft is applied inside the next verification kernel, on
 * the state tiles it loads anyway, so the commit costs no state round trip of
 * its own.  Equivalent to
 *     gdn_commit_path(B, N_prev, H, dk, dv, qkv_dtype, S, prev_factors,
 *                     last_accepted, NULL, NULL, dev_status, stream);
 *     gdn_chain_verify(B, N, H, dk, dv, qkv_dtype, S, q, k, v, beta, g,
 *                      scale, out, factors, stream);
 * and bitwise identical to them: each workgroup reads its state tile once,
 * applies the accepted path in the commit's operation order, writes the tile
 * back and verifies the new chain from registers.
 *   S             [B][H][dv][dk] float32, in place: on entry the state the
 *                 previous verification started from; on return the state
 *                 after its accepted path
 *   prev_factors  the previous verification's record, written with
 *                 (B, N_prev, H, dk, dv, qkv_dtype), 1 <= N_prev <= 64
 *   last_accepted [B] int32, -1 <= last < N_prev (-1: nothing to commit)
 *   dev_status    optional [B] int32: GDN_OK, or GDN_ERR_TOPOLOGY when
 *                 last_accepted is out of range or the previous record's
 *                 topology was rejected; that sequence's state is then left
 *                 as it was and the new chain is verified from it
 *   factors       the new record; must not overlap prev_factors
 *   other arguments as for gdn_chain_verify
 * One workgroup stages the new draft and the previous record's k rows in its
 * 160 KiB of LDS: with float32 q/k/v and large N + N_prev (e.g. 64 + 64 at
 * dk = 256) that does not fit, and the call returns GDN_ERR_UNSUPPORTED
 * before launching anything (bf16 inputs fit at every size).
 */
int gdn_chain_verify_delayed(int B, int N_prev, int N, int H, int dk, int dv, int qkv_dtype,
                             float* S, const void* prev_factors, const int32_t* last_accepted,
                             int32_t* dev_status, const void* q, const void* k, const void* v,
                             const float* beta, const float* g, float scale, float* out,
                             void* factors, void* stream);

/*
 * gdn_tree_verify_delayed - the delayed commit fused into the next tree
 * verification (same passages as gdn_chain_verify_delayed).  Equivalent to
 *     gdn_commit_path(B, N_prev, H, dk, dv, qkv_dtype, S, prev_factors,
 *                     last_accepted, NULL, NULL, commit_status, stream);
 *     gdn_tree_verify(B, N, H, dk, dv, qkv_dtype, S, parents, q, k, v, beta,
 *                     g, scale, out, factors, workspace, mask_out,
 *                     dev_status, stream);
 * with the committed state bitwise that of gdn_commit_path: each workgroup
 * applies the previous accepted path to the state tile it loads for the
 * verification, writes the tile back once and verifies from the registers.
 * The commit takes place even when the new draft's topology is rejected.
 *   S             in place, as for gdn_chain_verify_delayed
 *   prev_factors, N_prev, last_accepted   as for gdn_chain_verify_delayed
 *   commit_status optional [B] int32: GDN_OK, or GDN_ERR_TOPOLOGY when
 *                 last_accepted is out of range or the previous record's
 *                 topology was rejected (that sequence's state is then left
 *                 as it was)
 *   dev_status    optional [B] int32: the new draft's topology, as in
 *                 gdn_tree_verify
 *   factors       the new record; must not overlap prev_factors
 *   other arguments as for gdn_tree_verify
 */
int gdn_tree_verify_delayed(int B, int N_prev, int N, int H, int dk, int dv, int qkv_dtype,
                            float* S, const void* prev_factors, const int32_t* last_accepted,
                            int32_t* commit_status, const int32_t* parents, const void* q,
                            const void* k, const void* v, const float* beta, const float* g,
                            float scale, float* out, void* factors, void* workspace,
                            uint64_t* mask_out, int32_t* dev_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDNSPEC_H */
