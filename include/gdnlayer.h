/*
 * gdnlayer.h - C ABI of the layer scaffold around the GDN verifier in
 * libgdnspec: projections, the causal depthwise convolution evaluated along
 * draft-tree ancestor paths, SiLU output gating, the convolution-history
 * commit and a one-token recurrent decode step (the autoregressive baseline).
 *
 * Source: the Pith review of "SpecLA: Efficient Speculative Decoding for
 * Linear-Attention Models" (verdict page, skeptic critique; review page,
 * Referee Report major comment 1), which report the paper's Section 7 target
 * layer: Gated DeltaNet with 8 value heads of width 256, a width-4 causal
 * depthwise convolution and SiLU output gating.  The review page's axiom
 * ledger (paper Section 4.1, Figure 3) states the property the scaffold
 * relies on: running every draft node through layer l before layer l+1
 * gives what token-by-token decoding gives.  The rest of the layer follows
 * the usual GDN block:
 *
 *   P        = x W_in^T         columns q^ | k^ | v^ | gate
 *   q, k, v  = SiLU(conv4(q^, k^, v^)) along each node's root path, then
 *              q and k L2-normalised per head and rounded to bfloat16
 *   beta     = sigmoid(x . w_beta),  g = -softplus(x . w_alpha + gate_shift)
 *   o        = gdn_tree_verify(...)            (gdnspec.h)
 *   x_next   = x + (o * SiLU(gate)) W_o^T
 *
 * The 2H rows of the input projection that give the alpha and beta logits
 * are applied inside gdn_layer_prep (two dot products per node and head), so
 * the large projection has exactly 2H(dk + dv) columns.
 *
 * Conventions: the ones of gdnspec.h (status codes, 16-byte aligned device
 * pointers, caller-owned memory, work only enqueued on `stream`), plus:
 *   - bf16 arrays hold bfloat16 bits (uint16), rounded to nearest even.
 *   - Row-major, C-contiguous; "rows" are tokens or draft nodes.
 *   - Nothing is allocated; no state is kept between calls.
 */
#ifndef GDNLAYER_H
#define GDNLAYER_H

#include <stddef.h>
#include <stdint.h>

#include "gdnspec.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Weight layouts for gdn_linear. */
typedef enum {
  GDN_W_ROWS = 0,   /* bf16 [Nc][K], one output column per row (as in a linear layer) */
  GDN_W_PACKED = 1  /* the same values in MFMA fragment order, from gdn_pack_weights */
} gdn_wlayout_t;

/*
 * gdn_linear: C[m][n] = sum_k A[m][k] W[n][k] (+ R[m][n])  -- the block's
 * input and output projections (bf16 weights, FP32 accumulation).
 *   M      rows, 1 <= M <= 64 (the draft nodes of one sequence, or one token)
 *   Nc     output columns, Nc % 16 == 0
 *   K      reduction length, K % 256 == 0, 256 <= K <= 65536
 *   A      bf16 [M][K]
 *   W      bf16 weights in layout w_layout (GDN_W_ROWS or GDN_W_PACKED)
 *   R      optional FP32 [M][Nc] residual added to the product, or NULL
 *   C      optional FP32 [M][Nc] output, or NULL; may be the same buffer as R
 *          (each element is read before it is written by the same thread)
 *   C_bf16 optional bf16 [M][Nc] copy of C rounded to nearest even, or NULL
 * The sum order is fixed, so results are bitwise reproducible and identical
 * for both layouts.  M = 0 or Nc = 0 is a no-op.  Errors: GDN_ERR_SHAPE for
 * sizes out of range, GDN_ERR_ARG for a NULL A or W, an unknown layout, or
 * when C and C_bf16 are both NULL.
 */
int gdn_linear(int M, int Nc, int K, const void* A, const void* W, int w_layout, const float* R,
               float* C, void* C_bf16, void* stream);

/*
 * gdn_pack_weights: reorder W (bf16 [Nc][K]) into GDN_W_PACKED, the order in
 * which gdn_linear's matrix-core fragments read it: for each 16-column tile
 * and 32-wide k step, 64 lanes x 8 consecutive k values, lane l holding
 * column l % 16 and k offset 8 * (l / 16).  Each wave load is then one
 * contiguous kilobyte, which streams from HBM at the full rate (row-major
 * fragments touch 16 rows per load).  Done once per weight matrix.
 *   W_packed  bf16, Nc * K elements, must not overlap W
 * Same size limits as gdn_linear.
 */
int gdn_pack_weights(int Nc, int K, const void* W, void* W_packed, void* stream);

/*
 * gdn_layer_prep: the per-node inputs of the verifier from the projection
 * output P and the layer input x, for B sequences of N draft nodes, H heads
 * and hidden width D.
 *   P       FP32 [B][N][ldP], ldP = 2*H*(dk + dv); column blocks
 *           q^ [H*dk] | k^ [H*dk] | v^ [H*dv] | gate [H*dv]
 *   x       bf16 [B][N][D], the rows the projection consumed
 *   W_ab    bf16 [2H][D]: the input-projection rows of the alpha logits
 *           (heads 0..H-1) then of the beta logits
 *   parents int32 [B][N], -1 <= parents[t] < t (an entry outside that range
 *           is read as -1; gdn_tree_verify reports such a draft)
 *   conv_w  FP32 [Cc][4], Cc = H*(2*dk + dv): tap 0 multiplies the node's own
 *           input, tap i its i-th ancestor's (or the history's)
 *   hist    FP32 [B][3][Cc]: the pre-convolution inputs of the last three
 *           committed tokens, most recent first (zeros before any token)
 *   For channel c of node t with root path ... a_2, a_1, a_0 = t:
 *           conv[c] = sum_i conv_w[c][i] * X_i[c],  X_i = P[a_i] for i < depth(t),
 *           else hist[i - depth(t)]
 *   q, k    bf16 [B][N][H][dk]:  SiLU(conv) normalised to unit L2 norm per head
 *   v       bf16 [B][N][H][dv]:  SiLU(conv)
 *   beta, g FP32 [B][N][H]: sigmoid(x . W_ab[H + h]), -softplus(x . W_ab[h] + gate_shift)
 * Sizes as in gdnspec.h (N <= 64, dk, dv <= 256); 8 <= D <= 65536, D % 8 == 0.
 * Errors: GDN_ERR_SHAPE, GDN_ERR_ARG (NULL pointer, misalignment, non-finite
 * gate_shift).
 */
int gdn_layer_prep(int B, int N, int H, int dk, int dv, int D, const float* P, const void* x,
                   const void* W_ab, const int32_t* parents, const float* conv_w,
                   const float* hist, float gate_shift, void* q, void* k, void* v, float* beta,
                   float* g, void* stream);

/*
 * gdn_layer_prep_delayed: gdn_conv_commit of the previous step's accepted path
 * followed by gdn_layer_prep, in one launch, with the history double-buffered:
 *   hist       FP32 [B][3][Cc], the history before the previous step's commit
 *              (read only)
 *   P_prev     FP32 [B][N_prev][ldP], the previous step's projection output
 *   parents_prev int32 [B][N_prev], last_prev int32 [B] (-1: nothing accepted),
 *              the previous draft and its deepest accepted node
 *   hist_out   FP32 [B][3][Cc], written: the history after that commit,
 *              bitwise gdn_conv_commit's result (hist itself when last_prev is
 *              -1, out of range or on a rejected topology); must not overlap hist
 *   dev_status optional int32 [B]: GDN_OK, or GDN_ERR_TOPOLOGY when last_prev
 *              is out of range or parents_prev fails the verifier's topology
 *              check (some p[j] < -1 or p[j] >= j); the history then does not
 *              advance, as the state commit of that draft does not apply
 * The other arguments and all outputs are gdn_layer_prep's, computed from
 * hist_out, bitwise equal to gdn_conv_commit(P_prev, ...) followed by
 * gdn_layer_prep.  It is the history half of the delayed commit (SpecLA
 * review, Figures, Figure 7 caption, right side) for the block's causal
 * convolution (review: skeptic critique, on Section 7).  1 <= N_prev <= 64.
 * Errors: as gdn_layer_prep, plus GDN_ERR_SHAPE for N_prev and GDN_ERR_ARG for
 * overlapping histories or a NULL previous-step pointer.
 */
int gdn_layer_prep_delayed(int B, int N_prev, int N, int H, int dk, int dv, int D,
                           const float* P, const void* x, const void* W_ab,
                           const int32_t* parents, const float* conv_w, const float* hist,
                           float gate_shift, void* q, void* k, void* v, float* beta, float* g,
                           const float* P_prev, const int32_t* parents_prev,
                           const int32_t* last_prev, float* hist_out, int32_t* dev_status,
                           void* stream);

/*
 * gdn_gate_merge: Y[m][c] = bf16(o[m][c] * SiLU(gate[m][c])), the SiLU output
 * gate in front of the output projection.
 *   M, Cw   rows and columns, Cw % 4 == 0
 *   o       FP32 [M][Cw] (the verifier output [B][N][H][dv] has this shape)
 *   gate    FP32, row m at gate + m * ldg, ldg % 4 == 0, ldg >= Cw (the gate
 *           block of P: gate = P + H*(2*dk + dv), ldg = the P row length)
 *   Y       bf16 [M][Cw]
 */
int gdn_gate_merge(int M, int Cw, const float* o, const float* gate, int ldg, void* Y,
                   void* stream);

/*
 * gdn_layer_verify: the layer's tree verification with the SiLU output gate
 * fused into its epilogue, for bf16 q, k, v.  With prev_factors != NULL it is
 * gdn_tree_verify_delayed (the previous draft's accepted path is committed to
 * S first; N_prev, last_accepted and commit_status as there), else
 * gdn_tree_verify (S read only; N_prev, last_accepted ignored).  Instead of
 * the FP32 output O it writes
 *   Y  bf16 [B][N][H*dv]: Y[b][t][h*dv + c] = bf16(O[b][t][h][c] * SiLU(gate))
 *      with gate = gate[(b*N + t)*ldg + h*dv + c] (the gate block of P,
 *      ldg >= H*dv),
 * bitwise equal to the verify call followed by gdn_gate_merge on O.  The
 * factor record, S and the status words are exactly those of that verify call.
 * It is the verifier (SpecLA review, "Core claim"; "What carries the
 * argument") with the block's output gate (review: skeptic critique and
 * Referee Report major comment 1, both on Section 7) folded in, so a
 * layer's step saves the gate launch and the FP32 output round trip.
 * Errors: as the verify call, plus GDN_ERR_SHAPE for ldg < H*dv and GDN_ERR_ARG
 * for a NULL or misaligned gate or Y.
 */
int gdn_layer_verify(int B, int N_prev, int N, int H, int dk, int dv, float* S,
                     const void* prev_factors, const int32_t* last_accepted,
                     int32_t* commit_status, const int32_t* parents, const void* q,
                     const void* k, const void* v, const float* beta, const float* g,
                     float scale, const float* gate, int ldg, void* Y, void* factors,
                     int32_t* dev_status, void* stream);

/*
 * gdn_conv_commit: the convolution history after accepting the root path of
 * node last_accepted[b] (path p_1..p_n, root first): the new history is
 * P[p_n], P[p_{n-1}], ... followed by the old history, truncated to three
 * rows.  last_accepted[b] = -1 leaves hist[b] bitwise unchanged.
 *   P        FP32 [B][N][ldP]; the first Cc columns are the convolution inputs
 *   parents  int32 [B][N] as for gdn_layer_prep
 *   last_accepted int32 [B], -1 <= last < N
 *   hist     FP32 [B][3][Cc], updated in place
 *   dev_status optional int32 [B]: GDN_OK, or GDN_ERR_TOPOLOGY when last is
 *            out of range, or last >= 0 and parents fails the verifier's
 *            topology check (some p[j] < -1 or p[j] >= j): the rule under which
 *            gdn_commit_path rejects the same path.  hist[b] then stays
 *            unchanged
 * Cc % 4 == 0 and ldP % 4 == 0 are required.
 */
int gdn_conv_commit(int B, int N, int Cc, const float* P, int ldP, const int32_t* parents,
                    const int32_t* last_accepted, float* hist, int32_t* dev_status,
                    void* stream);

/*
 * gdn_decode_step: one token of the plain recurrence for B sequences, in place:
 *     S <- alpha S (I - beta k k^T) + beta v k^T,   out = scale * S q
 * (the recurrence of gdnspec.h with N = 1).  This is the one-token
 * autoregressive decode that speculative verification is measured against.
 *   S    FP32 [B][H][dv][dk], read and written once
 *   q, k [B][H][dk]; v [B][H][dv] in qkv_dtype; beta, g FP32 [B][H];
 *   out  FP32 [B][H][dv]
 * Sizes as in gdnspec.h.
 */
int gdn_decode_step(int B, int H, int dk, int dv, int qkv_dtype, float* S, const void* q,
                    const void* k, const void* v, const float* beta, const float* g,
                    float scale, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDNLAYER_H */
