"""Speculative and autoregressive decoding through a stack of GDN layers.

Sequencing and device buffers only: every arithmetic step is a libgdnspec
call (``gdnspec.py``).  Verification is layer-major (the Pith review's axiom
ledger, paper Section 4.1): all N draft nodes of a step go through layer l
before layer l + 1, so each layer's weights are read once per step instead
of once per node.  Per layer and step:

    gdn_linear       P = bf16(x) W_in^T   (q^ k^ v^ gate columns)
    gdn_layer_prep   conv along ancestor paths + SiLU + L2 norm; beta, g from
                     the last 2H rows of W_in
    gdn_layer_verify every node's output from the committed state (the tree
                     verifier), gated in its epilogue: bf16(o * SiLU(gate))
    gdn_linear       x <- x + (...) W_o^T   (FP32 residual, bf16 copy for the next layer)

and once the accepted node is known, per layer: gdn_commit_path (state) and
gdn_conv_commit (convolution history).  With the delayed commit (the
review's Figure 7 caption, right side), a step instead carries the previous
step's accepted node into every layer: gdn_layer_prep_delayed shifts the
previous path into the convolution history inside the layer's prep, and
gdn_layer_verify (as gdn_tree_verify_delayed) applies it to the layer's state
inside the verification; records, projection outputs and histories alternate
between two buffers per layer, and flush() applies the last pending commit.  The autoregressive baseline runs one token
per step through the same layers with gdn_decode_step in place of verify +
commit.
"""

from __future__ import annotations

from typing import List

import numpy as np
import torch

from . import gdnspec as G
from .workloads import StackShape

PK = G.GDN_W_PACKED


def _bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(
        torch.bfloat16)


def _f32(x: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)


class GdnStack:
    """Device weights, per-layer states and histories, and work buffers for
    B sequences verifying N-node drafts."""

    def __init__(self, shape: StackShape, B: int = 1, N: int = 32, device="cuda",
                 gate_shift: float = 2.0):
        if B * N > 64:
            raise ValueError("B * N must be at most 64 (rows of one projection)")
        self.shape, self.B, self.N, self.device = shape, B, N, device
        self.gate_shift = float(gate_shift)
        L, D, H, dk, dv = shape.layers, shape.D, shape.H, shape.dk, shape.dv
        bf, f32 = torch.bfloat16, torch.float32
        e = lambda *s, dt=f32: torch.empty(*s, dtype=dt, device=device)
        # projection weights in the packed fragment layout; the 2H logit rows of
        # the input projection stay row-major for gdn_layer_prep
        self.W_in = e(L, shape.n_proj, D, dt=bf)
        self.W_ab = e(L, 2 * H, D, dt=bf)
        self.W_o = e(L, D, H * dv, dt=bf)
        self.conv_w = e(L, shape.n_conv, 4)
        self.S = torch.zeros(L, B, H, dv, dk, dtype=f32, device=device)
        # conv histories, two sets: a delayed step reads one and writes the other
        self.hists = torch.zeros(2, L, B, 3, shape.n_conv, dtype=f32, device=device)
        self.hc = 0  # the set holding the committed history
        # speculative step buffers (M = B * N rows)
        M = B * N
        self.x = e(M, D)
        self.xb = e(M, D, dt=bf)
        self.P = e(2, L, B, N, shape.n_proj)  # two sets, used by alternate steps
        self.q = e(B, N, H, dk, dt=bf)
        self.k = e(B, N, H, dk, dt=bf)
        self.v = e(B, N, H, dv, dt=bf)
        self.beta = e(B, N, H)
        self.g = e(B, N, H)
        self.out = e(B, N, H, dv)
        self.Y = e(M, H * dv, dt=bf)
        self.rec: List[List[G.FactorRecord]] = [
            [G.FactorRecord.empty(B, N, H, dk, dv, G.GDN_BF16, device=device) for _ in range(L)]
            for _ in range(2)]
        self.cur = 0  # buffer set of the latest verification
        self.pending = None  # (parents, last) of a verified step not yet committed
        # per-sequence status words: the draft's topology check (verify), the
        # previous path's state commit and its history commit (delayed or not)
        self.status = torch.zeros(B, dtype=torch.int32, device=device)
        self.commit_status = torch.zeros(B, dtype=torch.int32, device=device)
        self.hist_status = torch.zeros(B, dtype=torch.int32, device=device)
        # autoregressive step buffers (one token per sequence)
        self.x1 = e(B, D)
        self.x1b = e(B, D, dt=bf)
        self.P1 = e(B, 1, shape.n_proj)
        self.q1 = e(B, 1, H, dk, dt=bf)
        self.k1 = e(B, 1, H, dk, dt=bf)
        self.v1 = e(B, 1, H, dv, dt=bf)
        self.beta1 = e(B, 1, H)
        self.g1 = e(B, 1, H)
        self.out1 = e(B, H, dv)
        self.Y1 = e(B, H * dv, dt=bf)
        self.root1 = torch.full((B, 1), -1, dtype=torch.int32, device=device)
        self.zero1 = torch.zeros(B, dtype=torch.int32, device=device)

    # ------------------------------------------------------------------ setup
    def load_layer(self, layer: int, w_in_bits, conv_w, w_o_bits, S0=None):
        """Weights as bf16 bits: w_in [n_in][D] (q^ k^ v^ gate rows, then alpha
        and beta rows), w_o [D][H*dv]; conv_w FP32 [n_conv][4]."""
        npj = self.shape.n_proj
        G.gdn_pack_weights(_bf16(w_in_bits[:npj], self.device), self.W_in[layer])
        self.W_ab[layer].copy_(_bf16(w_in_bits[npj:], self.device))
        G.gdn_pack_weights(_bf16(w_o_bits, self.device), self.W_o[layer])
        self.conv_w[layer].copy_(_f32(conv_w, self.device))
        if S0 is not None:
            self.S[layer].copy_(_f32(S0, self.device))

    @property
    def hist(self) -> torch.Tensor:
        """The committed convolution histories [L][B][3][n_conv]."""
        return self.hists[self.hc]

    @property
    def gate_cols(self):
        sh = self.shape
        return sh.n_conv, sh.n_conv + sh.H * sh.dv

    # ------------------------------------------------------- speculative step
    def set_inputs(self, x: torch.Tensor, x_bf16: torch.Tensor):
        """Layer-0 input rows [B*N][D]: the FP32 residual stream and its bf16
        projection input (the same values, bf16-representable)."""
        self.x.copy_(x)
        self.xb.copy_(x_bf16)

    def verify(self, parents: torch.Tensor, stream=None, layer_inputs=None, layer_outputs=None,
               prep_outputs=None, verify_inputs=None):
        """All layers, layer-major, for the draft tree `parents` [B][N]; the final
        hidden rows are left in self.x (FP32) and self.xb (bf16).  A step
        verified earlier and not yet committed (see step()) is committed first,
        fused into each layer's verification.

        Taps for checking the stack layer by layer (sequencing only):
        layer_inputs: optional per-layer pairs (FP32 [B*N][D], bf16 [B*N][D])
        copied into the hidden rows before each layer (each layer then runs on
        given inputs instead of the previous layer's output); layer_outputs:
        optional list that receives a copy of each layer's FP32 output rows;
        prep_outputs: optional list that receives copies of each layer's
        (q, k, v, beta, g) as the prep wrote them; verify_inputs: optional
        per-layer (q, k, v, beta, g) copied over the prep's before the layer's
        verification."""
        sh = self.shape
        g0, g1 = self.gate_cols
        M = self.B * self.N
        npj = sh.n_proj
        xb3 = self.xb.view(self.B, self.N, sh.D)
        prev, cur = self.cur, 1 - self.cur
        pend = self.pending
        hc = self.hc
        for l in range(sh.layers):
            if layer_inputs is not None:
                self.x.copy_(layer_inputs[l][0])
                self.xb.copy_(layer_inputs[l][1])
            P = self.P[cur, l]
            G.gdn_linear(self.xb, self.W_in[l], C=P.view(M, npj), w_layout=PK, stream=stream)
            if pend is None:
                G.gdn_layer_prep(P, xb3, self.W_ab[l], parents, self.conv_w[l], self.hists[hc, l],
                                 self.q, self.k, self.v, self.beta, self.g,
                                 gate_shift=self.gate_shift, stream=stream)
            else:  # the previous path enters this layer's history inside the prep
                G.gdn_layer_prep_delayed(P, xb3, self.W_ab[l], parents, self.conv_w[l],
                                         self.hists[hc, l], self.q, self.k, self.v, self.beta,
                                         self.g, self.P[prev, l], pend[0], pend[1],
                                         self.hists[1 - hc, l], gate_shift=self.gate_shift,
                                         dev_status=self.hist_status, stream=stream)
            vin = (self.q, self.k, self.v, self.beta, self.g)
            if prep_outputs is not None:
                prep_outputs.append(tuple(t.clone() for t in vin))
            if verify_inputs is not None:
                for dst, src in zip(vin, verify_inputs[l]):
                    dst.copy_(src)
            G.gdn_layer_verify(self.S[l], parents, self.q, self.k, self.v, self.beta, self.g,
                               P.view(M, npj)[:, g0:g1], self.Y, self.rec[cur][l],
                               prev_factors=None if pend is None else self.rec[prev][l],
                               last_accepted=None if pend is None else pend[1],
                               commit_status=None if pend is None else self.commit_status,
                               dev_status=self.status, stream=stream)
            G.gdn_linear(self.Y, self.W_o[l], C=self.x, R=self.x, C_bf16=self.xb, w_layout=PK,
                         stream=stream)
            if layer_outputs is not None:
                layer_outputs.append(self.x.clone())
        self.cur = cur
        if pend is not None:
            self.hc = 1 - hc
        self.pending = None

    def commit(self, parents: torch.Tensor, last: torch.Tensor, stream=None):
        """Apply the accepted path of the latest verification (deepest node `last`
        [B], -1 = none) in every layer now."""
        cur = self.cur
        for l in range(self.shape.layers):
            G.gdn_commit_path(self.S[l], self.rec[cur][l], last, dev_status=self.commit_status,
                              stream=stream)
            G.gdn_conv_commit(self.P[cur, l], parents, last, self.hist[l],
                              dev_status=self.hist_status, stream=stream)

    def check_status(self):
        """Raise if the latest verification rejected a draft's topology or a
        commit (state or history) rejected its accepted node (waits for the
        stream)."""
        for name, st in (("draft topology", self.status), ("state commit", self.commit_status),
                         ("history commit", self.hist_status)):
            bad = [int(x) for x in st.cpu()]
            if any(x != G.GDN_OK for x in bad):
                raise G.GdnError(G.GDN_ERR_TOPOLOGY, f"{name} status per sequence: {bad}")

    def defer_commit(self, parents: torch.Tensor, last: torch.Tensor):
        """Leave the latest verification's accepted path to the next verify()."""
        self.pending = (parents, last)

    def step(self, parents: torch.Tensor, last_prev=None, parents_prev=None, stream=None,
             **taps):
        """One speculative step with the delayed commit: the previous step's
        accepted node (last_prev, on its tree parents_prev) is committed inside
        this step's verification."""
        if last_prev is not None:
            self.defer_commit(parents_prev, last_prev)
        self.verify(parents, stream=stream, **taps)

    def flush(self, parents: torch.Tensor, last: torch.Tensor, stream=None):
        """Commit the latest verification's accepted path (end of a run)."""
        self.commit(parents, last, stream=stream)

    # ------------------------------------------------ autoregressive baseline
    def ar_step(self, x: torch.Tensor, x_bf16: torch.Tensor, stream=None):
        """One token per sequence ([B][D], FP32 and its bf16 copy) through every
        layer, committing state and history as it goes; the output rows are
        left in self.x1."""
        sh = self.shape
        g0, g1 = self.gate_cols
        B = self.B
        self.x1.copy_(x)
        self.x1b.copy_(x_bf16)
        npj = sh.n_proj
        xb3 = self.x1b.view(B, 1, sh.D)
        for l in range(sh.layers):
            P1 = self.P1
            G.gdn_linear(self.x1b, self.W_in[l], C=P1.view(B, npj), w_layout=PK, stream=stream)
            G.gdn_layer_prep(P1, xb3, self.W_ab[l], self.root1, self.conv_w[l],
                             self.hist[l], self.q1, self.k1, self.v1, self.beta1, self.g1,
                             gate_shift=self.gate_shift, stream=stream)
            G.gdn_conv_commit(P1, self.root1, self.zero1, self.hist[l], stream=stream)
            G.gdn_decode_step(self.S[l], self.q1.view(B, sh.H, sh.dk), self.k1.view(B, sh.H, sh.dk),
                              self.v1.view(B, sh.H, sh.dv), self.beta1.view(B, sh.H),
                              self.g1.view(B, sh.H), self.out1, stream=stream)
            G.gdn_gate_merge(self.out1.view(B, sh.H * sh.dv), P1.view(B, npj)[:, g0:g1],
                             self.Y1, stream=stream)
            G.gdn_linear(self.Y1, self.W_o[l], C=self.x1, R=self.x1, C_bf16=self.x1b,
                         w_layout=PK, stream=stream)
