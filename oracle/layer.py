"""CPU oracle for the GDN layer scaffold around the verifier (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline may
use this module.  float64 NumPy; shares no code with the GPU library.

The Pith review of SpecLA (verdict page, "skeptic critique"; review page,
Referee Report major comment 1; both citing the paper's Section 7) gives
the target layer as GDN with h_v = 8, d_k = d_v = 256, a depthwise causal
convolution of width 4 and an output gate through SiLU.
The rest of the layer follows the plainest GDN reading:

  P        = x W_in^T                        (x: [N][D]; W_in: [C_in][D])
             columns: q^ | k^ | v^ | gate (H*d each) | alpha logit (H) | beta logit (H)
  c_t      = sum_{i=0..3} w[:, i] * P_conv(a_i(t))    depthwise, per channel,
             a_0 = t, a_1 = parent, ... along the root path; past the root the
             committed history supplies the previous pre-conv inputs
  q, k, v  = SiLU(c) split per head; q and k L2-normalised per head
  beta     = sigmoid(beta logit);  g = -softplus(alpha logit + gate_shift)
  o        = GDN verify (oracle.oracle.tree_verify)
  y        = (o * SiLU(gate)) W_o^T;  x_next = x + y

The committed conv history holds the 3 most recent pre-conv inputs of the
accepted path, most recent first; a commit of the root path p_1..p_n shifts
in P_conv(p_n), ..., P_conv(p_1) ahead of the old history.

Precision: the workload fixes bf16 for the projections and for q, k, v.  With
``bf16=True`` the layer rounds to bf16 exactly there (the input of each
projection, and q, k, v after normalisation) and computes everything else in
float64; with ``bf16=False`` nothing is rounded (the pure algebra, used by
the exactness pins).
"""

from __future__ import annotations

import numpy as np

CONV_TAPS = 4


def silu(x):
    return x / (1.0 + np.exp(-x))


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    return np.logaddexp(0.0, x)


def round_bf16(x):
    """Nearest bfloat16 value (8 significant bits, ties to even), from float64.

    x = m 2^e with 1/2 <= |m| < 1; keeping 8 bits means rounding m 2^8 to an
    integer (np.rint rounds halves to even).  Finite, normal-range inputs."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


def root_path(parents, t):
    out = []
    while t >= 0:
        out.append(int(t))
        t = int(parents[t])
    return out[::-1]


def conv_inputs(Pc, parents, hist, t):
    """The CONV_TAPS pre-conv inputs seen by node t, current first: [taps][C]."""
    path = root_path(parents, t)[::-1]  # t, parent, grandparent, ...
    rows = [Pc[j] for j in path[:CONV_TAPS]]
    i = 0
    while len(rows) < CONV_TAPS:
        rows.append(hist[i])
        i += 1
    return np.stack(rows)


def tree_conv(Pc, parents, conv_w, hist):
    """Causal depthwise conv along root paths.  Pc [N][C], conv_w [C][taps]
    (tap 0 multiplies the current input), hist [taps-1][C] most recent first."""
    Pc = np.asarray(Pc, np.float64)
    N, C = Pc.shape
    out = np.zeros((N, C))
    for t in range(N):
        X = conv_inputs(Pc, parents, np.asarray(hist, np.float64), t)
        out[t] = np.sum(np.asarray(conv_w, np.float64).T * X, axis=0)
    return out


def layer_prep(P, parents, conv_w, hist, H, dk, dv, gate_shift=2.0):
    """q, k, v [N][H][d], beta, g [N][H] and the gate pre-activation [N][H*dv]."""
    P = np.asarray(P, np.float64)
    N = P.shape[0]
    cq, ck, cv = H * dk, H * dk, H * dv
    nconv = cq + ck + cv
    c = silu(tree_conv(P[:, :nconv], parents, conv_w, hist))
    q = c[:, :cq].reshape(N, H, dk)
    k = c[:, cq:cq + ck].reshape(N, H, dk)
    v = c[:, cq + ck:nconv].reshape(N, H, dv)
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    gate = P[:, nconv:nconv + H * dv]
    a_logit = P[:, nconv + H * dv:nconv + H * dv + H]
    b_logit = P[:, nconv + H * dv + H:nconv + H * dv + 2 * H]
    beta = sigmoid(b_logit)
    g = -softplus(a_logit + gate_shift)
    return q, k, v, beta, g, gate


def gate_merge(o, gate):
    """o [N][H][dv] times SiLU(gate) [N][H*dv] -> [N][H*dv]."""
    o = np.asarray(o, np.float64)
    N = o.shape[0]
    return o.reshape(N, -1) * silu(np.asarray(gate, np.float64))


def linear(x, W, resid=None):
    """x [M][K] times W^T (W [Nc][K]) (+ resid)."""
    y = np.asarray(x, np.float64) @ np.asarray(W, np.float64).T
    if resid is not None:
        y = y + np.asarray(resid, np.float64)
    return y


def commit_history(Pc, parents, hist, last):
    """New conv history after accepting the root path of node `last` (-1: none)."""
    hist = np.asarray(hist, np.float64)
    if last < 0:
        return hist.copy()
    path = root_path(parents, last)[::-1]  # most recent first
    rows = [np.asarray(Pc[j], np.float64) for j in path] + list(hist)
    return np.stack(rows[:CONV_TAPS - 1])


# --------------------------------------------------------------------------
# a stack of layers
# --------------------------------------------------------------------------


class StackWeights:
    """Per-layer weights: W_in [C_in][D], conv_w [3*H*d][taps], W_o [D][H*dv]."""

    def __init__(self, W_in, conv_w, W_o, H, dk, dv, gate_shift=2.0, bf16=False):
        self.W_in, self.conv_w, self.W_o = W_in, conv_w, W_o
        self.H, self.dk, self.dv, self.gate_shift = H, dk, dv, gate_shift
        self.bf16 = bf16

    @property
    def layers(self):
        return len(self.W_in)


def layer_forward(wt, layer, x, parents, S0, hist):
    """One layer on a draft tree (one sequence).  x [N][D]; S0 [H][dv][dk];
    hist [taps-1][3*H*d].  Returns (x_next, o, P, record) where record holds
    what the commit needs (the verify's u' and G plus k, v, beta, g)."""
    from oracle import oracle as O
    H, dk, dv = wt.H, wt.dk, wt.dv
    rnd = round_bf16 if wt.bf16 else (lambda a: a)
    P = linear(rnd(x), wt.W_in[layer])
    q, k, v, beta, g, gate = layer_prep(P, parents, wt.conv_w[layer], hist, H, dk, dv,
                                        wt.gate_shift)
    q, k, v = rnd(q), rnd(k), rnd(v)
    par = np.asarray(parents, np.int32)[None, :]
    o, up, G = O.tree_verify(np.asarray(S0)[None], par, q[None], k[None], v[None], beta[None],
                             g[None])
    y = linear(rnd(gate_merge(o[0], gate)), wt.W_o[layer], resid=x)
    return y, o[0], P, dict(k=k, v=v, beta=beta, g=g)


def layer_commit(wt, P, parents, S0, hist, rec, last):
    """Committed state and conv history of one layer after accepting `last`."""
    from oracle import oracle as O
    nconv = wt.H * (2 * wt.dk + wt.dv)
    par = np.asarray(parents, np.int32)[None, :]
    Snew, _, _ = O.commit(np.asarray(S0)[None], par, rec["k"][None], rec["v"][None],
                          rec["beta"][None], rec["g"][None], np.array([last], np.int32))
    return Snew[0], commit_history(np.asarray(P)[:, :nconv], parents, hist, last)


def stack_spec_step(wt, x0, parents, states, hists):
    """All layers on a draft tree; returns final outputs and per-layer data."""
    x = np.asarray(x0, np.float64)
    per_layer = []
    for layer in range(wt.layers):
        x_next, o, P, rec = layer_forward(wt, layer, x, parents, states[layer], hists[layer])
        per_layer.append(dict(x_in=x, o=o, P=P, rec=rec))
        x = x_next
    return x, per_layer


def stack_commit(wt, parents, states, hists, per_layer, last):
    new_states, new_hists = [], []
    for layer in range(wt.layers):
        d = per_layer[layer]
        S, h = layer_commit(wt, d["P"], parents, states[layer], hists[layer], d["rec"], last)
        new_states.append(S)
        new_hists.append(h)
    return new_states, new_hists
