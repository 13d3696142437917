"""Seeded synthetic draft workloads for tree-masked Gated DeltaNet verification.

This module only draws inputs: committed states, per-node q/k/v, write
strengths beta, log-decays g, draft topologies and accepted paths.  It holds
none of the verifier's arithmetic, so the HIP path and the CPU oracle can both
consume exactly the same bits.

Source: "SpecLA: Efficient Speculative Decoding for Linear-Attention Models"
(pith.science review pages).  The layer shape (h_v = 8, d_k = d_v = 256, FP32
state) is the one the review quotes from the paper's Section 7; the draft
budget (16 nodes, top-k 4) is from the review's free-parameter ledger.  The
pages measure on GSM8K, HumanEval and a mixed suite; these synthetic trees and
acceptance lengths stand in for the drafter/target pair those runs used.

Conventions fixed here (the pages leave them open):
  * node 0 is the root (parent -1); parents are topological, -1 <= p[t] < t;
  * depth counts the nodes on the root-to-node path (root depth 1);
  * q and k are L2-normalised per (sequence, node, head) in float64, rounded to
    float32, then (for bf16 workloads) rounded once to bf16 with
    round-to-nearest-even; both sides use the rounded values;
  * beta = sigmoid(z), g = -softplus(z + shift) computed in float64 and rounded
    to float32; alpha = exp(g) is never materialised here;
  * the accepted path of a sequence is encoded as ``last_accepted[b]`` (the
    deepest accepted node, -1 for a zero-length commit).
"""

from __future__ import annotations

import dataclasses
from collections import deque
from typing import Optional

import numpy as np

# --------------------------------------------------------------------------
# bf16 bit handling (storage format only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    if np.any((u & 0x7F800000) == 0x7F800000):
        raise ValueError("non-finite value in bf16 conversion")
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# topologies
# --------------------------------------------------------------------------


def chain_parents(n: int) -> np.ndarray:
    """A linear draft chain: parent of node t is t-1."""
    return np.arange(-1, n - 1, dtype=np.int32)


def binary_tree_parents(n: int) -> np.ndarray:
    """Complete binary tree in BFS numbering, left child first: p[t] = (t-1)//2."""
    p = np.empty(n, dtype=np.int32)
    p[0] = -1
    for t in range(1, n):
        p[t] = (t - 1) // 2
    return p


def depths_of(parents: np.ndarray) -> np.ndarray:
    """Nodes on each root-to-node path (root = 1), for topologically numbered parents."""
    n = len(parents)
    d = np.zeros(n, dtype=np.int32)
    for t in range(n):
        p = int(parents[t])
        d[t] = 1 if p < 0 else d[p] + 1
    return d


def window_tree_parents(n: int, rng: np.random.Generator, window: int = 4,
                        max_depth: int = 8) -> np.ndarray:
    """Random tree: node i's parent is uniform over max(0, i-window)..i-1.

    Candidates whose depth already equals ``max_depth`` are skipped; if the whole
    window is at the cap, the parent is drawn uniformly among all earlier nodes
    below the cap (the root always qualifies).
    """
    p = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int32)
    depth[0] = 1
    for i in range(1, n):
        cand = [j for j in range(max(0, i - window), i) if depth[j] < max_depth]
        if not cand:
            cand = [j for j in range(i) if depth[j] < max_depth]
        j = int(cand[int(rng.integers(len(cand)))])
        p[i] = j
        depth[i] = depth[j] + 1
    return p


def branching_tree_parents(n: int, rng: np.random.Generator, branches=(1, 2, 3),
                           max_depth: int = 10) -> np.ndarray:
    """Random BFS-numbered tree with per-node branching factor drawn from ``branches``.

    Each dequeued node below ``max_depth`` receives min(b, n - count) children.
    If the queue empties before ``n`` nodes exist the whole tree is redrawn.
    """
    while True:
        p = [-1]
        depth = [1]
        q = deque([0])
        while q and len(p) < n:
            u = q.popleft()
            if depth[u] >= max_depth:
                continue
            b = int(branches[int(rng.integers(len(branches)))])
            for _ in range(min(b, n - len(p))):
                p.append(u)
                depth.append(depth[u] + 1)
                q.append(len(p) - 1)
        if len(p) == n:
            return np.asarray(p, dtype=np.int32)


def spine_tree_parents(n: int, rng: np.random.Generator, p_chain: float = 0.75,
                       window: int = 6) -> np.ndarray:
    """Deep, narrow tree: node t continues the chain (parent t - 1) with
    probability p_chain, else branches off one of the `window` nodes before
    t - 1; root paths run to about p_chain * n nodes."""
    p = np.full(n, -1, dtype=np.int32)
    for t in range(1, n):
        if t == 1 or rng.random() < p_chain:
            p[t] = t - 1
        else:
            p[t] = int(rng.integers(max(0, t - 1 - window), t - 1))
    return p


def random_parents(n: int, rng: np.random.Generator) -> np.ndarray:
    """Uniform random recursive tree: parent of node t uniform over 0..t-1."""
    p = np.full(n, -1, dtype=np.int32)
    for t in range(1, n):
        p[t] = int(rng.integers(t))
    return p


def root_path(parents: np.ndarray, t: int) -> list:
    """Root-first list of the nodes on the path to node t (t included)."""
    out = []
    while t >= 0:
        out.append(int(t))
        t = int(parents[t])
    return out[::-1]


def leaves_of(parents: np.ndarray) -> np.ndarray:
    n = len(parents)
    has_child = np.zeros(n, dtype=bool)
    for t in range(n):
        if parents[t] >= 0:
            has_child[parents[t]] = True
    return np.nonzero(~has_child)[0]


def geometric_length(rng: np.random.Generator, mean: float) -> int:
    """P(L = l) = p (1 - p)^(l - 1), l >= 1, with p = 1 / mean."""
    return int(rng.geometric(1.0 / mean))


def accept_leaf_geometric(parents: np.ndarray, rng: np.random.Generator, mean: float) -> int:
    """Deepest accepted node: a uniform leaf's root path cut to a geometric length."""
    leaves = leaves_of(parents)
    leaf = int(leaves[int(rng.integers(len(leaves)))])
    path = root_path(parents, leaf)
    L = min(geometric_length(rng, mean), len(path))
    return path[L - 1]


# --------------------------------------------------------------------------
# drafts
# --------------------------------------------------------------------------


@dataclasses.dataclass
class Draft:
    """One verification problem: B sequences, N nodes, H heads.

    Layouts (all C-contiguous):
      S0      float32 [B][H][dv][dk]  (state rows run along d_k)
      q, k    [B][N][H][dk]; v [B][N][H][dv]; uint16 bf16 bits or float32
      beta, g float32 [B][N][H]
      parents int32 [B][N]; last_accepted int32 [B]
    """

    B: int
    N: int
    H: int
    dk: int
    dv: int
    dtype: str  # "bf16" or "f32"
    S0: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    g: np.ndarray
    parents: np.ndarray
    last_accepted: np.ndarray
    scale: float = 1.0
    name: str = ""

    def _wide(self, x: np.ndarray) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(x).astype(np.float64)
        return np.asarray(x, dtype=np.float32).astype(np.float64)

    def q64(self):
        return self._wide(self.q)

    def k64(self):
        return self._wide(self.k)

    def v64(self):
        return self._wide(self.v)

    def replace(self, **kw) -> "Draft":
        return dataclasses.replace(self, **kw)


def _l2n(x: np.ndarray) -> np.ndarray:
    nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(nrm, 1e-30)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def draw_node_inputs(rng: np.random.Generator, B: int, N: int, H: int, dk: int, dv: int,
                     dtype: str, gate_shift: float):
    """q, k, v, beta, g for one draft (in that draw order)."""
    q = _l2n(rng.standard_normal((B, N, H, dk))).astype(np.float32)
    k = _l2n(rng.standard_normal((B, N, H, dk))).astype(np.float32)
    v = rng.standard_normal((B, N, H, dv)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, N, H))))).astype(np.float32)
    g = (-_softplus(rng.standard_normal((B, N, H)) + gate_shift)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return q, k, v, beta, g


def make_draft(B: int, N: int, H: int, dk: int, dv: int, *, topology: str = "chain",
               accept: str = "uniform", accept_mean: float = 3.0, dtype: str = "bf16",
               state_std: float = 0.02, gate_shift: float = 2.0, seed: int = 0,
               scale: float = 1.0, name: str = "",
               rng: Optional[np.random.Generator] = None) -> Draft:
    """Draw a draft in the fixed order S0, q, k, v, beta, g, topology, acceptance.

    topology: "chain" | "window" (parent in the previous 4 nodes, depth <= 8) |
              "branching" (branching factor in {1,2,3}, depth <= 10) | "random" |
              "spine" (long main chain with short side branches: deep drafts)
    accept:   "uniform" (length uniform in 0..N on a chain) |
              "leaf_geometric" (uniform leaf, path cut to geometric(accept_mean)) |
              "full" (deepest node N-1) | "none" (-1)
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    S0 = (state_std * rng.standard_normal((B, H, dv, dk))).astype(np.float32)
    q, k, v, beta, g = draw_node_inputs(rng, B, N, H, dk, dv, dtype, gate_shift)
    parents = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        if topology == "chain":
            parents[b] = chain_parents(N)
        elif topology == "window":
            parents[b] = window_tree_parents(N, rng)
        elif topology == "branching":
            parents[b] = branching_tree_parents(N, rng)
        elif topology == "random":
            parents[b] = random_parents(N, rng)
        elif topology == "binary":
            parents[b] = binary_tree_parents(N)
        elif topology == "spine":
            parents[b] = spine_tree_parents(N, rng)
        else:
            raise ValueError(topology)
    last = np.empty(B, dtype=np.int32)
    for b in range(B):
        if accept == "uniform":
            if topology != "chain":
                raise ValueError("uniform acceptance length is defined on chains")
            last[b] = int(rng.integers(0, N + 1)) - 1
        elif accept == "leaf_geometric":
            last[b] = accept_leaf_geometric(parents[b], rng, accept_mean)
        elif accept == "full":
            last[b] = N - 1
        elif accept == "none":
            last[b] = -1
        else:
            raise ValueError(accept)
    return Draft(B, N, H, dk, dv, dtype, S0, q, k, v, beta, g, parents, last, scale, name)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------


def tiny_case(seed: int = 0):
    """1 head, d = 16, FP32 throughout: a 4-node chain and a 7-node binary tree.

    Both drafts start from the same S0 ~ N(0, 0.1^2).  alpha = exp(-softplus(z)).
    The tree's accepted path is root -> left -> left, i.e. nodes (0, 1, 3).
    Returns (chain_draft, tree_draft).
    """
    rng = np.random.default_rng(seed)
    d = 16
    S0 = (0.1 * rng.standard_normal((1, 1, d, d))).astype(np.float32)
    out = []
    for n, parents, last in ((4, chain_parents(4), 3), (7, binary_tree_parents(7), 3)):
        q, k, v, beta, g = draw_node_inputs(rng, 1, n, 1, d, d, "f32", 0.0)
        out.append(Draft(1, n, 1, d, d, "f32", S0, q, k, v, beta, g, parents[None, :].copy(),
                         np.array([last], dtype=np.int32), 1.0,
                         "tiny-chain4" if n == 4 else "tiny-binary7"))
    return tuple(out)


def chain8_layer(seed: int = 0) -> Draft:
    """One GDN layer (H=8, d=256, FP32 state, bf16 q/k/v), B=1, an 8-node chain."""
    return make_draft(1, 8, 8, 256, 256, topology="chain", accept="uniform", seed=seed,
                      name="chain8-b1-h8-d256")


def tree32_layer(seed: int = 0) -> Draft:
    """Same layer, B=1, a 32-node window tree (depth <= 8), geometric(3) acceptance."""
    return make_draft(1, 32, 8, 256, 256, topology="window", accept="leaf_geometric",
                      accept_mean=3.0, seed=seed, name="tree32-b1-h8-d256")


def tree64_batch8(seed: int = 0) -> Draft:
    """Same layer, B=8 sequences each with its own S0 and 64-node branching tree."""
    return make_draft(8, 64, 8, 256, 256, topology="branching", accept="leaf_geometric",
                      accept_mean=4.0, seed=seed, name="tree64-b8-h8-d256")


def chain64_layer(seed: int = 0) -> Draft:
    """Deep-draft case: the same layer, B=1, a 64-node chain (root paths up to
    64 nodes), geometric(4) acceptance along it."""
    return make_draft(1, 64, 8, 256, 256, topology="chain", accept="leaf_geometric",
                      accept_mean=4.0, seed=seed, name="chain64-b1-h8-d256")


def spine64_batch8(seed: int = 0) -> Draft:
    """Deep-draft case: B=8 sequences, each a 64-node spine tree (a long main
    chain with short side branches, root paths of 25-35 nodes)."""
    return make_draft(8, 64, 8, 256, 256, topology="spine", accept="leaf_geometric",
                      accept_mean=4.0, seed=seed, name="spine64-b8-h8-d256")


WORKLOADS = {
    "chain8-b1-h8-d256": chain8_layer,
    "tree32-b1-h8-d256": tree32_layer,
    "tree64-b8-h8-d256": tree64_batch8,
    # deep drafts (paths past 16 nodes): timing cases for the blocked solve
    # and the chain-decomposed verifier, not configurations of the metric
    "chain64-b1-h8-d256": chain64_layer,
    "spine64-b8-h8-d256": spine64_batch8,
}


# --------------------------------------------------------------------------
# candidate trees with confidences, for draft pruning
# --------------------------------------------------------------------------


def candidate_tree(rng: np.random.Generator, top_k: int = 4, depth: int = 4,
                   logit_std: float = 2.0):
    """A synthetic drafter's candidate tree: every node above `depth` expands
    its top_k continuations (BFS numbering, so parents precede children).  The
    edge probabilities of one node's children are a softmax of N(0,
    logit_std^2) logits over top_k draws (the top_k of a longer vocabulary are
    stood in for by the draws themselves); a node's confidence is the
    cumulative log-probability of its root path (root 0), so it never
    increases from a node to its children.  Returns parents int32 [M] and
    confidences float32 [M]."""
    parents, conf, level = [-1], [0.0], [0]
    i = 0
    while i < len(parents):
        if level[i] < depth:
            z = rng.standard_normal(top_k) * logit_std
            logp = z - np.logaddexp.reduce(z)
            for j in np.argsort(-logp):  # most likely continuation first
                parents.append(i)
                conf.append(conf[i] + float(logp[j]))
                level.append(level[i] + 1)
        i += 1
    return np.asarray(parents, np.int32), np.asarray(conf, np.float32)


def candidate_batch(B: int, seed: int = 0, **kw):
    """B candidate trees of the same shape: parents [B][M], conf [B][M]."""
    rng = np.random.default_rng(seed)
    trees = [candidate_tree(rng, **kw) for _ in range(B)]
    return np.stack([t[0] for t in trees]), np.stack([t[1] for t in trees])


# --------------------------------------------------------------------------
# the decode loop over a stack of GDN layers
# --------------------------------------------------------------------------


@dataclasses.dataclass
class StackShape:
    """Sizes of a stack of GDN layers with hidden width D and H heads."""

    layers: int
    D: int = 2048
    H: int = 8
    dk: int = 256
    dv: int = 256

    @property
    def n_conv(self) -> int:  # channels of the depthwise convolution (q^, k^, v^)
        return self.H * (2 * self.dk + self.dv)

    @property
    def n_proj(self) -> int:  # input projection columns q^ k^ v^ gate
        return 2 * self.H * (self.dk + self.dv)

    @property
    def n_in(self) -> int:  # all input projection rows: q^ k^ v^ gate, then alpha, beta
        return self.n_proj + 2 * self.H


def stack_layer_weights(shape: StackShape, rng: np.random.Generator):
    """One layer's weights: W_in bf16 bits [n_in][D] ~ N(0, 1/D), conv_w f32
    [n_conv][4] ~ N(0, 1/4), W_o bf16 bits [D][H*dv] ~ N(0, 1/(H*dv))."""
    D, Hv = shape.D, shape.H * shape.dv
    w_in = rng.standard_normal((shape.n_in, D), dtype=np.float32) * np.float32(D ** -0.5)
    conv = (0.5 * rng.standard_normal((shape.n_conv, 4))).astype(np.float32)
    w_o = rng.standard_normal((D, Hv), dtype=np.float32) * np.float32(Hv ** -0.5)
    return f32_to_bf16_bits(w_in), conv, f32_to_bf16_bits(w_o)


def stack_states(shape: StackShape, B: int, rng: np.random.Generator, state_std: float = 0.02):
    """Per-layer FP32 states [layers][B][H][dv][dk] ~ N(0, state_std^2)."""
    S = rng.standard_normal((shape.layers, B, shape.H, shape.dv, shape.dk), dtype=np.float32)
    return S * np.float32(state_std)


def stack_inputs(rng: np.random.Generator, rows: int, D: int) -> np.ndarray:
    """Layer-0 inputs: bf16 bits [rows][D] of N(0, 1) values (no vocabulary)."""
    return f32_to_bf16_bits(rng.standard_normal((rows, D), dtype=np.float32))


def stack_drafts(rng: np.random.Generator, steps: int, N: int = 32, accept_mean: float = 3.0):
    """Per step a window tree (parent among the previous 4 nodes, depth <= 8)
    and the deepest accepted node: a uniform leaf's path cut to a
    geometric(accept_mean) length.  Returns parents [steps][N], last [steps]."""
    parents = np.empty((steps, N), np.int32)
    last = np.empty(steps, np.int32)
    for s in range(steps):
        parents[s] = window_tree_parents(N, rng)
        last[s] = accept_leaf_geometric(parents[s], rng, accept_mean)
    return parents, last


# The decode loop over 24 layers: hidden 2048, h=8, d=256, 32-node window
# trees, geometric(3) acceptance, compared with one-token decoding.
STACK_WORKLOADS = {
    "decode24-b1-h8-d256": dict(layers=24, D=2048, H=8, dk=256, dv=256, N=32, accept_mean=3.0),
}

