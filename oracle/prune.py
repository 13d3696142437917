"""CPU oracle of confidence-guided draft pruning (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may use this module; it shares no code with the GPU library.

The Pith review of SpecLA (review page, Figures, Figure 8 caption; Axiom &
Free-Parameter Ledger, "Tree margin tau_tree" and "Draft budget") describes the
pruning of a candidate draft tree before verification: nodes whose confidence
lies within tau_tree of the best confidence q* are kept, the monotonicity of
the confidence along root paths makes that window ancestor-closed, and the
budget T then truncates the selection.  Read plainly:

  q_t       the node's confidence (a path score that never increases from a
            node to its children, e.g. the cumulative log-probability)
  q*        the largest confidence among the candidates
  window    {t : q_t >= q* - tau}, the threshold formed in FP32 (the kernel's
            precision; the comparison then decides which integers survive)
  budget    the first T window nodes in the order (q descending, index
            ascending); a parent precedes its children in this order (its
            confidence is at least theirs and its index smaller), so the
            selection stays ancestor-closed
  output    the kept nodes in their original (topological) order, renumbered
            0..n-1, with parents mapped to the new numbers

Plain Python over one sequence at a time: obviously correct, slow.
"""

from __future__ import annotations

import numpy as np


def check_candidates(parents, conf):
    """True when parents are topological (-1 <= p[t] < t), no confidence is
    NaN, and confidences never increase from a parent to a child."""
    par = [int(p) for p in parents]
    q = [float(c) for c in np.asarray(conf, np.float32)]
    for t, p in enumerate(par):
        if p < -1 or p >= t or q[t] != q[t]:
            return False
        if p >= 0 and q[t] > q[p]:
            return False
    return True


def prune(parents, conf, tau, budget):
    """Kept node indices (ascending) and their parents in the new numbering,
    for one sequence; (None, None) when the candidates fail check_candidates."""
    if not check_candidates(parents, conf):
        return None, None
    q = np.asarray(conf, np.float32)
    par = [int(p) for p in parents]
    thr = np.float32(np.float32(q.max()) - np.float32(tau))  # FP32, as the kernel forms it
    window = [t for t in range(len(q)) if q[t] >= thr]
    window.sort(key=lambda t: (-float(q[t]), t))
    kept = sorted(window[:budget])
    new_of = {t: i for i, t in enumerate(kept)}
    new_par = [new_of[par[t]] if par[t] >= 0 else -1 for t in kept]
    return kept, new_par


def prune_batch(parents, conf, tau, budget):
    """prune() over [B][M] arrays: kept [B][T] and new parents [B][T] padded
    with -1, counts [B] (-1 for a sequence whose candidates are rejected)."""
    parents = np.asarray(parents)
    B = parents.shape[0]
    kept = np.full((B, budget), -1, np.int32)
    newp = np.full((B, budget), -1, np.int32)
    n = np.zeros(B, np.int32)
    for b in range(B):
        k, p = prune(parents[b], conf[b], tau, budget)
        if k is None:
            n[b] = -1
            continue
        n[b] = len(k)
        kept[b, :len(k)] = k
        newp[b, :len(p)] = p
    return kept, newp, n
