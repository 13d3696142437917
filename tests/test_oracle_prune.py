"""Pins for the pruning oracle (oracle/prune.py): a worked example by hand,
the defining properties (window, budget order, ancestor closure) checked by
brute force, and the rejection of candidates that break the preconditions."""

import itertools

import numpy as np
import pytest

from linear_attention_gdn_amd import workloads as W
from oracle import prune as PR

# A 7-node candidate tree (BFS numbering) with log-confidences:
#        0 (0.0)
#       /        \
#    1 (-0.5)   2 (-1.0)
#    /   \          \
#  3(-0.7) 4(-2.0)  5(-1.0)
#   |
#  6 (-3.0)
PAR = np.array([-1, 0, 0, 1, 1, 2, 3], np.int32)
CONF = np.array([0.0, -0.5, -1.0, -0.7, -2.0, -1.0, -3.0], np.float32)


def test_worked_example():
    # tau = 1.5: window = {q >= -1.5} = {0, 1, 2, 3, 5}; order by (-q, index):
    # 0, 1, 3, 2, 5 (2 and 5 tie at -1.0; 2 first)
    kept, newp = PR.prune(PAR, CONF, 1.5, 16)
    assert kept == [0, 1, 2, 3, 5] and newp == [-1, 0, 0, 1, 2]
    # budget 4 cuts node 5 (the later of the tied pair)
    kept, newp = PR.prune(PAR, CONF, 1.5, 4)
    assert kept == [0, 1, 2, 3] and newp == [-1, 0, 0, 1]
    # budget 3: 0, 1, 3 (node 3 outranks node 2)
    kept, newp = PR.prune(PAR, CONF, 1.5, 3)
    assert kept == [0, 1, 3] and newp == [-1, 0, 1]
    # tau = 0: only the best node; tau = 10: everything up to the budget
    assert PR.prune(PAR, CONF, 0.0, 16) == ([0], [-1])
    assert PR.prune(PAR, CONF, 10.0, 16)[0] == list(range(7))


def _is_valid_selection(par, q, tau, T, kept):
    """The definition, checked without sorting: every kept node is in the
    window, every kept node ranks before every window node left out, the count
    is min(T, |window|), and the kept set is ancestor-closed."""
    thr = np.float32(np.float32(q.max()) - np.float32(tau))
    window = {t for t in range(len(q)) if q[t] >= thr}
    ks = set(kept)
    if not ks <= window or len(ks) != min(T, len(window)):
        return False
    for k_, w in itertools.product(ks, window - ks):
        if (q[w], -w) > (q[k_], -k_):
            return False
    return all(par[t] < 0 or par[t] in ks for t in ks)


@pytest.mark.parametrize("seed", range(6))
def test_selection_meets_the_definition(seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        par, q = W.candidate_tree(rng, top_k=int(rng.integers(1, 5)),
                                  depth=int(rng.integers(1, 5)))
        # ties on purpose: round confidences to a coarse grid
        if rng.random() < 0.5:
            q = (np.round(q * 2) / 2).astype(np.float32)
        tau = float(rng.uniform(0, 6))
        T = int(rng.integers(1, 20))
        kept, newp = PR.prune(par, q, tau, T)
        assert _is_valid_selection(par, q, tau, T, kept)
        assert kept == sorted(kept)
        for i, t in enumerate(kept):  # parents renumbered
            assert (newp[i] == -1) == (par[t] == -1)
            if par[t] >= 0:
                assert kept[newp[i]] == par[t]


def test_brute_force_on_tiny_trees():
    """All ancestor-closed subsets of a 6-node tree: the oracle's choice is the
    unique one of the right size whose worst member outranks every member of
    the window left out."""
    par = np.array([-1, 0, 0, 1, 1, 2], np.int32)
    rng = np.random.default_rng(3)
    for _ in range(30):
        logp = -rng.exponential(1.0, size=6)
        logp[0] = 0.0
        q = np.zeros(6)
        for t in range(1, 6):
            q[t] = q[par[t]] + logp[t]
        q = q.astype(np.float32)
        tau, T = float(rng.uniform(0, 3)), int(rng.integers(1, 7))
        kept, _ = PR.prune(par, q, tau, T)
        good = [set(S) for r in range(7) for S in itertools.combinations(range(6), r)
                if _is_valid_selection(par, q, tau, T, S)]
        assert good == [set(kept)]


def test_fp32_threshold():
    """q* - tau is formed in FP32: a node exactly at the FP32 threshold is kept
    even where the float64 difference would exclude it."""
    par = np.array([-1, 0], np.int32)
    qstar, tau = np.float32(-2.877079486846924), np.float32(0.06611054390668869)
    thr32 = np.float32(qstar - tau)  # rounds below the exact difference
    conf = np.array([qstar, thr32], np.float32)
    assert float(thr32) < float(qstar) - float(tau)
    kept, _ = PR.prune(par, conf, float(tau), 4)
    assert kept == [0, 1]


def test_rejects_broken_preconditions():
    assert PR.prune([-1, 0, 3, 1], [0, -1, -1, -1], 1.0, 4) == (None, None)   # not topological
    assert PR.prune([-1, 0, 1], [0.0, -1.0, -0.5], 1.0, 4) == (None, None)    # child above parent
    assert PR.prune([-1, 0], [0.0, float("nan")], 1.0, 4) == (None, None)     # NaN
    kept, newp, n = PR.prune_batch(np.array([[-1, 0, 1], [-1, 0, 1]]),
                                   np.array([[0, -1, -2], [0, -1, 0.5]], np.float32), 5.0, 2)
    assert n.tolist() == [2, -1] and kept[0].tolist() == [0, 1] and kept[1].tolist() == [-1, -1]


def test_candidate_tree_confidences_are_monotone():
    rng = np.random.default_rng(0)
    par, q = W.candidate_tree(rng, top_k=4, depth=4)
    assert len(par) == 1 + 4 + 16 + 64 + 256
    assert PR.check_candidates(par, q)
