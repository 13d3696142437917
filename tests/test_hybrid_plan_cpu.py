"""Host-side checks of the hybrid verifier's plan (gdn_hybrid_plan): the
chains partition the nodes, each chain follows first-child links from its
head, and every chain's level exceeds the level of the chain holding its
head's parent (so one launch per level respects every dependency)."""

import numpy as np
import pytest

from linear_attention_gdn_amd import gdnspec as G
from linear_attention_gdn_amd import workloads as W


def _chains(plan, b):
    pl = plan.plan_host.reshape(plan.N, plan.B, plan.N, 2)
    return [[int(h) for h in pl[l, b, :, 0] if h >= 0] for l in range(plan.levels)]


def _ends(plan, b):
    pl = plan.plan_host.reshape(plan.N, plan.B, plan.N, 2)
    return [[int(e) for h, e in pl[l, b] if h >= 0] for l in range(plan.levels)]


@pytest.mark.parametrize("topo", ["chain", "spine", "branching", "random", "window", "binary"])
def test_plan_partitions_nodes_into_dependency_ordered_chains(topo):
    rng = np.random.default_rng(7)
    N, B = 40, 5
    make = {"chain": lambda: W.chain_parents(N), "spine": lambda: W.spine_tree_parents(N, rng),
            "branching": lambda: W.branching_tree_parents(N, rng),
            "random": lambda: W.random_parents(N, rng),
            "window": lambda: W.window_tree_parents(N, rng),
            "binary": lambda: W.binary_tree_parents(N)}[topo]
    par = np.stack([make() for _ in range(B)]).astype(np.int32)
    plan = G.HybridPlan(par, device="cpu")
    for l in range(plan.levels):
        assert plan.chains_per_level[l] == max(len(_chains(plan, b)[l]) for b in range(B))
    assert not plan.chains_per_level[plan.levels:].any()
    for b in range(B):
        p = par[b]
        first = {}
        for t in range(N - 1, -1, -1):
            if p[t] >= 0:
                first[int(p[t])] = t
        level_of = np.full(N, -1)
        seen = np.zeros(N, int)
        for l, (heads, ends) in enumerate(zip(_chains(plan, b), _ends(plan, b))):
            for h, e in zip(heads, ends):
                assert p[h] < 0 or first[int(p[h])] != h  # a head is no first child
                if p[h] >= 0:
                    assert 0 <= level_of[p[h]] < l  # its parent's chain ran earlier
                t = h
                while t >= 0:
                    seen[t] += 1
                    level_of[t] = l
                    last = t
                    t = first.get(t, -1)
                assert e == last  # the plan's last node of the chain
        assert (seen == 1).all()  # every node in exactly one chain
    if topo == "chain":
        assert plan.levels == 1 and plan.chains_per_level[0] == 1


def test_plan_rejects_bad_topology():
    par = np.array([[-1, 0, 3, 1]], np.int32)
    with pytest.raises(G.GdnError) as e:
        G.HybridPlan(par, device="cpu")
    assert e.value.status == G.GDN_ERR_TOPOLOGY
    assert G.lib().gdn_hybrid_plan_entries(0, 4) == 0
    assert G.lib().gdn_hybrid_plan_entries(2, 65) == 0
