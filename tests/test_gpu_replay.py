"""GPU parity of the replay baselines (include/gdnnext.h) against the oracle:
root-to-leaf replay gives every node's output (each written once, by the
first path that holds it), token replay gives the committed state."""

import sys

import numpy as np
import pytest
import torch

from _gpu import TOL_OUT, TOL_STATE, dev_tensors, out_err, slice_rel_err, to_np
from linear_attention_gdn_amd import gdnspec as G
from linear_attention_gdn_amd import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _leaf_ends(parents):
    """[B][P] leaves of every sequence, padded with -1 (P = most leaves)."""
    leaves = [W.leaves_of(p) for p in parents]
    P = max(len(l) for l in leaves)
    ends = np.full((len(parents), P), -1, np.int32)
    for b, l in enumerate(leaves):
        ends[b, :len(l)] = l
    return ends


CASES = [("tiny binary tree", lambda: W.tiny_case(0)[1]),
         ("tiny chain", lambda: W.tiny_case(0)[0]),
         ("tree32", lambda: W.tree32_layer(1)),
         ("tree64 batch 8", lambda: W.tree64_batch8(0)),
         ("ragged random", lambda: W.make_draft(3, 37, 3, 72, 52, topology="random",
                                                accept="leaf_geometric", seed=5)),
         ("deep chain 64 fp32", lambda: W.make_draft(1, 64, 2, 64, 32, topology="chain",
                                                     accept="full", dtype="f32", seed=6))]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_replay_verify_matches_oracle(name, make):
    d = make()
    _say(f"replay verify: {name} B={d.B} N={d.N} H={d.H} dk={d.dk} dv={d.dv} {d.dtype}")
    t = dev_tensors(d)
    ends = torch.from_numpy(_leaf_ends(d.parents)).cuda()
    out = torch.full((d.B, d.N, d.H, d.dv), float("nan"), device="cuda")
    st = torch.full((d.B,), 77, dtype=torch.int32, device="cuda")
    S_before = t["S0"].clone()
    G.gdn_replay_verify(t["S0"], t["parents"], t["q"], t["k"], t["v"], t["beta"], t["g"], ends,
                        out, scale=d.scale, dev_status=st)
    torch.cuda.synchronize()
    assert torch.equal(t["S0"], S_before)  # read only
    assert np.all(to_np(st) == G.GDN_OK)
    ref_out, _, _ = O.draft_verify(d)
    e = out_err(out, ref_out)
    _say(f"  outputs max rel err {e:.2e}")
    assert e <= TOL_OUT


def test_replay_verify_every_node_as_an_end_agrees_bitwise():
    """Ends = all nodes (many paths share prefixes, so every node is written
    by several slots): the outputs equal those of the leaf ends bitwise, since
    each slot replays a node's root path in the same order."""
    d = W.tree32_layer(2)
    t = dev_tensors(d)
    outs = []
    for ends_np in (_leaf_ends(d.parents), np.arange(d.N, dtype=np.int32)[None, :]):
        out = torch.full((d.B, d.N, d.H, d.dv), float("nan"), device="cuda")
        G.gdn_replay_verify(t["S0"], t["parents"], t["q"], t["k"], t["v"], t["beta"], t["g"],
                            torch.from_numpy(ends_np).cuda(), out, scale=d.scale)
        outs.append(out)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[1]).any()
    ref_out, _, _ = O.draft_verify(d)
    assert out_err(outs[1], ref_out) <= TOL_OUT
    assert torch.equal(outs[0], outs[1])  # the same recurrence along the same path


def test_replay_verify_rejects_bad_topology_and_ends():
    d = W.make_draft(3, 12, 2, 64, 32, topology="random", accept="leaf_geometric", seed=9)
    t = dev_tensors(d)
    par = d.parents.copy()
    par[1, 5] = 7  # not topological: sequence 1 is not replayed
    ends = _leaf_ends(d.parents)
    ends[2, 0] = d.N  # out of range: that slot is skipped, reported
    out = torch.full((d.B, d.N, d.H, d.dv), float("nan"), device="cuda")
    st = torch.full((d.B,), 77, dtype=torch.int32, device="cuda")
    G.gdn_replay_verify(t["S0"], torch.from_numpy(par).cuda(), t["q"], t["k"], t["v"], t["beta"],
                        t["g"], torch.from_numpy(ends).cuda(), out, scale=d.scale, dev_status=st)
    torch.cuda.synchronize()
    assert to_np(st).tolist() == [G.GDN_OK, G.GDN_ERR_TOPOLOGY, G.GDN_ERR_TOPOLOGY]
    assert torch.isnan(out[1]).all()
    ref_out, _, _ = O.draft_verify(d)
    assert slice_rel_err(to_np(out[:1]).transpose(0, 2, 1, 3),
                         ref_out[:1].transpose(0, 2, 1, 3)) <= TOL_OUT


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_replay_commit_matches_oracle(name, make):
    d = make()
    _say(f"replay commit: {name}")
    t = dev_tensors(d)
    rng = np.random.default_rng(4)
    lasts = [d.last_accepted, np.full(d.B, -1, np.int32),
             np.array([int(rng.integers(0, d.N)) for _ in range(d.B)], np.int32)]
    for last in lasts:
        last = np.asarray(last, np.int32)
        S = t["S0"].clone()
        st = torch.full((d.B,), 77, dtype=torch.int32, device="cuda")
        G.gdn_replay_commit(S, t["parents"], t["k"], t["v"], t["beta"], t["g"],
                            torch.from_numpy(last).cuda(), dev_status=st)
        torch.cuda.synchronize()
        assert np.all(to_np(st) == G.GDN_OK)
        ref_S, _, _ = O.draft_commit(d, last_accepted=last)
        e = slice_rel_err(to_np(S), ref_S)
        _say(f"  last {last.tolist()}: state max rel err {e:.2e}")
        assert e <= TOL_STATE
        for b in range(d.B):
            if last[b] < 0:
                assert torch.equal(S[b], t["S0"][b])


def test_replay_commit_rejects_out_of_range():
    d = W.make_draft(2, 10, 2, 64, 32, topology="random", accept="leaf_geometric", seed=3)
    t = dev_tensors(d)
    S = t["S0"].clone()
    st = torch.full((d.B,), 77, dtype=torch.int32, device="cuda")
    G.gdn_replay_commit(S, t["parents"], t["k"], t["v"], t["beta"], t["g"],
                        torch.tensor([d.N, -2], dtype=torch.int32, device="cuda"), dev_status=st)
    torch.cuda.synchronize()
    assert to_np(st).tolist() == [G.GDN_ERR_TOPOLOGY, G.GDN_ERR_TOPOLOGY]
    assert torch.equal(S, t["S0"])
