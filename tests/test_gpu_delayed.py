"""GPU checks of the delayed commit fused into the next verification
(gdn_chain_verify_delayed): bitwise equal to gdn_commit_path followed by the
plain verification, for previous records written from chains and from
trees, and close to the oracle's commit-then-verify."""

import numpy as np
import pytest
import torch

from linear_attention_gdn_amd import gdnspec as G
from linear_attention_gdn_amd import workloads as W
from oracle import oracle as O

from _gpu import TOL_OUT, TOL_STATE, code_of, dev_tensors, run_chain, run_tree, slice_rel_err

pytestmark = pytest.mark.gpu


def _lasts(prev: W.Draft, rng):
    B, Np = prev.B, prev.N
    cases = [np.full(B, -1), np.full(B, Np - 1), prev.last_accepted.copy()]
    cases.append(np.array([int(rng.integers(-1, Np)) for _ in range(B)]))
    bad = prev.last_accepted.copy()
    bad[0] = Np  # out of range: that sequence is not committed
    cases.append(bad)
    return [c.astype(np.int32) for c in cases]


@pytest.mark.parametrize("dtype,B,Np,N,H,dk,dv,prev_topo", [
    ("bf16", 1, 8, 8, 8, 256, 256, "chain"),
    ("bf16", 2, 12, 5, 3, 64, 24, "random"),
    ("f32", 2, 7, 9, 2, 40, 32, "chain"),
    ("bf16", 3, 64, 16, 2, 256, 64, "branching"),
    ("bf16", 1, 1, 3, 1, 16, 8, "chain"),
    ("bf16", 1, 64, 64, 2, 256, 16, "chain"),  # largest LDS footprint (~136 KB)
])
def test_delayed_chain_verify_is_commit_then_verify(dtype, B, Np, N, H, dk, dv, prev_topo):
    seed = B * 100 + Np + N
    accept = "uniform" if prev_topo == "chain" else "leaf_geometric"
    prev = W.make_draft(B, Np, H, dk, dv, topology=prev_topo, accept=accept, dtype=dtype,
                        seed=seed)
    new = W.make_draft(B, N, H, dk, dv, topology="chain", accept="none", dtype=dtype,
                       seed=seed + 1)
    if prev_topo == "chain":
        _, rec_prev, tp = run_chain(prev)
    else:
        _, rec_prev, _, st, tp = run_tree(prev)
        assert (st.cpu().numpy() == G.GDN_OK).all()
    tn = dev_tensors(new)
    rng = np.random.default_rng(seed)
    for last in _lasts(prev, rng):
        last_t = torch.from_numpy(last).cuda()
        # two calls
        S_a = tp["S0"].clone()
        st_a = torch.full((B,), 77, dtype=torch.int32, device="cuda")
        G.gdn_commit_path(S_a, rec_prev, last_t, dev_status=st_a)
        out_a = torch.full((B, N, H, dv), float("nan"), device="cuda")
        rec_a = G.FactorRecord.empty(B, N, H, dk, dv, code_of(new))
        rec_a.buf.zero_()
        G.gdn_chain_verify(S_a, tn["q"], tn["k"], tn["v"], tn["beta"], tn["g"], out_a, rec_a)
        # one fused call
        S_b = tp["S0"].clone()
        st_b = torch.full((B,), 77, dtype=torch.int32, device="cuda")
        out_b = torch.full((B, N, H, dv), float("nan"), device="cuda")
        rec_b = G.FactorRecord.empty(B, N, H, dk, dv, code_of(new))
        rec_b.buf.zero_()
        G.gdn_chain_verify_delayed(S_b, rec_prev, last_t, tn["q"], tn["k"], tn["v"], tn["beta"],
                                   tn["g"], out_b, rec_b, dev_status=st_b)
        torch.cuda.synchronize()
        assert torch.equal(st_a, st_b), (last, st_a, st_b)
        assert torch.equal(S_a, S_b), last
        assert torch.equal(out_a, out_b), last
        assert torch.equal(rec_a.buf, rec_b.buf), last
        for b in range(B):
            ok = -1 <= last[b] < Np
            assert int(st_b[b]) == (G.GDN_OK if ok else G.GDN_ERR_TOPOLOGY)


def test_delayed_chain_verify_matches_oracle():
    """Commit of a tree path then a chain verification, against the oracle's
    replay of the same two steps."""
    prev = W.make_draft(2, 32, 8, 256, 256, topology="window", accept="leaf_geometric",
                        dtype="bf16", seed=31)
    new = W.make_draft(2, 8, 8, 256, 256, topology="chain", accept="none", dtype="bf16",
                       seed=32)
    _, rec_prev, _, _, tp = run_tree(prev)
    tn = dev_tensors(new)
    S = tp["S0"].clone()
    out = torch.empty(2, 8, 8, 256, device="cuda")
    rec = G.FactorRecord.empty(2, 8, 8, 256, 256, G.GDN_BF16)
    G.gdn_chain_verify_delayed(S, rec_prev, tp["last"], tn["q"], tn["k"], tn["v"], tn["beta"],
                               tn["g"], out, rec)
    torch.cuda.synchronize()
    S_ref, _, _ = O.draft_commit(prev)
    out_ref, _, _ = O.tree_verify(S_ref, new.parents, new.q64(), new.k64(), new.v64(), new.beta,
                                  new.g, new.scale)
    assert slice_rel_err(S.cpu().numpy(), S_ref) <= TOL_STATE
    assert slice_rel_err(out.cpu().numpy().transpose(0, 2, 1, 3),
                         out_ref.transpose(0, 2, 1, 3)) <= TOL_OUT


def _prev_record(prev: W.Draft):
    if (prev.parents == W.chain_parents(prev.N)[None]).all():
        _, rec, tp = run_chain(prev)
    else:
        _, rec, _, st, tp = run_tree(prev)
        assert (st.cpu().numpy() == G.GDN_OK).all()
    return rec, tp


@pytest.mark.parametrize("dtype,B,Np,N,H,dk,dv,prev_topo,new_topo", [
    ("bf16", 1, 32, 32, 8, 256, 256, "window", "window"),      # 16-row tiles
    ("bf16", 8, 64, 64, 8, 256, 256, "branching", "branching"),  # 64-row tiles
    ("bf16", 2, 40, 12, 3, 64, 40, "chain", "random"),         # 40-node path: 3 chunks
    ("f32", 2, 9, 17, 2, 40, 24, "random", "window"),
    ("bf16", 1, 5, 1, 1, 16, 8, "binary", "chain"),
    # deep drafts (blocked solve) with long previous paths, wide and narrow tiles
    ("bf16", 8, 64, 64, 8, 256, 256, "spine", "spine"),
    ("bf16", 1, 48, 48, 8, 256, 256, "spine", "spine"),
    # 64-row tiles: a 64-node accepted path (four staging rounds, a full last
    # group of four) and ragged dk, dv and N with short paths
    ("bf16", 8, 64, 16, 8, 256, 256, "chain", "window"),
    ("bf16", 32, 23, 17, 8, 72, 100, "random", "random"),
    # 32-row tiles: full, and ragged with a 40-node accepted path
    ("bf16", 4, 40, 40, 8, 256, 256, "branching", "branching"),
    ("bf16", 6, 40, 29, 8, 96, 168, "chain", "random"),
    # 16-row tiles (four state waves, a quarter of the columns each): ragged
    # dk (the last two quarters all padding) and dv (a half last tile), and a
    # 40-node accepted path (commit from global memory)
    ("bf16", 1, 24, 20, 16, 96, 120, "random", "branching"),
    ("bf16", 2, 40, 12, 8, 256, 256, "chain", "random"),
    # 32-row tiles, deep drafts on both sides (a 48-node accepted path, the
    # blocked solve)
    ("bf16", 4, 48, 48, 8, 256, 256, "spine", "spine"),
])
def test_delayed_tree_verify_is_commit_then_verify(dtype, B, Np, N, H, dk, dv, prev_topo,
                                                   new_topo):
    _fused_equals_separate(dtype, B, Np, N, H, dk, dv, prev_topo, new_topo, reject=False)


# The split-role kernel's rejected-draft path with a pending commit: 64-row
# tiles (commit applied from global memory there) with short and long
# previous paths, and 16- and 32-row tiles (commit applied before the first
# wait on the head waves, split over four state waves).  The last sequence's
# new draft is not topological.
@pytest.mark.parametrize("B,Np,N,H,prev_topo", [
    (8, 64, 64, 8, "branching"),
    (8, 64, 64, 8, "spine"),
    (1, 32, 32, 8, "window"),
    (4, 40, 40, 8, "spine"),
])
def test_delayed_tree_verify_rejected_draft_is_commit_then_verify(B, Np, N, H, prev_topo):
    _fused_equals_separate("bf16", B, Np, N, H, 256, 256, prev_topo, "branching", reject=True)


def _fused_equals_separate(dtype, B, Np, N, H, dk, dv, prev_topo, new_topo, reject):
    seed = 7 * B + Np + N + (1000 if reject else 0)
    accept = "full" if prev_topo == "chain" else "leaf_geometric"
    prev = W.make_draft(B, Np, H, dk, dv, topology=prev_topo, accept=accept, dtype=dtype,
                        seed=seed)
    new = W.make_draft(B, N, H, dk, dv, topology=new_topo, accept="none", dtype=dtype,
                       seed=seed + 1)
    if reject:
        bad = new.parents.copy()
        bad[B - 1, N - 2] = N - 1  # a parent after its child
        new = new.replace(parents=bad)
    rec_prev, tp = _prev_record(prev)
    tn = dev_tensors(new)
    rng = np.random.default_rng(seed)
    for last in _lasts(prev, rng):
        last_t = torch.from_numpy(last).cuda()
        outs = []
        for fused in (False, True):
            S = tp["S0"].clone()
            cst = torch.full((B,), 77, dtype=torch.int32, device="cuda")
            dst = torch.full((B,), 77, dtype=torch.int32, device="cuda")
            msk = torch.zeros((B, N), dtype=torch.int64, device="cuda")
            out = torch.full((B, N, H, dv), float("nan"), device="cuda")
            rec = G.FactorRecord.empty(B, N, H, dk, dv, code_of(new))
            rec.buf.zero_()
            if fused:
                G.gdn_tree_verify_delayed(S, rec_prev, last_t, tn["parents"], tn["q"], tn["k"],
                                          tn["v"], tn["beta"], tn["g"], out, rec,
                                          commit_status=cst, mask_out=msk, dev_status=dst)
            else:
                G.gdn_commit_path(S, rec_prev, last_t, dev_status=cst)
                G.gdn_tree_verify(S, tn["parents"], tn["q"], tn["k"], tn["v"], tn["beta"],
                                  tn["g"], out, rec, mask_out=msk, dev_status=dst)
            outs.append((S, out, rec.buf, cst, dst, msk))
        torch.cuda.synchronize()
        for a, b_ in zip(*outs):
            assert torch.equal(a, b_), last
        if reject:
            dst = outs[1][4]
            assert int(dst[B - 1]) == G.GDN_ERR_TOPOLOGY
            assert (outs[1][1][B - 1] == 0).all()


def test_delayed_tree_commit_lands_when_new_topology_is_rejected():
    prev = W.make_draft(2, 16, 2, 64, 32, topology="window", accept="leaf_geometric",
                        dtype="bf16", seed=51)
    new = W.make_draft(2, 8, 2, 64, 32, topology="chain", accept="none", dtype="bf16", seed=52)
    rec_prev, tp = _prev_record(prev)
    tn = dev_tensors(new)
    tn["parents"][1, 5] = 6  # not topological: sequence 1's draft is rejected
    S_a = tp["S0"].clone()
    G.gdn_commit_path(S_a, rec_prev, tp["last"])
    S_b = tp["S0"].clone()
    out = torch.full((2, 8, 2, 32), float("nan"), device="cuda")
    rec = G.FactorRecord.empty(2, 8, 2, 64, 32, G.GDN_BF16)
    dst = torch.full((2,), 77, dtype=torch.int32, device="cuda")
    G.gdn_tree_verify_delayed(S_b, rec_prev, tp["last"], tn["parents"], tn["q"], tn["k"],
                              tn["v"], tn["beta"], tn["g"], out, rec, dev_status=dst)
    torch.cuda.synchronize()
    assert torch.equal(S_a, S_b)
    assert dst.tolist() == [G.GDN_OK, G.GDN_ERR_TOPOLOGY]
    assert (out[1] == 0).all() and torch.isfinite(out[0]).all()


@pytest.mark.parametrize("B,Np,N,H,dk,dv,topo,delayed,reject", [
    (1, 32, 32, 8, 256, 256, "window", True, False),     # the 24-layer step's shape
    (1, 32, 32, 8, 256, 256, "window", False, False),
    (2, 9, 17, 3, 64, 40, "random", True, False),        # ragged: N and dv not multiples of 16
    (8, 64, 64, 8, 256, 256, "branching", True, False),  # wide tiles
    (4, 40, 40, 8, 256, 256, "branching", True, True),   # 32-row tiles, one draft rejected
    (2, 9, 17, 3, 64, 40, "random", True, True),         # sequence 1's new parents rejected
    (2, 12, 12, 2, 32, 16, "random", False, True),
])
def test_layer_verify_is_verify_then_gate(B, Np, N, H, dk, dv, topo, delayed, reject):
    """gdn_layer_verify == the verify call followed by gdn_gate_merge, bitwise
    (outputs through the gate, state, record, status words), also when a
    sequence's topology is rejected (its outputs are gated zeros)."""
    seed = 7000 + B * 100 + N
    prev = W.make_draft(B, Np, H, dk, dv, topology=topo, accept="leaf_geometric",
                        dtype="bf16", seed=seed)
    new = W.make_draft(B, N, H, dk, dv, topology=topo, accept="none", dtype="bf16",
                       seed=seed + 1)
    if reject:
        bad = new.parents.copy()
        bad[B - 1, N - 2] = N - 1  # a parent after its child
        new = new.replace(parents=bad)
    _, rec_prev, _, st, tp = run_tree(prev)
    assert (st.cpu().numpy() == G.GDN_OK).all()
    tn = dev_tensors(new)
    rng = np.random.default_rng(seed)
    ldg = H * dv + 24  # the gate block sits inside wider rows, as in P
    gate_rows = torch.from_numpy(rng.standard_normal((B * N, ldg)).astype(np.float32)).cuda()
    gate = gate_rows[:, 8:8 + H * dv]
    last_t = torch.from_numpy(prev.last_accepted.astype(np.int32)).cuda()
    code = code_of(new)

    S_a = tp["S0"].clone()
    out_a = torch.empty((B, N, H, dv), device="cuda")
    rec_a = G.FactorRecord.empty(B, N, H, dk, dv, code)
    rec_a.buf.zero_()
    st_a = torch.full((B,), 77, dtype=torch.int32, device="cuda")
    cs_a = torch.full((B,), 77, dtype=torch.int32, device="cuda")
    if delayed:
        G.gdn_tree_verify_delayed(S_a, rec_prev, last_t, tn["parents"], tn["q"], tn["k"], tn["v"],
                                  tn["beta"], tn["g"], out_a, rec_a, commit_status=cs_a,
                                  dev_status=st_a)
    else:
        G.gdn_tree_verify(S_a, tn["parents"], tn["q"], tn["k"], tn["v"], tn["beta"], tn["g"],
                          out_a, rec_a, dev_status=st_a)
    Y_a = torch.empty((B * N, H * dv), dtype=torch.bfloat16, device="cuda")
    G.gdn_gate_merge(out_a.view(B * N, H * dv), gate, Y_a)

    S_b = tp["S0"].clone()
    rec_b = G.FactorRecord.empty(B, N, H, dk, dv, code)
    rec_b.buf.zero_()
    st_b = torch.full((B,), 77, dtype=torch.int32, device="cuda")
    cs_b = torch.full((B,), 77, dtype=torch.int32, device="cuda")
    Y_b = torch.full((B * N, H * dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    G.gdn_layer_verify(S_b, tn["parents"], tn["q"], tn["k"], tn["v"], tn["beta"], tn["g"], gate,
                       Y_b, rec_b, prev_factors=rec_prev if delayed else None,
                       last_accepted=last_t if delayed else None,
                       commit_status=cs_b if delayed else None, dev_status=st_b)
    torch.cuda.synchronize()
    assert torch.equal(Y_a.view(torch.int16), Y_b.view(torch.int16))
    assert torch.equal(S_a, S_b)
    assert torch.equal(rec_a.buf, rec_b.buf)
    assert torch.equal(st_a, st_b)
    if reject:
        assert int(st_b[B - 1]) == G.GDN_ERR_TOPOLOGY
        assert torch.all(Y_b.view(B, N, H * dv)[B - 1].float() == 0)
    if delayed:
        assert torch.equal(cs_a, cs_b)


@pytest.mark.parametrize("B,N,H,topo", [(1, 32, 8, "window"), (8, 64, 8, "branching")])
def test_delayed_tree_verify_repeats_bitwise(B, N, H, topo):
    """The delayed tree verify gives the same bits on every run (state, outputs,
    record), with nothing to commit and with a path: each workgroup's result
    depends only on its inputs, never on the timing of other waves."""
    dk = dv = 256
    prev = W.make_draft(B, N, H, dk, dv, topology=topo, accept="leaf_geometric", dtype="bf16",
                        seed=31)
    new = W.make_draft(B, N, H, dk, dv, topology=topo, accept="none", dtype="bf16", seed=32)
    _, rec_prev, _, _, tp = run_tree(prev)
    tn = dev_tensors(new)
    for last_np in (np.full(B, -1, np.int32), prev.last_accepted.astype(np.int32)):
        last = torch.from_numpy(last_np).cuda()
        runs = []
        for _ in range(5):
            S = tp["S0"].clone()
            out = torch.empty((B, N, H, dv), device="cuda")
            rec = G.FactorRecord.empty(B, N, H, dk, dv, code_of(new))
            rec.buf.zero_()
            G.gdn_tree_verify_delayed(S, rec_prev, last, tn["parents"], tn["q"], tn["k"], tn["v"],
                                      tn["beta"], tn["g"], out, rec)
            runs.append((S, out, rec.buf))
        torch.cuda.synchronize()
        for r in runs[1:]:
            for a, b_ in zip(runs[0], r):
                assert torch.equal(a, b_), last_np
