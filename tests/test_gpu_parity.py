"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Masks, parent copies, key copies and accepted paths must match exactly;
floating-point results within the per-(sequence, head) max-relative-error
bounds in ``_gpu``: 2e-3 for outputs and u', 1e-3 for committed states.
Sizes span several MFMA tiles and ragged tails (N, dk, dv not multiples of
the tile sizes) and include the three full-size layer workloads.
"""

import sys

import numpy as np
import pytest
import torch

from _gpu import (TOL_OUT, TOL_STATE, TOL_UP, dev_tensors, elem_rel_err, out_err, run_chain,
                  run_commit, run_tree, slice_rel_err, to_np)
from linear_attention_gdn_amd import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_verify(d, out, rec, mask=None, st=None):
    ref_out, ref_up, ref_G = O.draft_verify(d)
    e_out = out_err(out, ref_out)
    e_up = slice_rel_err(to_np(rec.uprime), ref_up)
    el_out = elem_rel_err(to_np(out).transpose(0, 2, 1, 3), ref_out.transpose(0, 2, 1, 3))
    el_up = elem_rel_err(to_np(rec.uprime), ref_up)
    _say(f"  slice max rel err: out {e_out:.2e}, u' {e_up:.2e}; elementwise (floor 1e-6 of "
         f"the slice max): out {el_out:.2e}, u' {el_up:.2e}")
    assert e_out <= TOL_OUT, f"outputs: {e_out:.3e}"
    assert e_up <= TOL_UP, f"u': {e_up:.3e}"
    np.testing.assert_allclose(to_np(rec.G), ref_G, rtol=1e-5, atol=1e-5)
    m_ref, _ = O.masks(d.parents)
    assert np.array_equal(to_np(rec.mask).view(np.uint64), m_ref)
    assert np.array_equal(to_np(rec.parents), d.parents)
    kk = to_np(rec.K.view(torch.int16) if d.dtype == "bf16" else rec.K)
    kin = d.k.view(np.int16) if d.dtype == "bf16" else d.k
    assert np.array_equal(kk, kin.transpose(0, 2, 1, 3))
    if mask is not None:
        assert np.array_equal(to_np(mask).view(np.uint64), m_ref)
    if st is not None:
        assert np.all(to_np(st) == 0)
    return e_out, e_up


def _check_commits(d, rec, t, lasts):
    for last in lasts:
        last = np.asarray(last, np.int32)
        S, path, plen, st = run_commit(d, rec, t["S0"], last)
        ref_S, ref_path, ref_plen = O.draft_commit(d, last_accepted=last)
        assert np.array_equal(to_np(plen), ref_plen)
        assert np.array_equal(to_np(path), ref_path)
        assert np.all(to_np(st) == 0)
        e = slice_rel_err(to_np(S), ref_S)
        _say(f"  commit {last.tolist()}: slice max rel err {e:.2e}, elementwise "
             f"{elem_rel_err(to_np(S), ref_S):.2e}")
        assert e <= TOL_STATE, f"state after commit to {last}: {e:.3e}"
        for b in range(d.B):
            if last[b] < 0:
                assert torch.equal(S[b], t["S0"][b])


# --------------------------------------------------------------------------
# the five... the three single-layer workloads and the tiny case
# --------------------------------------------------------------------------


def test_tiny_case_chain_and_binary_tree():
    chain, tree = W.tiny_case(0)
    _say("tiny chain4 / binary7, d=16, f32")
    out, rec, t = run_chain(chain)
    _check_verify(chain, out, rec)
    _check_commits(chain, rec, t, [[x] for x in range(-1, 4)])
    out, rec, mask, st, t = run_tree(chain)
    _check_verify(chain, out, rec, mask, st)
    _check_commits(chain, rec, t, [[x] for x in range(-1, 4)])
    out, rec, mask, st, t = run_tree(tree)
    _check_verify(tree, out, rec, mask, st)
    _check_commits(tree, rec, t, [[x] for x in range(-1, 7)])


def test_chain8_layer_all_accepted_lengths():
    d = W.chain8_layer(0)
    _say("chain8 B=1 H=8 d=256 bf16: chain verify + commits 0..8")
    out, rec, t = run_chain(d)
    e = _check_verify(d, out, rec)
    _say("  errors", e)
    _check_commits(d, rec, t, [[L - 1] for L in range(0, 9)])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree32_layer(seed):
    d = W.tree32_layer(seed)
    _say(f"tree32 B=1 H=8 d=256 bf16 seed={seed}")
    out, rec, mask, st, t = run_tree(d)
    e = _check_verify(d, out, rec, mask, st)
    _say("  errors", e)
    leaves = W.leaves_of(d.parents[0])
    _check_commits(d, rec, t, [d.last_accepted, [-1], [leaves[0]], [leaves[-1]]])


def test_tree64_batch8():
    d = W.tree64_batch8(0)
    _say("tree64 B=8 H=8 d=256 bf16")
    out, rec, mask, st, t = run_tree(d)
    e = _check_verify(d, out, rec, mask, st)
    _say("  errors", e)
    deepest = [int(np.argmax(W.depths_of(d.parents[b]))) for b in range(d.B)]
    mixed = [(-1 if b % 3 == 0 else deepest[b]) for b in range(d.B)]
    _check_commits(d, rec, t, [d.last_accepted, deepest, mixed])


# --------------------------------------------------------------------------
# ragged and extreme shapes
# --------------------------------------------------------------------------

SHAPES = [
    # B, N, H, dk, dv, dtype, topology
    (3, 37, 3, 72, 52, "bf16", "random"),
    (2, 17, 2, 40, 20, "f32", "branching"),
    (1, 64, 2, 256, 256, "bf16", "chain"),
    (2, 64, 2, 256, 256, "f32", "random"),
    (2, 1, 2, 8, 4, "bf16", "chain"),
    (1, 33, 1, 128, 100, "bf16", "window"),
    (4, 64, 1, 256, 256, "bf16", "branching"),
    # root paths of 9-12 and 13-16 nodes: the two register-block solves
    (2, 11, 2, 32, 48, "f32", "chain"),
    (1, 14, 2, 64, 64, "bf16", "chain"),
    # deep drafts (root paths of 17 to 64 nodes): the blocked solve
    (2, 17, 2, 64, 32, "bf16", "chain"),
    (2, 20, 2, 64, 64, "f32", "spine"),
    (3, 33, 2, 128, 96, "bf16", "spine"),
    (2, 48, 8, 256, 256, "bf16", "spine"),
    (8, 64, 8, 256, 256, "bf16", "spine"),
    (1, 40, 3, 72, 52, "f32", "chain"),
    # 64-row state tiles (batch x heads >= 256 tiles): products chained in
    # registers, ragged dv (a partial last tile) and N
    (32, 37, 8, 72, 100, "bf16", "random"),
    (16, 24, 16, 40, 68, "f32", "spine"),
    # 32-row state tiles (batch x heads x dv / 64 < 256 <= batch x heads x dv / 32):
    # full and ragged (a partial last tile, dk and N off the 16 grid)
    (4, 40, 8, 256, 256, "bf16", "branching"),
    (6, 29, 8, 96, 168, "bf16", "random"),
    # 16-row state tiles (the column parts summed apart): ragged dk and dv, and
    # a 40-node chain (the blocked solve)
    (1, 20, 16, 96, 120, "bf16", "branching"),
    (2, 40, 8, 256, 256, "bf16", "chain"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_ragged_shapes(shape):
    B, N, H, dk, dv, dtype, topo = shape
    _say("shape", shape)
    d = W.make_draft(B, N, H, dk, dv, topology=topo, accept="full", dtype=dtype, seed=5,
                     state_std=0.05, gate_shift=1.0, scale=0.7)
    out, rec, mask, st, t = run_tree(d)
    _check_verify(d, out, rec, mask, st)
    rng = np.random.default_rng(1)
    lasts = [d.last_accepted, rng.integers(-1, N, size=B)]
    _check_commits(d, rec, t, lasts)
    if topo == "chain":
        out2, rec2, t2 = run_chain(d, t)
        _check_verify(d, out2, rec2)
        _check_commits(d, rec2, t2, lasts)


# --------------------------------------------------------------------------
# invariants on the GPU
# --------------------------------------------------------------------------


def test_runs_are_bitwise_deterministic():
    d = W.tree64_batch8(1)
    o1, r1, _, _, t = run_tree(d)
    o2, r2, _, _, _ = run_tree(d, t)
    assert torch.equal(o1, o2) and torch.equal(r1.buf, r2.buf)
    c = W.chain8_layer(1)
    o1, r1, t = run_chain(c)
    o2, r2, _ = run_chain(c, t)
    assert torch.equal(o1, o2) and torch.equal(r1.buf, r2.buf)


@pytest.mark.parametrize("kind", ["window", "spine", "window_b8", "spine_b8"])
def test_non_descendants_bitwise_unchanged(kind):
    """Masked terms are exact zeros, in the per-path solve (window trees) and
    in the blocked solve of deep drafts (spine trees, paths past 16 nodes),
    with narrow state-row tiles (batch 1: products through LDS) and wide ones
    (batch 8: products chained in registers)."""
    if kind == "window":
        d = W.tree32_layer(3)
        x = 5
    elif kind == "window_b8":
        d = W.make_draft(8, 64, 8, 256, 256, topology="window", accept="full", seed=13)
        x = 7
    else:
        B = 8 if kind == "spine_b8" else 1
        d = W.make_draft(B, 64, 8, 256, 256, topology="spine", accept="full", seed=12)
        assert W.depths_of(d.parents[0]).max() > 16
        x = 20
    out, _, mask, _, t = run_tree(d)
    m = to_np(mask).view(np.uint64)[0]
    desc = np.array([(int(m[i]) >> x) & 1 for i in range(d.N)], dtype=bool)
    t2 = dict(t)
    for key in ("q", "k", "v"):
        t2[key] = t[key].clone()
        t2[key][0, x] = -t2[key][0, x]
    t2["beta"] = t["beta"].clone()
    t2["beta"][0, x] = 0.5
    t2["g"] = t["g"].clone()
    t2["g"][0, x] -= 0.25
    out2, _, _, _, _ = run_tree(d, t2)
    assert torch.equal(out2[0, torch.from_numpy(~desc).cuda()],
                       out[0, torch.from_numpy(~desc).cuda()])
    assert not torch.equal(out2[0, x], out[0, x])


def test_tree_kernel_on_chain_matches_chain_kernel():
    d = W.chain8_layer(2)
    o_c, r_c, t = run_chain(d)
    o_t, r_t, _, _, _ = run_tree(d, t)
    ref, _, _ = O.draft_verify(d)
    scale = np.abs(ref).max()
    assert float((o_c - o_t).abs().max()) <= 2 * TOL_OUT * scale
    assert torch.equal(r_c.mask, r_t.mask) and torch.equal(r_c.parents, r_t.parents)


def test_sibling_relabelling():
    d = W.make_draft(1, 24, 2, 64, 64, topology="branching", accept="full", seed=3)
    par = d.parents[0]
    kids = [[] for _ in range(d.N)]
    for i in range(1, d.N):
        kids[par[i]].append(i)
    order = [0]
    i = 0
    while i < len(order):
        order.extend(reversed(kids[order[i]]))
        i += 1
    order = np.array(order)
    new_of_old = np.empty(d.N, dtype=np.int64)
    new_of_old[order] = np.arange(d.N)
    newpar = np.array([-1 if par[o] < 0 else new_of_old[par[o]] for o in order], np.int32)
    d2 = d.replace(q=d.q[:, order], k=d.k[:, order], v=d.v[:, order], beta=d.beta[:, order],
                   g=d.g[:, order], parents=newpar[None, :])
    o1, _, _, _, _ = run_tree(d)
    o2, _, _, _, _ = run_tree(d2)
    scale = float(o1.abs().max())
    assert float((o2 - o1[:, torch.from_numpy(order).cuda()]).abs().max()) <= 1e-5 * scale


# --------------------------------------------------------------------------
# error paths forced from the host (every kernel still exits normally)
# --------------------------------------------------------------------------


def test_rejected_topology_zeroes_outputs_and_blocks_commit():
    d = W.make_draft(2, 12, 2, 32, 16, topology="random", accept="full", seed=4)
    bad = d.parents.copy()
    bad[1, 5] = 7  # not topological
    d = d.replace(parents=bad)
    out, rec, mask, st, t = run_tree(d)
    assert list(to_np(st)) == [0, -3]
    assert torch.all(out[1] == 0) and torch.all(rec.uprime[1] == 0)
    assert torch.all(mask[1] == 0)
    good = d.replace(B=1, S0=d.S0[:1], q=d.q[:1], k=d.k[:1], v=d.v[:1], beta=d.beta[:1],
                     g=d.g[:1], parents=d.parents[:1], last_accepted=d.last_accepted[:1])
    ref_out, _, _ = O.draft_verify(good)
    assert out_err(out[:1], ref_out) <= TOL_OUT
    S, path, plen, cst = run_commit(d, rec, t["S0"], [11, 3])
    assert list(to_np(cst)) == [0, -3] and int(plen[1]) == -1
    assert torch.equal(S[1], t["S0"][1])
    ref_S, _, _ = O.draft_commit(good, last_accepted=np.array([11], np.int32))
    assert slice_rel_err(to_np(S[:1]), ref_S) <= TOL_STATE


def test_commit_rejects_out_of_range_index():
    d = W.chain8_layer(0)
    out, rec, t = run_chain(d)
    S, path, plen, st = run_commit(d, rec, t["S0"], [8])
    assert int(st[0]) == -3 and int(plen[0]) == -1
    assert torch.equal(S, t["S0"])
    S, path, plen, st = run_commit(d, rec, t["S0"], [-5])
    assert int(st[0]) == -3 and torch.equal(S, t["S0"])
