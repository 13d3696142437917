"""GPU parity of the chain-decomposed hybrid verifier (gdn_hybrid_verify)
against the oracle: outputs, the factor record (u', G; masks, parents and the
k copy exactly), and commits from its record, on deep drafts (17- to 64-node
root paths) and ordinary trees."""

import sys

import numpy as np
import pytest
import torch

from _gpu import (TOL_OUT, TOL_STATE, TOL_UP, code_of, dev_tensors, out_err, run_commit,
                  slice_rel_err, to_np)
from linear_attention_gdn_amd import gdnspec as G
from linear_attention_gdn_amd import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_hybrid(d, t=None):
    t = t or dev_tensors(d)
    plan = G.HybridPlan(d.parents)
    out = torch.full((d.B, d.N, d.H, d.dv), float("nan"), device="cuda")
    rec = G.FactorRecord.empty(d.B, d.N, d.H, d.dk, d.dv, code_of(d))
    st = torch.full((d.B,), 77, dtype=torch.int32, device="cuda")
    G.gdn_hybrid_verify(t["S0"], t["parents"], t["q"], t["k"], t["v"], t["beta"], t["g"], out,
                        rec, plan, scale=d.scale, dev_status=st)
    torch.cuda.synchronize()
    return out, rec, st, t, plan


CASES = [
    # B, N, H, dk, dv, dtype, topology
    (1, 64, 8, 256, 256, "bf16", "chain"),
    (8, 64, 8, 256, 256, "bf16", "spine"),
    (2, 40, 3, 72, 52, "f32", "chain"),
    (3, 33, 2, 128, 96, "bf16", "spine"),
    (2, 17, 2, 64, 32, "bf16", "chain"),
    (1, 32, 8, 256, 256, "bf16", "window"),
    (4, 64, 2, 256, 256, "bf16", "branching"),
    (2, 7, 1, 16, 16, "f32", "binary"),
    (2, 1, 2, 8, 4, "bf16", "chain"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_hybrid_matches_oracle(case):
    B, N, H, dk, dv, dtype, topo = case
    d = W.make_draft(B, N, H, dk, dv, topology=topo, accept="full", dtype=dtype, seed=11,
                     state_std=0.05, gate_shift=1.0, scale=0.7)
    out, rec, st, t, plan = run_hybrid(d)
    _say(f"hybrid {case}: {plan.levels} levels, chains {plan.chains_per_level[:plan.levels]}")
    assert np.all(to_np(st) == G.GDN_OK)
    ref_out, ref_up, ref_G = O.draft_verify(d)
    e_out = out_err(out, ref_out)
    e_up = slice_rel_err(to_np(rec.uprime), ref_up)
    _say(f"  outputs {e_out:.2e}, u' {e_up:.2e}")
    assert e_out <= TOL_OUT and e_up <= TOL_UP
    np.testing.assert_allclose(to_np(rec.G), ref_G, rtol=1e-5, atol=1e-5)
    m_ref, _ = O.masks(d.parents)
    assert np.array_equal(to_np(rec.mask).view(np.uint64), m_ref)
    assert np.array_equal(to_np(rec.parents), d.parents)
    kk = to_np(rec.K.view(torch.int16) if dtype == "bf16" else rec.K)
    kin = d.k.view(np.int16) if dtype == "bf16" else d.k
    assert np.array_equal(kk, kin.transpose(0, 2, 1, 3))
    rng = np.random.default_rng(2)
    for last in (d.last_accepted, rng.integers(-1, N, size=B).astype(np.int32)):
        S, _, _, cst = run_commit(d, rec, t["S0"], last)
        ref_S, _, _ = O.draft_commit(d, last_accepted=np.asarray(last, np.int32))
        assert np.all(to_np(cst) == G.GDN_OK)
        assert slice_rel_err(to_np(S), ref_S) <= TOL_STATE


def test_hybrid_rejected_topology_zeroes_that_sequence():
    d = W.make_draft(2, 12, 2, 32, 16, topology="spine", accept="full", seed=4)
    plan_par = d.parents.copy()
    t = dev_tensors(d)
    bad = d.parents.copy()
    bad[1, 5] = 7  # the device copy of sequence 1 is not topological
    t["parents"] = torch.from_numpy(bad).cuda()
    plan = G.HybridPlan(plan_par)
    out = torch.full((d.B, d.N, d.H, d.dv), float("nan"), device="cuda")
    rec = G.FactorRecord.empty(d.B, d.N, d.H, d.dk, d.dv, code_of(d))
    st = torch.full((d.B,), 77, dtype=torch.int32, device="cuda")
    G.gdn_hybrid_verify(t["S0"], t["parents"], t["q"], t["k"], t["v"], t["beta"], t["g"], out,
                        rec, plan, dev_status=st)
    torch.cuda.synchronize()
    assert to_np(st).tolist() == [G.GDN_OK, G.GDN_ERR_TOPOLOGY]
    assert torch.all(out[1] == 0) and torch.all(rec.uprime[1] == 0) and torch.all(rec.mask[1] == 0)
    good = d.replace(B=1, S0=d.S0[:1], q=d.q[:1], k=d.k[:1], v=d.v[:1], beta=d.beta[:1],
                     g=d.g[:1], parents=d.parents[:1], last_accepted=d.last_accepted[:1])
    ref_out, _, _ = O.draft_verify(good)
    assert out_err(out[:1], ref_out) <= TOL_OUT
