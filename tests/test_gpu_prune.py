"""GPU parity of confidence-guided pruning (gdn_prune_draft) against the
oracle (oracle/prune.py): bit-exact kept indices, renumbered parents and
counts, on synthetic candidate trees with ties, every budget and margin
regime, the largest candidate count, and broken preconditions."""

import numpy as np
import pytest
import torch

from linear_attention_gdn_amd import gdnspec as G
from linear_attention_gdn_amd import workloads as W
from oracle import prune as PR

pytestmark = pytest.mark.gpu


def _run(par, conf, tau, T):
    B = par.shape[0]
    pt = torch.from_numpy(np.ascontiguousarray(par, np.int32)).cuda()
    ct = torch.from_numpy(np.ascontiguousarray(conf, np.float32)).cuda()
    kept = torch.full((B, T), 77, dtype=torch.int32, device="cuda")
    newp = torch.full((B, T), 77, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), 77, dtype=torch.int32, device="cuda")
    st = torch.full((B,), 77, dtype=torch.int32, device="cuda")
    G.gdn_prune_draft(pt, ct, tau, kept, newp, cnt, dev_status=st)
    torch.cuda.synchronize()
    return kept.cpu().numpy(), newp.cpu().numpy(), cnt.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("top_k,depth,B", [(4, 4, 8), (4, 2, 3), (2, 8, 2), (3, 5, 4), (1, 20, 2),
                                           (4, 5, 1)])
@pytest.mark.parametrize("tau,T", [(3.0, 16), (0.0, 16), (50.0, 64), (1.0, 1), (6.0, 64)])
def test_prune_matches_oracle(top_k, depth, B, tau, T):
    par, conf = W.candidate_batch(B, seed=top_k * 100 + depth, top_k=top_k, depth=depth)
    if par.shape[1] > 1024:
        par, conf = par[:, :1024], conf[:, :1024]  # BFS prefix: still a candidate tree
    conf = conf.copy()
    conf[::2] = np.round(conf[::2] * 4) / 4  # ties in every other sequence
    kept, newp, cnt, st = _run(par, conf, tau, T)
    rk, rp, rn = PR.prune_batch(par, conf, tau, T)
    assert np.all(st == G.GDN_OK)
    np.testing.assert_array_equal(cnt, rn)
    np.testing.assert_array_equal(kept, rk)
    np.testing.assert_array_equal(newp, rp)


def test_prune_rejects_broken_preconditions():
    par, conf = W.candidate_batch(4, seed=9, top_k=3, depth=3)
    par, conf = par.copy(), conf.copy()
    par[1, 7] = 9          # not topological
    conf[2, 5] = conf[2, par[2, 5]] + 0.5  # a child above its parent
    conf[3, 4] = np.nan
    kept, newp, cnt, st = _run(par, conf, 3.0, 16)
    assert st.tolist() == [G.GDN_OK] + [G.GDN_ERR_TOPOLOGY] * 3
    assert cnt.tolist()[1:] == [-1, -1, -1]
    assert np.all(kept[1:] == -1) and np.all(newp[1:] == -1)
    rk, rp, rn = PR.prune_batch(par[:1], conf[:1], 3.0, 16)
    np.testing.assert_array_equal(kept[:1], rk)
