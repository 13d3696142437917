"""The seeded tiny case still reproduces its stored inputs and oracle answers."""

import json
import os

import numpy as np

from linear_attention_gdn_amd import workloads as W
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_case.json")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)["drafts"]


def test_generator_reproduces_stored_inputs():
    for rec, d in zip(_load(), W.tiny_case(0)):
        assert rec["name"] == d.name
        for key in ("S0", "q", "k", "v", "beta", "g"):
            assert np.array_equal(np.asarray(rec[key], np.float32),
                                  getattr(d, key).ravel().astype(np.float32)), key
        assert rec["parents"] == d.parents.ravel().tolist()


def test_oracle_reproduces_stored_answers():
    for rec in _load():
        B, N, H, dk, dv = rec["B"], rec["N"], rec["H"], rec["dk"], rec["dv"]
        f = lambda key, shape: np.asarray(rec[key], np.float64).reshape(shape)
        S0 = f("S0", (B, H, dv, dk))
        par = np.asarray(rec["parents"], np.int32).reshape(B, N)
        args = (f("q", (B, N, H, dk)), f("k", (B, N, H, dk)), f("v", (B, N, H, dv)),
                f("beta", (B, N, H)), f("g", (B, N, H)))
        out, up, G = O.tree_verify(S0, par, *args)
        np.testing.assert_allclose(out.ravel(), rec["out"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(up.ravel(), rec["uprime"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(G.ravel(), rec["G"], rtol=0, atol=1e-15)
        for c in rec["commits"]:
            Snew, path, plen = O.commit(S0, par, args[1], args[2], args[3], args[4],
                                        np.array([c["last_accepted"]], np.int32))
            assert path[0, :plen[0]].tolist() == c["path"]
            np.testing.assert_allclose(Snew.ravel(), c["S_new"], rtol=0, atol=1e-15)
