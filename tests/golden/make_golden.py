"""Write tests/golden/tiny_case.json: the 1-head, d=16 FP32 case and the oracle's answers.

The SpecLA review pages print no worked example, so this fixture is a
regression record of the oracle on the seeded tiny case (a 4-node chain and a
7-node binary tree sharing one S0, accepted path root -> left -> left).  It
calls only the seeded generator and oracle/.  Re-run after a justified change
to the oracle: ``python tests/golden/make_golden.py``.
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from linear_attention_gdn_amd import workloads as W  # noqa: E402
from oracle import oracle as O  # noqa: E402


def main():
    out = {"source": "seeded tiny case (seed 0); expected values from oracle/ only",
           "drafts": []}
    for d in W.tiny_case(0):
        o, up, G = O.draft_verify(d)
        commits = []
        for last in range(-1, d.N):
            Snew, path, plen = O.draft_commit(d, last_accepted=[last])
            commits.append({"last_accepted": last, "path": path[0, :plen[0]].tolist(),
                            "S_new": Snew.ravel().tolist()})
        out["drafts"].append({
            "name": d.name, "B": d.B, "N": d.N, "H": d.H, "dk": d.dk, "dv": d.dv,
            "S0": d.S0.ravel().tolist(), "q": d.q.ravel().tolist(), "k": d.k.ravel().tolist(),
            "v": d.v.ravel().tolist(), "beta": d.beta.ravel().tolist(),
            "g": d.g.ravel().tolist(), "parents": d.parents.ravel().tolist(),
            "last_accepted": d.last_accepted.tolist(), "out": o.ravel().tolist(),
            "uprime": up.ravel().tolist(), "G": G.ravel().tolist(), "commits": commits})
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_case.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
