"""Write the stored oracle outputs for the tiny case (regression fixture).

The pages print no worked GDN example, so no stored value comes from them.
This script calls only the oracle (and the seeded input generators) and
writes tiny_case_oracle.json: the recurrent outputs o [64, 16] and the final
state S_T [16, 16] of the one-sequence, one-head, d=16 fp32 case (seed 1,
T=64, scale 1, no conv, no epilogue).  A test recomputes it and requires an
exact match, so any later change to the oracle's arithmetic shows up here.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gdn_inputs  # noqa: E402
from oracle import gdn_oracle as O  # noqa: E402


def tiny_oracle():
    c = gdn_inputs.tiny_case()
    g, beta = O.gating(c.a, c.b, c.A_log, c.dt_bias)
    o, S_T, _ = O.gated_delta_rule(O.l2norm(c.q), O.l2norm(c.k), c.v, g, beta, None, 1.0)
    return o[:, 0], S_T[0]


if __name__ == "__main__":
    o, S = tiny_oracle()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_case_oracle.json")
    with open(path, "w") as f:
        json.dump({"case": "tiny seed=1 T=64 d=16 fp32 scale=1", "o": [[repr(float(x)) for x in r] for r in o],
                   "S_T": [[repr(float(x)) for x in r] for r in S]}, f, indent=0)
    print("wrote", path)
