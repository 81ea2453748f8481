"""Write oracle_small.json: the float64 oracle on one tiny seeded case (regression fixture).

Calls only the oracle and the seeded input generators. Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import gated_delta_rule  # noqa: E402
from workloads import draw  # noqa: E402

CASE = dict(B=2, L=5, Hk=1, Hv=2, D=4, regime="R1", seed=7, lengths=[5, 3], s0_rows=2)


def compute():
    x = draw(CASE["B"], CASE["L"], CASE["Hk"], CASE["Hv"], CASE["D"], CASE["regime"], CASE["seed"],
             lengths=CASE["lengths"], s0_rows=CASE["s0_rows"])
    o, s = gated_delta_rule(x.q.double().numpy(), x.k.double().numpy(), x.v.double().numpy(),
                            x.g.double().numpy(), x.beta.double().numpy(), lengths=x.lengths.numpy(),
                            s0=x.s0.double().numpy())
    return o, s


if __name__ == "__main__":
    o, s = compute()
    out = {"case": CASE, "o": o.tolist(), "s_final": s.tolist()}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json"), "w") as f:
        json.dump(out, f, indent=0)
    print("wrote oracle_small.json")
