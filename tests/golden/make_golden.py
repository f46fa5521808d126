"""Writes oracle_small.json: oracle outputs for small seeded problems.

Calls only the oracle and the seeded input generator.  The pages print no
worked numeric example of the attention outputs, so this fixture is a
regression record of the (pinned) oracle, used by the CPU tests and by the GPU
parity tests as a fixed small case.  Regenerate with
``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import attn_inputs as gen  # noqa: E402
import oracle.attention as att  # noqa: E402

CASES = [
    dict(B=1, Hq=2, Hkv=1, Sq=5, Sk=7, layout=gen.BSHD, causal=True, seed=900),
    dict(B=1, Hq=2, Hkv=2, Sq=3, Sk=9, layout=gen.BHSD, causal=False, seed=901),
]


def main():
    out = {"about": "oracle outputs (float64, logical [B,Hq,Sq,D] / [B,Hq,Sq]) for "
                    "seeded inputs from attn_inputs.prefill_inputs; written by "
                    "make_golden.py from oracle.attention only", "cases": []}
    for c in CASES:
        p = gen.prefill_inputs(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"],
                               layout=c["layout"], causal=c["causal"], seed=c["seed"])
        o, lse = att.attention(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                               p.causal, p.layout)
        d = dict(c)
        d["o"] = [float(x) for x in o.ravel()]
        d["lse"] = [None if x == -np.inf else float(x) for x in lse.ravel()]
        out["cases"].append(d)
    with open(os.path.join(HERE, "oracle_small.json"), "w") as f:
        json.dump(out, f, indent=0)


if __name__ == "__main__":
    main()
