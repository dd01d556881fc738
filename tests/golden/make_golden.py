"""Write oracle_tiny.json: tiny seeded inputs and the fp64 oracle's outputs.

Calls only ``oracle`` and ``workloads`` (never the HIP library). Run from the
repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

CASES = [
    dict(B=1, Hq=2, Hkv=1, Sq=3, Skv=5, d=4, causal=True, seed=501),
    dict(B=2, Hq=2, Hkv=2, Sq=4, Skv=4, d=4, causal=False, seed=502),
    dict(B=1, Hq=4, Hkv=2, Sq=1, Skv=6, d=8, causal=True, seed=503),
]


def main():
    out = []
    for c in CASES:
        case = workloads.prefill_case(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Skv"], c["d"], c["causal"], "bf16",
                                      seed=c["seed"])
        q, k, v = case.as_f64()
        o, lse = oracle.attention(q, k, v, case.scale, case.causal)
        out.append(dict(c, scale=case.scale, q_bits=case.q.reshape(-1).tolist(), k_bits=case.k.reshape(-1).tolist(),
                        v_bits=case.v.reshape(-1).tolist(), o=o.reshape(-1).tolist(), lse=lse.reshape(-1).tolist()))
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as f:
        json.dump({"generator": "tests/golden/make_golden.py", "cases": out}, f, indent=1)


if __name__ == "__main__":
    main()
