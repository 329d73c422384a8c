"""Write tests/golden/oracle_regression.json from the float64 oracle alone.

The pages print no worked numeric example, so no stored value here comes from them.  This
file is a regression snapshot: the inputs are drawn from a seeded numpy generator and rounded
to bf16, and the expected outputs are what oracle/ computes for them.  Re-running this script
after a change to the oracle's arithmetic shows the change in the diff; the commit that makes
such a change names the passage (or the reading of it) that justifies it.

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402

B, HQ, HKV, T, D, TOPK = 1, 2, 1, 64 * 5 + 7, 4, 1


def main():
    r = np.random.default_rng(20251203)
    q = O.round_to_dtype(r.standard_normal((B, HQ, T, D)), "bf16")
    k = O.round_to_dtype(r.standard_normal((B, HKV, T, D)), "bf16")
    v = O.round_to_dtype(r.standard_normal((B, HKV, T, D)), "bf16")
    doc = {"shape": dict(B=B, Hq=HQ, Hkv=HKV, T=T, D=D, topk=TOPK, block=64, n_sink=1, n_local=2),
           "dtype": "bf16", "q": q.tolist(), "k": k.tolist(), "v": v.tolist(), "expected": {}}
    for mode in ["plain", "sas", "hils"]:
        res = O.prefill(q, k, v, topk=TOPK, mode=mode, dtype="bf16")
        doc["expected"][mode] = {"idx": res["idx"].tolist(), "out": res["out"].tolist(),
                                 "lm": res["lm"].tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
    with open(path, "w") as f:
        json.dump(doc, f, separators=(",", ":"))
    print("wrote", path)


if __name__ == "__main__":
    main()
