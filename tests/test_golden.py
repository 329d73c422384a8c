"""The oracle still reproduces its stored regression snapshot (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
def test_oracle_regression_snapshot(mode):
    with open(os.path.join(HERE, "golden", "oracle_regression.json")) as f:
        doc = json.load(f)
    q, k, v = (np.array(doc[n], dtype=np.float64) for n in ("q", "k", "v"))
    res = O.prefill(q, k, v, topk=doc["shape"]["topk"], mode=mode, dtype=doc["dtype"])
    exp = doc["expected"][mode]
    np.testing.assert_array_equal(res["idx"], np.array(exp["idx"]))
    np.testing.assert_array_equal(res["lm"], np.array(exp["lm"]))
    np.testing.assert_allclose(res["out"], np.array(exp["out"]), rtol=0, atol=1e-13)
