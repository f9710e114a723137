"""The stored small cases: the oracle still reproduces them, and the stored
outputs satisfy the singular-value closed form (so the fixture is pinned to
mathematics, not only to the oracle that wrote it)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from test_oracle import closed_form, relF

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "oracle_small_cases.json")) as f:
    CASES = json.load(f)["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_oracle_reproduces_fixture(case):
    if case["kind"] == "step":
        O, Mn, Wn = oracle.muon_step(np.array(case["W"]), np.array(case["G"]), np.array(case["M"]),
                                     lr=case["lr"], beta=case["beta"], nesterov=case["nesterov"],
                                     iters=case["iters"], col_blocks=case["col_blocks"])
        assert np.allclose(O, case["O"], rtol=0, atol=1e-14)
        assert np.allclose(Mn, case["M_new"], rtol=0, atol=1e-14)
        assert np.allclose(Wn, case["W_new"], rtol=0, atol=1e-14)
    else:
        O = oracle.newton_schulz_blockwise(np.array(case["X"]), case["col_blocks"], iters=case["iters"])
        assert np.allclose(O, case["O"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_fixture_satisfies_closed_form(case):
    if case["kind"] == "step":
        G, M = np.array(case["G"]), np.array(case["M"])
        Mn = case["beta"] * M + G
        X = G + case["beta"] * Mn if case["nesterov"] else Mn
        assert relF(case["O"], closed_form(X, case["iters"])) < 1e-12
        dW = np.array(case["W"]) - np.array(case["W_new"])
        assert relF(dW, case["lr"] * closed_form(X, case["iters"])) < 1e-12
    else:
        X = np.array(case["X"])
        k = case["col_blocks"]
        w = X.shape[1] // k
        O = np.array(case["O"])
        for j in range(k):
            assert relF(O[:, j * w:(j + 1) * w], closed_form(X[:, j * w:(j + 1) * w], case["iters"])) < 1e-12
