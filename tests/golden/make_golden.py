"""Writes oracle_small_cases.json: tiny fixed inputs and the CPU oracle's
float64 outputs for them. Calls nothing but the oracle package.

The pages print no worked example, so every stored value here comes from the
oracle; test_golden.py pins the stored outputs themselves to the
singular-value closed form of the iteration, so a wrong value cannot hide here.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def pattern(rows, cols, p, q, r, scale):
    """A fixed, non-symmetric integer pattern scaled to floats."""
    i = np.arange(rows)[:, None]
    j = np.arange(cols)[None, :]
    return (((i * p + j * q + i * j) % r) - (r // 2)).astype(np.float64) * scale


def main():
    cases = []
    # whole step, wide, float32-exact inputs
    G = pattern(6, 10, 7, 3, 11, 0.125)
    M = pattern(6, 10, 5, 2, 13, 0.25)
    W = pattern(6, 10, 3, 1, 7, 0.015625)
    O, Mn, Wn = oracle.muon_step(W, G, M, lr=0.02, beta=0.95)
    cases.append(dict(name="step_wide_6x10", kind="step", lr=0.02, beta=0.95,
                      nesterov=False, iters=5, col_blocks=1,
                      W=W.tolist(), G=G.tolist(), M=M.tolist(),
                      O=O.tolist(), M_new=Mn.tolist(), W_new=Wn.tolist()))
    # whole step, tall, nesterov on
    G = pattern(12, 5, 2, 5, 9, 0.5)
    M = pattern(12, 5, 3, 7, 17, 0.0625)
    W = pattern(12, 5, 1, 4, 5, 0.03125)
    O, Mn, Wn = oracle.muon_step(W, G, M, lr=0.02, beta=0.9, nesterov=True)
    cases.append(dict(name="step_tall_nesterov_12x5", kind="step", lr=0.02, beta=0.9,
                      nesterov=True, iters=5, col_blocks=1,
                      W=W.tolist(), G=G.tolist(), M=M.tolist(),
                      O=O.tolist(), M_new=Mn.tolist(), W_new=Wn.tolist()))
    # newton-schulz only, blockwise, 3 column blocks of 4x4
    X = pattern(4, 12, 5, 3, 7, 1.0)
    O = oracle.newton_schulz_blockwise(X, 3)
    cases.append(dict(name="ns_blockwise_4x12_k3", kind="ns", iters=5, col_blocks=3,
                      X=X.tolist(), O=O.tolist()))
    # newton-schulz only, 2 iterations, square
    X = pattern(8, 8, 3, 5, 11, 0.1)
    O = oracle.newton_schulz(X, iters=2)
    cases.append(dict(name="ns_square_8x8_it2", kind="ns", iters=2, col_blocks=1,
                      X=X.tolist(), O=O.tolist()))
    out = dict(
        note="outputs from the CPU oracle (float64); coefficients (3.4445, -4.7750, 2.0315), eps 1e-7",
        cases=cases)
    with open(os.path.join(HERE, "oracle_small_cases.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
