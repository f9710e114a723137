"""Host placement of whole matrices on data-parallel ranks (muon_place):
round robin against longest-processing-time-first, pinned by brute-force
optimal partitions on small instances and by Graham's bound for LPT,
makespan <= (4/3 - 1/(3R)) * optimum."""
import itertools
import math
import random

import pytest

import muon_newton_schulz_03_amd as mu


def brute_opt(costs, ranks):
    """Smallest achievable maximum rank load, by enumerating every owner map."""
    best = math.inf
    for owners in itertools.product(range(ranks), repeat=len(costs)):
        load = [0.0] * ranks
        for c, r in zip(costs, owners):
            load[r] += c
        best = min(best, max(load))
    return best


def test_round_robin_assignment():
    owner, load, imb = mu.muon_place([1, 2, 3, 4, 5, 6, 7], 3, "rr")
    assert owner == [0, 1, 2, 0, 1, 2, 0]
    assert load == [12.0, 7.0, 9.0]
    assert imb == pytest.approx(12.0 / (28.0 / 3))


def test_lpt_classic_worst_case():
    # Graham's tight example for R = 3: LPT 11, optimum 9 (5+4, 5+4, 3+3+3)
    costs = [5, 5, 4, 4, 3, 3, 3]
    owner, load, imb = mu.muon_place(costs, 3, "lpt")
    assert owner == [0, 1, 2, 2, 0, 1, 0]
    assert load == [11.0, 8.0, 8.0]
    assert brute_opt(costs, 3) == 9
    assert max(load) / 9 == pytest.approx(4 / 3 - 1 / 9)


def test_lpt_within_graham_bound_and_consistent():
    rng = random.Random(7)
    for _ in range(60):
        ranks = rng.randint(1, 3)
        costs = [rng.choice([0, 1, 2, 3, 5, 8, 13]) for _ in range(rng.randint(0, 8))]
        owner, load, imb = mu.muon_place(costs, ranks, "lpt")
        assert all(0 <= o < ranks for o in owner)
        got = [0.0] * ranks
        for c, o in zip(costs, owner):
            got[o] += c
        assert got == load
        if sum(costs) > 0:
            opt = brute_opt(costs, ranks)
            assert max(load) <= (4 / 3 - 1 / (3 * ranks)) * opt + 1e-12
            assert imb == pytest.approx(max(load) / (sum(costs) / ranks))
        else:
            assert imb == 1.0


def test_ties_break_toward_lower_index_and_rank():
    owner, load, _ = mu.muon_place([2, 2, 2, 2], 2, "lpt")
    assert owner == [0, 1, 0, 1]
    owner, _, _ = mu.muon_place([1, 3, 3, 1], 2, "lpt")
    assert owner == [0, 0, 1, 1]  # order 1, 2 (cost 3), then 0, 3 (cost 1)


def test_cost_estimates_beat_round_robin_on_mixed_shapes():
    """The pages expect estimated costs to place better than round robin:
    one Qwen3-30B-A3B-shaped block (q, k, v, o and 128 experts) with the
    planner's cost model, over 8 ranks."""
    from muon_newton_schulz_03_amd.workloads import WORKLOADS
    shapes = WORKLOADS["qwen3_block"].shapes
    costs = []
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        costs.append(5 * (4 * m * m * n + 2 * m ** 3))
    _, load_rr, imb_rr = mu.muon_place(costs, 8, "rr")
    _, load_lpt, imb_lpt = mu.muon_place(costs, 8, "lpt")
    assert imb_lpt < imb_rr
    assert max(load_lpt) >= sum(costs) / 8


def test_invalid_arguments():
    with pytest.raises(mu.MuonError):
        mu.muon_place([1.0], 0)
    with pytest.raises(mu.MuonError):
        mu.muon_place([1.0, -1.0], 2)
    with pytest.raises(mu.MuonError):
        mu.muon_place([float("nan")], 2)
    with pytest.raises(mu.MuonError):
        mu.muon_place([1.0], 2, policy=7)
