"""Load balancing on virtual ranks and slack-aware budgets: the oracle's brute
force pinned on hand-worked cases and invariants, and the library's host
planner (C ABI, no GPU) checked against it."""

import itertools
import json
import os
import random

import numpy as np
import pytest

from adaptive_block_sparse_reorder_amd import fva as F
from oracle import fva_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
TOPO = {"pairs": F.FVA_RLB_PAIRS, "ring": F.FVA_RLB_RING}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(F.LIB_PATH):
        from adaptive_block_sparse_reorder_amd import build
        build.build(verbose=False)
    return F.load_library()


def _check_plan_valid(W, R, topology, to, hd):
    place = O.contiguous_placement(len(W), R)
    senders = [r for r in range(R) if to[r] >= 0]
    receivers = [to[r] for r in senders]
    assert sorted(senders) == sorted(receivers)           # every mover sends and receives one
    assert len(set(receivers)) == len(receivers)
    for r in senders:
        assert to[r] != r and place[hd[r]] == r              # sends one of its own heads
        if topology == "pairs":
            assert to[to[r]] == r                            # swaps
        else:
            assert to[r] == (r + 1) % R


def test_rlb_worked_examples(lib):
    g = json.load(open(os.path.join(GOLD, "rlb_worked.json")))
    for c in g["cases"]:
        for topo in ("pairs", "ring"):
            (mx, sq), (to, hd) = O.rlb_plan(c["W"], c["ranks"], topo)
            before = O.plan_objective(O.rank_loads(c["W"], O.contiguous_placement(len(c["W"]), c["ranks"]), c["ranks"]))
            assert before[0] == c["max_before"]
            if topo == "pairs" or c["ranks"] == 2:
                assert (mx, sq) == (c["max_after"], c["sumsq_after"]), (c, topo)
                assert sum(1 for t in to if t >= 0) == c["migrations"]
            cto, chd, roh, st = F.fva_rlb_plan(c["W"], c["ranks"], TOPO[topo])
            loads = O.rank_loads(c["W"], roh, c["ranks"])
            assert O.plan_objective(loads) == (mx, sq), (c, topo)
            assert st.max_before == c["max_before"] and st.max_after == mx
            assert st.lambda_before == pytest.approx(c["max_before"] * c["ranks"] / sum(c["W"]))


def test_oracle_invariants():
    rng = random.Random(1)
    for _ in range(40):
        R = rng.randint(2, 5)
        W = [rng.randint(0, 50) for _ in range(R * rng.randint(1, 3))]
        for topo in ("pairs", "ring"):
            (mx, sq), (to, hd) = O.rlb_plan(W, R, topo)
            _check_plan_valid(W, R, topo, to, hd)
            place = O.apply_plan(len(W), R, to, hd)
            L = O.rank_loads(W, place, R)
            assert L.sum() == sum(W)
            assert (int(L.max()), int((L * L).sum())) == (mx, sq)
            L0 = O.rank_loads(W, O.contiguous_placement(len(W), R), R)
            assert mx <= L0.max()
            # no plan of the topology is strictly better (re-check by enumeration)
            for t2, h2 in O.rlb_plans(W, R, topo):
                ob = O.plan_objective(O.rank_loads(W, O.apply_plan(len(W), R, t2, h2), R))
                if ob[0] < L0.max():
                    assert (mx, sq) <= ob


@pytest.mark.parametrize("topo", ["pairs", "ring"])
def test_planner_matches_bruteforce(lib, topo):
    rng = random.Random(2 if topo == "pairs" else 3)
    for trial in range(60):
        R = rng.randint(2, 6)
        per = rng.randint(1, 3)
        W = [rng.choice([rng.randint(0, 20), rng.randint(50, 400)]) for _ in range(R * per)]
        best, _ = O.rlb_plan(W, R, topo)
        to, hd, roh, st = F.fva_rlb_plan(W, R, TOPO[topo])
        _check_plan_valid(W, R, topo, to, hd)
        assert list(roh) == list(O.apply_plan(len(W), R, to, hd))
        assert O.plan_objective(O.rank_loads(W, roh, R)) == best, (W, R)
        assert st.max_after == best[0]
        assert st.migrations == sum(1 for t in to if t >= 0)


def test_planner_eight_ranks_bruteforce(lib):
    # the pages' default: 8 ranks; two heads per rank keeps brute force small
    rng = random.Random(4)
    for trial in range(6):
        W = [rng.randint(100, 5000) for _ in range(16)]
        for topo in ("pairs", "ring"):
            best, _ = O.rlb_plan(W, 8, topo)
            to, hd, roh, st = F.fva_rlb_plan(W, 8, TOPO[topo])
            assert O.plan_objective(O.rank_loads(W, roh, 8)) == best


def test_planner_forty_heads_is_fast_and_valid(lib):
    # 40 heads on 8 ranks (5 each): plans are valid, never worse than no
    # migration, and the search stays within a millisecond
    rng = np.random.default_rng(5)
    for _ in range(5):
        W = (rng.uniform(0.1, 0.95, size=40) * 591 * 591).astype(int).tolist()
        for topo in ("pairs", "ring"):
            to, hd, roh, st = F.fva_rlb_plan(W, 8, TOPO[topo])
            _check_plan_valid(W, 8, topo, to, hd)
            assert st.lambda_after <= st.lambda_before
            assert st.solve_us < 50000


def test_planner_rejects_bad_arguments(lib):
    with pytest.raises(F.FvaError):
        F.fva_rlb_plan([1, 2, 3], 4)                         # more ranks than heads
    with pytest.raises(F.FvaError):
        F.fva_rlb_plan([1] * 26, 13, F.FVA_RLB_PAIRS)        # pair search size cap
    with pytest.raises(F.FvaError):
        F.fva_rlb_plan([1, -1], 1)


def test_sasa_budget_worked_and_random(lib):
    # loads after balancing 11 and 10 (heads [10,1] and [9,1] on ranks 0,1):
    # slack of rank 1 = 1, alpha 1 -> one extra pair to its lower head id
    W, roh = [10, 1, 9, 1], [0, 0, 1, 1]
    hb = O.sasa_budget(W, roh, 2, 1.0, 1000)
    assert hb.tolist() == [10, 1, 10, 1]
    hb2, rl = F.fva_sasa_budget(W, 2, roh, 1.0, 1000)
    assert hb2 == hb.tolist() and rl == [11, 11]
    rng = random.Random(6)
    for _ in range(100):
        R = rng.randint(1, 6)
        W = [rng.randint(0, 300) for _ in range(R * rng.randint(1, 4))]
        roh = [rng.randrange(R) for _ in W]
        alpha = rng.choice([0.0, 0.25, 0.5, 0.8, 1.0])
        cap = rng.choice([50, 300, 10 ** 6])
        ref = O.sasa_budget(W, roh, R, alpha, cap)
        got, rl = F.fva_sasa_budget(W, R, roh, alpha, cap)
        assert got == ref.tolist(), (W, roh, alpha, cap)
        # the budgeted loads never exceed the critical path
        L = O.rank_loads(W, roh, R)
        assert max(rl) <= max(L.max(), 0) or cap < max(W)
