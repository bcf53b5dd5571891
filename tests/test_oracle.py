"""Pins for the CPU oracle: closed forms, hand-worked fixtures, brute force on
tiny inputs and reduction to a library routine (dense attention).  None of
these tests re-types the oracle's own formulas."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import fva_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- reorder

def test_block_order_golden():
    g = _load("block_order_T2H3W5_b1x2x2.json")
    got = O.block_order(*g["grid"], *g["block"])
    assert got.tolist() == g["order"]


@pytest.mark.parametrize("grid,block", [
    ((5, 16, 16), (1, 8, 8)), ((3, 13, 19), (1, 8, 8)), ((21, 30, 52), (1, 8, 16)),
    ((3, 7, 11), (2, 4, 4)), ((1, 1, 1), (1, 8, 8)), ((4, 9, 10), (3, 8, 8))])
def test_block_order_is_bijection(grid, block):
    o = O.block_order(*grid, *block)
    N = grid[0] * grid[1] * grid[2]
    assert o.shape == (N,)
    assert np.array_equal(np.sort(o), np.arange(N))


def test_block_order_exact_tiling_closed_form():
    # 5x16x16 grid, 1x8x8 tiles: block b is tile (t=b//4, ty=(b//2)%2, tx=b%2)
    o = O.block_order(5, 16, 16, 1, 8, 8)
    for b in range(20):
        t, ty, tx = b // 4, (b // 2) % 2, b % 2
        want = [(t * 16 + ty * 8 + y) * 16 + tx * 8 + x for y in range(8) for x in range(8)]
        assert o[b * 64:(b + 1) * 64].tolist() == want


def test_block_order_tokens_stay_in_their_tile():
    # every token of a tile is contiguous in the order, and the tile's tokens
    # are exactly the clipped box
    T, H, W, bt, bh, bw = 3, 7, 11, 2, 4, 4
    o = O.block_order(T, H, W, bt, bh, bw)
    pos = 0
    for t0 in range(0, T, bt):
        for y0 in range(0, H, bh):
            for x0 in range(0, W, bw):
                box = {(t * H + y) * W + x for t in range(t0, min(t0 + bt, T))
                       for y in range(y0, min(y0 + bh, H)) for x in range(x0, min(x0 + bw, W))}
                seg = o[pos:pos + len(box)].tolist()
                assert set(seg) == box and seg == sorted(seg)
                pos += len(box)
    assert pos == T * H * W


def test_reorder_roundtrip_and_padding():
    grid, block = (3, 13, 19), (1, 8, 8)
    N, BLK, nB, Npad = O.sizes(*grid, *block)
    assert (N, BLK, nB, Npad) == (741, 64, 12, 768)
    x = np.random.default_rng(0).standard_normal((2, N, 3, 16)).astype(np.float32)
    y = O.reorder(x, grid, block)
    assert y.shape == (2, 3, Npad, 16)
    assert np.all(y[:, :, N:, :] == 0)
    assert np.array_equal(O.unreorder(y, grid, block), x)
    # position r of the reordered tensor holds token block_order[r]
    o = O.block_order(*grid, *block)
    assert np.array_equal(y[1, 2, 100], x[1, o[100], 2])


# ----------------------------------------------------------------- pooling

def test_pool_constant_and_ramp_closed_forms():
    grid, block = (5, 16, 16), (1, 8, 8)
    N, BLK, nB, Npad = O.sizes(*grid, *block)
    x = np.zeros((1, N, 1, 2), dtype=np.float32)
    x[0, :, 0, 0] = 3.25
    x[0, :, 0, 1] = np.arange(N)            # token index ramp
    p = O.pool(O.reorder(x, grid, block), N, BLK)
    assert np.all(p[0, 0, :, 0] == 3.25)
    for b in range(nB):
        t, ty, tx = b // 4, (b // 2) % 2, b % 2
        want = (t * 16 + ty * 8 + 3.5) * 16 + tx * 8 + 3.5
        assert p[0, 0, b, 1] == pytest.approx(want, abs=1e-9)


def test_pool_partial_last_block_uses_real_tokens_only():
    grid, block = (1, 5, 6), (1, 2, 2)          # N=30, BLK=4 -> 8 blocks, last has 2 tokens
    N, BLK, nB, Npad = O.sizes(*grid, *block)
    assert (nB, Npad) == (8, 32)
    x = np.ones((1, N, 1, 1), dtype=np.float32) * 7.0
    p = O.pool(O.reorder(x, grid, block), N, BLK)
    assert np.all(p == 7.0)                       # padding would drag the last mean to 3.5
    x[0, :, 0, 0] = np.arange(N)
    p = O.pool(O.reorder(x, grid, block), N, BLK)
    # by hand: the last tile row (row 4) holds tiles {24,25}, {26,27}, {28,29};
    # block 7 = reordered positions 28..29 = tokens 28, 29 -> mean 28.5
    order = O.block_order(*grid, *block)
    assert order[-6:].tolist() == [24, 25, 26, 27, 28, 29]
    assert p[0, 0, 7, 0] == 28.5


# ----------------------------------------------------------------- scores

def test_scores_rank_one_closed_form():
    # blocks hold constant vectors a_b*u (queries) and c_b*u (keys):
    # s_ij = a_i c_j |u|^2 * scale; asymmetric a, c catch a transposed operand
    nB, BLK, d = 5, 4, 8
    rng = np.random.default_rng(1)
    u = rng.standard_normal(d)
    a = np.array([1.0, -2.0, 0.5, 3.0, -1.5])
    c = np.array([0.25, 4.0, -1.0, 2.0, 0.0])
    qr = np.repeat(a[:, None] * u[None, :], BLK, axis=0)[None, None]
    kr = np.repeat(c[:, None] * u[None, :], BLK, axis=0)[None, None]
    N = nB * BLK
    S = O.block_scores(O.pool(qr, N, BLK), O.pool(kr, N, BLK), 0.125)
    want = np.outer(a, c) * float(u @ u) * 0.125
    assert np.allclose(S[0, 0], want, rtol=1e-12, atol=1e-12)


def test_scores_f32_is_round_to_nearest():
    x = np.array([[1.0 + 2.0 ** -30, -1.0 / 3.0]])
    assert O.scores_f32(x).dtype == np.float32
    assert O.scores_f32(x)[0, 0] == np.float32(1.0)
    assert O.scores_f32(x)[0, 1] == np.float32(-1.0 / 3.0)


# ----------------------------------------------------------------- routing

def test_route_worked_examples():
    g = _load("route_worked.json")
    for case in g["cases"]:
        s = np.array(case["s"], dtype=np.float32)[None, None, None, :]
        mask, counts, _ = O.route(s, case["p"], case["k"])
        got = np.nonzero(mask[0, 0, 0])[0].tolist()
        assert got == case["selected"], case
        assert counts[0, 0, 0] == len(case["selected"])


def test_route_margin_worked_examples():
    # the cut's distance from flipping, worked by hand in the fixture
    g = _load("route_worked.json")
    for case in g["cases"]:
        s = np.array(case["s"], dtype=np.float32)[None, None, None, :]
        _, _, margin = O.route(s, case["p"], case["k"])
        if case["margin"] is None:
            assert margin[0, 0, 0] == np.inf, case
        else:
            assert margin[0, 0, 0] == pytest.approx(case["margin"], abs=2e-10), case


def test_head_workload_hand_worked():
    # W_h counts the selected (query block, key block) pairs of a head;
    # B = 2, Hh = 2, nB = 3 masks written out by hand
    m = np.zeros((2, 2, 3, 3), dtype=bool)
    m[0, 0] = np.eye(3, dtype=bool)               # 3 pairs, one per row
    m[0, 1] = True                                # all 9 pairs
    m[1, 1, 0, :] = True                          # head (1,0) stays empty
    m[1, 1, 2, 1] = True                          # 3 + 1 pairs
    assert O.head_workload(m).tolist() == [[3, 9], [0, 4]]


def _brute_min_card(s, p):
    """Smallest subset size whose softmax mass reaches p (math.fsum, all subsets)."""
    n = len(s)
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    Z = math.fsum(e)
    best = None
    closest = float("inf")
    for r in range(1, n + 1):
        for sub in itertools.combinations(range(n), r):
            mass = math.fsum(e[j] for j in sub) / Z
            closest = min(closest, abs(mass - p))
            if mass >= p and best is None:
                best = r
    return best, closest


def test_route_bruteforce_minimal_prefix():
    rng = np.random.default_rng(2)
    checked = 0
    for trial in range(120):
        n = int(rng.integers(2, 11))
        s = (rng.standard_normal(n) * rng.uniform(0.2, 3.0)).astype(np.float32)
        p = float(np.float32(rng.uniform(0.05, 0.99)))
        k = int(rng.integers(0, n + 2))
        nmin, closest = _brute_min_card([float(x) for x in s], p)
        if closest < 1e-9:
            continue                                   # too close to call
        mask, counts, margin = O.route(s[None, None, None, :], p, k)
        sel = mask[0, 0, 0]
        want = min(n, max(nmin, k))
        assert sel.sum() == want == counts[0, 0, 0]
        # prefix of the importance order: every kept block beats every dropped one
        for a in np.nonzero(sel)[0]:
            for b in np.nonzero(~sel)[0]:
                assert s[a] > s[b] or (s[a] == s[b] and a < b)
        checked += 1
    assert checked > 100


def test_route_special_cases():
    rng = np.random.default_rng(3)
    S = rng.standard_normal((1, 2, 9, 9)).astype(np.float32)
    # p >= 1 keeps everything, whatever k
    m, c, _ = O.route(S, 1.0, 0)
    assert m.all() and (c == 9).all()
    # k >= nB keeps everything
    m, c, _ = O.route(S, 0.1, 50)
    assert m.all()
    # p -> 0 keeps exactly the k highest scores of each row
    m, c, _ = O.route(S, 1e-12, 3)
    for h in range(2):
        for i in range(9):
            row = S[0, h, i]
            kept = np.nonzero(m[0, h, i])[0]
            assert len(kept) == 3
            # every kept score >= every dropped score (brute pairwise)
            dropped = [j for j in range(9) if j not in kept]
            assert min(row[kept]) >= max(row[dropped])
    # p <= 0 with k = 0 selects nothing
    m, c, _ = O.route(S, 0.0, 0)
    assert not m.any() and (c == 0).all()


def test_route_mass_invariants_random():
    rng = np.random.default_rng(4)
    S = (rng.standard_normal((1, 3, 16, 16)) * 2).astype(np.float32)
    p, k = 0.8, 2
    m, c, margin = O.route(S, p, k)
    for h in range(3):
        for i in range(16):
            s = S[0, h, i].astype(np.float64)
            e = np.exp(s - s.max())
            w = e / math.fsum(e)
            sel = m[0, h, i]
            assert math.fsum(w[sel]) >= p - 1e-12
            assert sel.sum() >= k
            if sel.sum() > k:
                # dropping the weakest kept block falls below p
                kept = np.nonzero(sel)[0]
                weakest = kept[np.lexsort((-kept, s[kept]))[0]]
                assert math.fsum(w[sel]) - w[weakest] < p


def test_route_rejects_nan():
    S = np.zeros((1, 1, 2, 2), dtype=np.float32)
    S[0, 0, 1, 1] = np.nan
    with pytest.raises(ValueError):
        O.route(S, 0.5, 1)


# ----------------------------------------------------------------- top-up

def test_sasa_topup_bruteforce():
    rng = np.random.default_rng(5)
    nB = 6
    for trial in range(20):
        S = rng.integers(-3, 4, size=(1, 2, nB, nB)).astype(np.float32)   # many ties
        mask, _, _ = O.route(S, 0.5, 1)
        budget = int(rng.integers(0, nB * nB + 3))
        out = O.sasa_topup(S, mask, budget)
        for h in range(2):
            W = int(mask[0, h].sum())
            W2 = int(out[0, h].sum())
            assert W2 == max(W, min(budget, nB * nB))
            assert np.all(out[0, h] | ~mask[0, h])              # original kept
            added = [(i, j) for i in range(nB) for j in range(nB)
                     if out[0, h, i, j] and not mask[0, h, i, j]]
            rest = [(i, j) for i in range(nB) for j in range(nB) if not out[0, h, i, j]]
            for (i, j) in added:
                for (a, b) in rest:
                    sa, sb = S[0, h, i, j], S[0, h, a, b]
                    assert sa > sb or (sa == sb and (i, j) < (a, b))


def test_sasa_disabled_and_saturated():
    S = np.random.default_rng(6).standard_normal((1, 1, 4, 4)).astype(np.float32)
    mask, _, _ = O.route(S, 0.5, 1)
    assert np.array_equal(O.sasa_topup(S, mask, 0), mask)
    assert O.sasa_topup(S, mask, 10 ** 6).all()


def test_sasa_budget_cap_hand_worked():
    # contiguous heads [10, 1 | 2, 1] on 2 ranks: loads 11 and 3, so rank 1 has
    # slack 8; alpha 1 gives it 8 extra pairs, 4 per head: wanted 6 and 5
    roh = [0, 0, 1, 1]
    assert O.sasa_budget([10, 1, 2, 1], roh, 2, 1.0, 1000).tolist() == [10, 1, 6, 5]
    # a cap below W_h + share binds: both heads stop at 5
    assert O.sasa_budget([10, 1, 2, 1], roh, 2, 1.0, 5).tolist() == [10, 1, 5, 5]
    # heads [10, 1 | 7, 1]: loads 11 and 8, slack 3 -> shares 2 (lower id) and 1
    assert O.sasa_budget([10, 1, 7, 1], roh, 2, 1.0, 1000).tolist() == [10, 1, 9, 2]
    # a cap below W_h never lowers a head's budget under its own workload
    assert O.sasa_budget([10, 1, 7, 1], roh, 2, 1.0, 5).tolist() == [10, 1, 7, 2]
    # alpha 0.5: floor(1.5) = 1 extra pair, to the lower head id
    assert O.sasa_budget([10, 1, 7, 1], roh, 2, 0.5, 1000).tolist() == [10, 1, 8, 1]


def test_sasa_budget_invariants_when_the_cap_binds():
    rng = np.random.default_rng(9)
    for _ in range(200):
        R = int(rng.integers(1, 6))
        W = [int(x) for x in rng.integers(0, 200, size=R * int(rng.integers(1, 4)))]
        roh = [int(x) for x in rng.integers(0, R, size=len(W))]
        alpha = float(rng.choice([0.25, 0.5, 1.0]))
        cap = int(rng.integers(0, 250))
        hb = O.sasa_budget(W, roh, R, alpha, cap)
        loose = O.sasa_budget(W, roh, R, alpha, 10 ** 9)
        for h in range(len(W)):
            assert hb[h] >= W[h]                           # never below the workload
            assert hb[h] <= max(cap, W[h])                 # never above the cap
            assert hb[h] == max(W[h], min(loose[h], cap))  # the cap only clips


# ----------------------------------------------------------------- imbalance

def _rec(row, xcc, hw, t0, t1):
    return [row, xcc, hw, row, t0 & 0xFFFFFFFF, t0 >> 32, t1 & 0xFFFFFFFF, t1 >> 32]


def test_imbalance_hand_worked_trace():
    # four items on three compute units, times straddling a 32-bit wrap of the
    # counter's low word.  Unit A = XCD 0, CU 3: two items of 30 and 25 ticks
    # (different wave/SIMD bits in HW_ID, junk above bit 3 of XCC_ID); unit B =
    # XCD 1, CU 3: 15 ticks; unit C = XCD 0, CU 3 of shader engine 1 (HW_ID
    # bit 13): 45 ticks.
    base = (1 << 32) - 60
    recs = [_rec(0, 0x30, 0x0325, base, base + 30),
            _rec(1, 0x00, 0x0311, base + 35, base + 60),
            _rec(2, 0x01, 0x0300, base + 2, base + 17),
            _rec(3, 0x00, 0x2300, base + 10, base + 55)]
    assert O.trace_unit_busy(recs) == {0x003: 55, 0x103: 15, 0x023: 45}
    # 4 CUs, one idle: loads 55, 15, 45, 0 -> mean 28.75, factor 55 / 28.75
    assert O.cu_imbalance(recs, 4) == pytest.approx(55 / 28.75, rel=1e-15)
    assert O.cu_imbalance(recs, 3) == pytest.approx(55 / (115 / 3), rel=1e-15)
    # 4 slots: the span (60 ticks) over the mean slot load (115 / 4)
    assert O.slot_imbalance(recs, 4) == pytest.approx(60 * 4 / 115, rel=1e-15)


def test_load_imbalance_rank_form():
    # section 2's factor on ranks: W = [10, 9, 1, 1] on 2 ranks carries 19 and 2
    L = O.rank_loads([10, 9, 1, 1], O.contiguous_placement(4, 2), 2)
    assert O.load_imbalance(L) == pytest.approx(19 / 10.5, rel=1e-15)
    assert O.load_imbalance([7, 7, 7]) == 1.0
    assert O.load_imbalance([12, 0, 0]) == 3.0


# ----------------------------------------------------------------- queue

def test_heaviest_first_order():
    rng = np.random.default_rng(7)
    counts = rng.integers(0, 5, size=(1, 3, 7))
    q = O.heaviest_first(counts)
    flat = counts.reshape(-1)
    assert sorted(q.tolist()) == list(range(21))
    for a, b in zip(q[:-1], q[1:]):
        assert flat[a] > flat[b] or (flat[a] == flat[b] and a < b)


# ----------------------------------------------------------------- attention

def _sdpa64(q, k, v, scale):
    # q, k, v: [B, N, Hh, d] -> dense softmax attention, library routine, float64
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3))))
                  .to(torch.float64) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return np.transpose(o.numpy(), (0, 2, 1, 3))


@pytest.mark.parametrize("grid,block,d", [((3, 13, 19), (1, 8, 8), 16),
                                          ((2, 5, 6), (1, 2, 2), 8)])
def test_all_selected_equals_dense_attention(grid, block, d):
    N = grid[0] * grid[1] * grid[2]
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((1, N, 2, d)).astype(np.float32) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    o, r = O.forward(q, k, v, grid, block, top_p=1.0, topk=0)
    assert r["mask"].all()
    assert np.abs(o - _sdpa64(q, k, v, scale)).max() < 1e-11
    # a large floor instead of p = 1 reaches the same full mask
    o2, r2 = O.forward(q, k, v, grid, block, top_p=0.5, topk=10 ** 6)
    assert np.abs(o2 - o).max() < 1e-12


def test_block_indicator_values_measure_block_mass():
    grid, block = (3, 5, 7), (1, 2, 4)        # N=105, BLK=8, nB=14, ragged tail
    N, BLK, nB, Npad = O.sizes(*grid, *block)
    d = 16
    rng = np.random.default_rng(9)
    qr = np.zeros((1, 1, Npad, d)); kr = np.zeros((1, 1, Npad, d))
    qr[0, 0, :N] = rng.standard_normal((N, d)); kr[0, 0, :N] = rng.standard_normal((N, d))
    vr = np.zeros((1, 1, Npad, d))
    for r in range(N):
        vr[0, 0, r, r // BLK] = 1.0
    mask, _, _ = O.route(O.scores_f32(O.block_scores(O.pool(qr, N, BLK), O.pool(kr, N, BLK), 0.25)), 0.6, 2)
    out = O.sparse_attention(qr, kr, vr, mask, N, BLK, 0.25)
    for i in range(nB):
        lo, hi = i * BLK, min((i + 1) * BLK, N)
        blockmass = out[0, 0, lo:hi, :nB]
        assert np.all(blockmass[:, ~mask[0, 0, i]] == 0.0)
        assert np.all(blockmass[:, mask[0, 0, i]] > 0.0)
        assert np.allclose(blockmass.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(out[0, 0, N:] == 0)


def _lse_case(seed, Hh=2, d=16):
    grid, block = (3, 5, 7), (1, 2, 4)        # N=105, BLK=8, nB=14, ragged tail
    N, BLK, nB, Npad = O.sizes(*grid, *block)
    rng = np.random.default_rng(seed)
    qr = rng.standard_normal((1, Hh, Npad, d))
    kr = 1.5 * rng.standard_normal((1, Hh, Npad, d))   # garbage in the pad rows too
    return N, BLK, nB, Npad, qr, kr, rng


def test_lse_full_mask_equals_library_logsumexp():
    import scipy.special
    N, BLK, nB, Npad, qr, kr, _ = _lse_case(21)
    full = np.ones((1, 2, nB, nB), dtype=bool)
    lse = O.sparse_lse(qr, kr, full, N, BLK, 0.3)
    logits = 0.3 * np.einsum("bhnd,bhmd->bhnm", qr[:, :, :N], kr[:, :, :N])
    ref = scipy.special.logsumexp(logits, axis=-1)
    assert lse.shape == (1, 2, N)
    assert np.abs(lse - ref).max() < 1e-12
    assert np.abs(O.mask_recall(lse, ref) - 1.0).max() < 1e-12


def test_recall_equals_dense_mass_on_selected_blocks():
    # dense attention with block-indicator values gives each query's softmax
    # mass per key block; recall of a mask is the sum over its selected blocks
    N, BLK, nB, Npad, qr, kr, rng = _lse_case(22, Hh=1)
    vr = np.zeros((1, 1, Npad, qr.shape[-1]))                             # d >= nB columns
    for r in range(N):
        vr[0, 0, r, r // BLK] = 1.0
    full = np.ones((1, 1, nB, nB), dtype=bool)
    mass = O.sparse_attention(qr, kr, vr, full, N, BLK, 0.4)[0, 0, :N, :nB]  # [N, nB]
    mask = rng.random((1, 1, nB, nB)) < 0.35
    mask[0, 0, 3] = False                                                  # a row with nothing
    rec = O.mask_recall(O.sparse_lse(qr, kr, mask, N, BLK, 0.4),
                        O.sparse_lse(qr, kr, full, N, BLK, 0.4))[0, 0]
    row_mask = np.repeat(mask[0, 0], BLK, axis=0)[:N]                      # [N, nB]
    expect = (mass * row_mask).sum(axis=1)
    assert np.abs(rec - expect).max() < 1e-12
    assert np.all(rec[3 * BLK:4 * BLK] == 0.0)
    assert np.all(rec <= 1.0 + 1e-12)


def test_lse_is_logaddexp_of_single_block_lses():
    N, BLK, nB, Npad, qr, kr, rng = _lse_case(23, Hh=1)
    mask = rng.random((1, 1, nB, nB)) < 0.5
    mask[..., nB - 1] = True                                               # include the ragged block
    lse = O.sparse_lse(qr, kr, mask, N, BLK, 0.25)[0, 0]
    parts = []
    for j in range(nB):
        one = np.zeros_like(mask)
        one[..., j] = mask[..., j]
        parts.append(O.sparse_lse(qr, kr, one, N, BLK, 0.25)[0, 0])
    assert np.abs(lse - np.logaddexp.reduce(np.stack(parts), axis=0)).max() < 1e-12


def test_zero_queries_average_selected_real_values():
    grid, block = (3, 5, 7), (1, 2, 4)
    N, BLK, nB, Npad = O.sizes(*grid, *block)
    rng = np.random.default_rng(10)
    qr = np.zeros((1, 1, Npad, 4))
    kr = rng.standard_normal((1, 1, Npad, 4))
    vr = rng.standard_normal((1, 1, Npad, 4))        # garbage in the pad rows
    mask = rng.random((1, 1, nB, nB)) < 0.4
    mask[0, 0, :, nB - 1] = True                       # always include the ragged block
    out = O.sparse_attention(qr, kr, vr, mask, N, BLK, 0.5)
    for i in range(nB):
        keys = [r for j in range(nB) if mask[0, 0, i, j]
                for r in range(j * BLK, min((j + 1) * BLK, N))]
        want = vr[0, 0, keys].mean(axis=0)
        lo, hi = i * BLK, min((i + 1) * BLK, N)
        assert np.allclose(out[0, 0, lo:hi], want[None, :], atol=1e-12)


def test_empty_selection_gives_zero_rows():
    grid, block = (1, 4, 4), (1, 2, 2)
    N, BLK, nB, Npad = O.sizes(*grid, *block)
    x = np.random.default_rng(11).standard_normal((1, 1, Npad, 4))
    mask = np.zeros((1, 1, nB, nB), dtype=bool)
    mask[0, 0, 1, 2] = True
    out = O.sparse_attention(x, x, x, mask, N, BLK, 1.0)
    assert np.all(out[0, 0, 0:4] == 0) and np.all(out[0, 0, 8:] == 0)
    assert np.any(out[0, 0, 4:8] != 0)


def test_sparse_output_equals_dense_on_selected_keys_only():
    # one query block, mask picks blocks {0, 2}: equals SDPA over exactly those keys
    grid, block = (1, 4, 8), (1, 2, 4)
    N, BLK, nB, Npad = O.sizes(*grid, *block)
    rng = np.random.default_rng(12)
    qr, kr, vr = (rng.standard_normal((1, 1, Npad, 8)) for _ in range(3))
    mask = np.zeros((1, 1, nB, nB), dtype=bool)
    mask[0, 0, 1, [0, 2]] = True
    out = O.sparse_attention(qr, kr, vr, mask, N, BLK, 0.3)
    keys = list(range(0, 8)) + list(range(16, 24))
    q = torch.from_numpy(qr[0, 0, 8:16])[None, None]
    k = torch.from_numpy(kr[0, 0, keys])[None, None]
    v = torch.from_numpy(vr[0, 0, keys])[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.3)[0, 0].numpy()
    assert np.abs(out[0, 0, 8:16] - ref).max() < 1e-12


# ----------------------------------------------------------------- Hilbert order

@pytest.mark.parametrize("bits", [1, 2, 3])
def test_hilbert_curve_is_a_face_adjacent_walk_of_the_cube(bits):
    n = 1 << bits
    cells = sorted(((t, y, x) for t in range(n) for y in range(n) for x in range(n)),
                   key=lambda c: O.hilbert_index_3d(*c, bits))
    idx = sorted(O.hilbert_index_3d(*c, bits) for c in cells)
    assert idx == list(range(n ** 3))                      # a bijection onto 0..n^3-1
    for a, b in zip(cells[:-1], cells[1:]):
        assert sum(abs(u - v) for u, v in zip(a, b)) == 1  # consecutive cells share a face
    # self-similar: every aligned half-size sub-cube is one contiguous run
    h = n // 2
    if h >= 1:
        for k in range(8):
            run = cells[k * h ** 3:(k + 1) * h ** 3]
            assert len({(c[0] // h, c[1] // h, c[2] // h) for c in run}) == 1


def test_hilbert_tile_order_restricts_the_cube_walk():
    # a 3 x 6 x 5 tile grid inside the 8^3 cube: in-grid cells in cube-walk order
    T, H, W, bt, bh, bw = 3, 48, 80, 1, 8, 16
    nt, ny, nx = O.tile_grid(T, H, W, bt, bh, bw)
    assert (nt, ny, nx) == (3, 6, 5)
    walk = sorted(((t, y, x) for t in range(8) for y in range(8) for x in range(8)),
                  key=lambda c: O.hilbert_index_3d(*c, 3))
    want = [(t * ny + y) * nx + x for (t, y, x) in walk if t < nt and y < ny and x < nx]
    assert O.tile_order(T, H, W, bt, bh, bw, "hilbert") == want
    o = O.block_order(T, H, W, bt, bh, bw, "hilbert")
    assert np.array_equal(np.sort(o), np.arange(T * H * W))


def test_hilbert_reorder_roundtrip_and_dense_equivalence():
    grid, block = (3, 13, 19), (1, 8, 8)
    N = 3 * 13 * 19
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((1, N, 2, 16)).astype(np.float32) for _ in range(3))
    y = O.reorder(q, grid, block, "hilbert")
    assert np.array_equal(O.unreorder(y, grid, block, "hilbert"), q)
    o, _ = O.forward(q, k, v, grid, block, top_p=1.0, topk=0, order="hilbert")
    assert np.abs(o - _sdpa64(q, k, v, 0.25)).max() < 1e-11
