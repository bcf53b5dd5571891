"""CPU oracle for adaptive block-sparse video attention (FVAttn's routing
frontend and block-sparse attention).  TEST INFRASTRUCTURE ONLY.

This module is the parity reference.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code with the HIP library: it is written directly from the FVAttn
pages (papers.paperslantern.ai/papers/2607.16190) in plain numpy, float64
unless a step's interface fixes another precision, with no blocking, fusion or
reordering beyond what each step's definition states.

Steps and the passages they follow (all on the FVAttn page):
  block_order / reorder / unreorder  section 3.1, video-aware block organization
                                     (reading: raster or Hilbert order over clipped
                                     tiles, raster order inside a tile, tail padding)
  hilbert_index_3d / tile_order      section 3.1 (blocks ordered along a Hilbert
                                     curve), Skilling's transpose method
  pool                               section 3.1, block similarities from pooled Q/K
  block_scores                       section 2 (importance score per head, q-block,
                                     k-block) and section 3.1 (pooled Q/K)
  route                              section 2 (Top-p: the shortest importance-ordered
                                     run of key blocks holding at least a share p of
                                     the row's normalized scores; Top-k floor)
                                     and section 3.1 (Top-p CDF threshold, Top-k floor)
  head_workload                      section 2 (realized per-head workload = number
                                     of selected block pairs)
  sasa_topup                         section 3.3 (extra budget spent in the
                                     importance order produced by routing), one-GPU
                                     per-head form
  rlb_plan / sasa_budget             section 3.2 (one-send-one-receive head
                                     migration, lexicographic objective) and
                                     section 3.3 (slack times the augmentation
                                     coefficient), on virtual ranks
  heaviest_first                     section 3.2 (load balancing on realized
                                     workloads), one-GPU work-queue form
  load_imbalance / trace_unit_busy /  section 2 (load-imbalance factor: largest
  cu_imbalance / slot_imbalance      unit load over the mean unit load), with the
                                     units taken as the GPU's compute units or
                                     resident workgroup slots and a unit's load
                                     as the time it spent on work items
  sparse_attention                   section 2 (attention is computed for the
                                     chosen query-block/key-block pairs and no others)
  sparse_lse / mask_recall           section 2 (the softmax normalizer over the keys
                                     of the selected blocks); recall as the share of
                                     the full softmax mass those keys hold (reading;
                                     block-sparse quality is framed as attention
                                     recall on the DFSAttn abstract listed at
                                     thelatestinai.com/papers/2607.16190)

Every function here is pinned by tests against closed forms, brute force on
tiny inputs, or a library routine for a special case (dense attention).
"""

from __future__ import annotations

import itertools
import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# Video-aware block organization (section 3.1)
# --------------------------------------------------------------------------

def hilbert_index_3d(c0: int, c1: int, c2: int, bits: int) -> int:
    """Index of cell (c0, c1, c2) along the 3-D Hilbert curve of a 2^bits cube,
    by the transpose method of J. Skilling, "Programming the Hilbert curve"
    (AIP Conf. Proc. 707, 2004): from the top bit down, for each lower-bit
    mask either invert the low bits of the first coordinate (bit set) or
    exchange low bits between the first coordinate and this one (bit clear);
    then Gray-encode across coordinates, apply the final correction, and read
    the index by interleaving bits from the top, first coordinate first."""
    x = [int(c0), int(c1), int(c2)]
    top = 1 << (bits - 1)
    q = top
    while q > 1:
        low = q - 1
        for i in range(3):
            if x[i] & q:
                x[0] ^= low
            else:
                swap = (x[0] ^ x[i]) & low
                x[0] ^= swap
                x[i] ^= swap
        q >>= 1
    for i in range(1, 3):
        x[i] ^= x[i - 1]
    corr = 0
    q = top
    while q > 1:
        if x[2] & q:
            corr ^= q - 1
        q >>= 1
    x = [v ^ corr for v in x]
    h = 0
    for j in range(bits - 1, -1, -1):
        for i in range(3):
            h = (h << 1) | ((x[i] >> j) & 1)
    return h


def tile_grid(T, H, W, bt, bh, bw) -> Tuple[int, int, int]:
    return -(-T // bt), -(-H // bh), -(-W // bw)


def tile_order(T, H, W, bt, bh, bw, order: str = "raster") -> List[int]:
    """Tile raster ids (tile-frame, tile-row, tile-column raster numbering) in
    visiting order: 'raster', or 'hilbert' = ascending Hilbert index of the
    tile coordinates on the bounding 2^m cube (cells outside the grid do not
    exist and are skipped)."""
    nt, ny, nx = tile_grid(T, H, W, bt, bh, bw)
    ids = list(range(nt * ny * nx))
    if order == "raster":
        return ids
    if order != "hilbert":
        raise ValueError(order)
    bits = max(1, int(math.ceil(math.log2(max(nt, ny, nx)))))
    key = {i: hilbert_index_3d(i // (ny * nx), (i // nx) % ny, i % nx, bits) for i in ids}
    return sorted(ids, key=lambda i: key[i])


def block_order(T: int, H: int, W: int, bt: int, bh: int, bw: int,
                order: str = "raster") -> np.ndarray:
    """Reordered position r -> source token index, length N = T*H*W.

    Tiles of bt x bh x bw tokens are visited in tile order (raster by default:
    tile t, then tile row, then tile column; or Hilbert); tiles at the grid
    edge are clipped.  Inside a tile the tokens are visited in raster order
    (t, y, x).  Source token index of (t, y, x) is (t*H + y)*W + x.
    """
    nt, ny, nx = tile_grid(T, H, W, bt, bh, bw)
    out: List[np.ndarray] = []
    for tid in tile_order(T, H, W, bt, bh, bw, order):
        t0, y0, x0 = (tid // (ny * nx)) * bt, ((tid // nx) % ny) * bh, (tid % nx) * bw
        ts = np.arange(t0, min(t0 + bt, T))
        ys = np.arange(y0, min(y0 + bh, H))
        xs = np.arange(x0, min(x0 + bw, W))
        tok = (ts[:, None, None] * H + ys[None, :, None]) * W + xs[None, None, :]
        out.append(tok.reshape(-1))
    result = np.concatenate(out).astype(np.int64)
    assert result.shape[0] == T * H * W
    return result


def sizes(T, H, W, bt, bh, bw) -> Tuple[int, int, int, int]:
    """(N, BLK, nB, Npad): tokens, tokens per block, blocks, padded length."""
    N = T * H * W
    BLK = bt * bh * bw
    nB = -(-N // BLK)
    return N, BLK, nB, nB * BLK


def reorder(x: np.ndarray, grid: Sequence[int], block: Sequence[int],
            order: str = "raster") -> np.ndarray:
    """[B, N, Hh, d] -> [B, Hh, Npad, d] in block order, pad rows zero.
    Pure data movement: the dtype is kept."""
    N, BLK, nB, Npad = sizes(*grid, *block)
    B, n, Hh, d = x.shape
    assert n == N
    order = block_order(*grid, *block, order=order)
    y = np.zeros((B, Hh, Npad, d), dtype=x.dtype)
    y[:, :, :N, :] = np.transpose(x[:, order, :, :], (0, 2, 1, 3))
    return y


def unreorder(y: np.ndarray, grid: Sequence[int], block: Sequence[int],
              order: str = "raster") -> np.ndarray:
    """[B, Hh, Npad, d] -> [B, N, Hh, d]; padded rows are dropped."""
    N, BLK, nB, Npad = sizes(*grid, *block)
    B, Hh, npad, d = y.shape
    assert npad == Npad
    order = block_order(*grid, *block, order=order)
    x = np.empty((B, N, Hh, d), dtype=y.dtype)
    x[:, order, :, :] = np.transpose(y[:, :, :N, :], (0, 2, 1, 3))
    return x


# --------------------------------------------------------------------------
# Routing frontend (sections 2 and 3.1)
# --------------------------------------------------------------------------

def pool(xr: np.ndarray, N: int, BLK: int) -> np.ndarray:
    """Mean of each block's real tokens: [B, Hh, Npad, d] -> [B, Hh, nB, d] f64.
    The last block may be partial; its mean is over its real tokens only."""
    B, Hh, Npad, d = xr.shape
    nB = Npad // BLK
    out = np.empty((B, Hh, nB, d), dtype=np.float64)
    for b in range(nB):
        lo, hi = b * BLK, min((b + 1) * BLK, N)
        out[:, :, b, :] = xr[:, :, lo:hi, :].astype(np.float64).sum(axis=2) / (hi - lo)
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """s[b,h,i,j] = (qbar_i . kbar_j) * scale, float64 [B, Hh, nB, nB]."""
    return np.matmul(qbar, np.swapaxes(kbar, -1, -2)) * scale


def scores_f32(S: np.ndarray) -> np.ndarray:
    """The routing interface carries scores as IEEE float32 (round to nearest)."""
    return S.astype(np.float32)


def route_order(S32: np.ndarray) -> np.ndarray:
    """Key-block importance order per row: score descending, ties by key-block
    index ascending.  -0 and +0 compare equal.  NaN scores are rejected."""
    S32 = np.asarray(S32, dtype=np.float32)
    if np.isnan(S32).any():
        raise ValueError("NaN block score")
    nB = S32.shape[-1]
    flat = S32.reshape(-1, nB)
    j = np.broadcast_to(np.arange(nB), flat.shape)
    # lexsort: last key is primary -> primary = -score (desc), secondary = j (asc)
    neg = -(flat.astype(np.float64))
    order = np.lexsort((j, neg), axis=-1)
    return order.reshape(S32.shape)


def route(S32: np.ndarray, top_p: float, topk: int):
    """Top-p CDF cut with a Top-k floor, per (batch, head, query block) row.

    S32: float32 [..., nB, nB] block scores.  top_p is taken at its float32
    value.  For each row, key blocks are put in importance order; the softmax of
    the row's scores is accumulated in that order in float64
    (e_j = exp(s_j - max), C_n = e_1 + ... + e_n in sequence, Z = C_nB) and the
    Top-p set is the shortest prefix with C_n >= p*Z (all blocks when p >= 1,
    none when p <= 0).  The Top-k floor extends it to at least k blocks; the
    union of the two prefixes is the longer one.

    Returns (mask bool [..., nB, nB], counts int64 [..., nB], margin f64 [..., nB])
    where margin is min(|C_n* - pZ|, |C_(n*-1) - pZ|) / Z, the distance of the
    cut from flipping (inf where the cut was not decided by the CDF).
    """
    S32 = np.asarray(S32, dtype=np.float32)
    nB = S32.shape[-1]
    rows = S32.reshape(-1, nB)
    order = route_order(rows)
    p = float(np.float32(top_p))
    R = rows.shape[0]
    counts = np.empty(R, dtype=np.int64)
    margin = np.full(R, np.inf)
    mask = np.zeros((R, nB), dtype=bool)
    for r in range(R):
        s = rows[r, order[r]].astype(np.float64)
        if p >= 1.0:
            nstar = nB
        elif p <= 0.0:
            nstar = 0
        else:
            e = np.exp(s - s[0])
            C = np.cumsum(e)               # sequential, importance order
            Z = C[-1]
            target = p * Z
            nstar = int(np.argmax(C >= target)) + 1
            m = abs(C[nstar - 1] - target)
            if nstar >= 2:
                m = min(m, abs(C[nstar - 2] - target))
            margin[r] = m / Z
        n = min(nB, max(nstar, int(topk)))
        counts[r] = n
        mask[r, order[r, :n]] = True
    return (mask.reshape(S32.shape), counts.reshape(S32.shape[:-1]),
            margin.reshape(S32.shape[:-1]))


def head_workload(mask: np.ndarray) -> np.ndarray:
    """W_h: number of selected (q-block, k-block) pairs per (batch, head)."""
    return mask.reshape(mask.shape[0], mask.shape[1], -1).sum(axis=-1).astype(np.int64)


def sasa_topup(S32: np.ndarray, mask: np.ndarray, budget) -> np.ndarray:
    """One-GPU form of slack-aware augmentation: per head, when its workload
    W_h is below its budget (pairs), add the budget - W_h unselected pairs with
    the highest scores (ties: query block ascending, then key block ascending).
    Heads at or above the budget are unchanged.  `budget` is one number for
    every head (<= 0 disables it) or an array with one budget per (b, h)."""
    out = mask.copy()
    B, Hh, nB, _ = mask.shape
    per_head = np.ndim(budget) > 0
    if not per_head and budget <= 0:
        return out
    ii, jj = np.meshgrid(np.arange(nB), np.arange(nB), indexing="ij")
    for b in range(B):
        for h in range(Hh):
            m = out[b, h]
            bud = int(np.asarray(budget).reshape(-1)[b * Hh + h]) if per_head else int(budget)
            need = bud - int(m.sum())
            if need <= 0:
                continue
            free = ~m
            s = S32[b, h][free].astype(np.float64)
            fi, fj = ii[free], jj[free]
            pick = np.lexsort((fj, fi, -s))[:need]
            m[fi[pick], fj[pick]] = True
    return out


def load_imbalance(loads) -> float:
    """Load-imbalance factor of section 2: the largest unit load divided by the
    mean load over all R units (idle units count with load 0).  1 means
    perfectly balanced; R means one unit carries everything."""
    L = [float(x) for x in loads]
    if not L:
        raise ValueError("no units")
    mean = sum(L) / len(L)
    if mean <= 0.0:
        raise ValueError("total load is zero")
    return max(L) / mean


# Attention trace records: 8 uint32 per processed work item,
#   (row, XCC_ID register, HW_ID register, workgroup id, t0 lo, t0 hi, t1 lo, t1 hi)
# with t0/t1 the item's start and end on the 100 MHz real-time counter.  The
# compute unit that ran the item is named by the XCC_ID register's bits 3:0
# (which XCD) and the HW_ID register's bits 15:8 (CU id bits 11:8, shader array
# bit 12, shader engine bits 15:13, unique inside one XCD).  The HW_ID bits
# below 8 (wave, SIMD, pipe) vary inside one CU and are not part of the name.

def _record_fields(rec):
    r = [int(x) & 0xFFFFFFFF for x in rec]
    unit = ((r[1] & 0xF) << 8) | ((r[2] >> 8) & 0xFF)
    t0 = r[4] | (r[5] << 32)
    t1 = r[6] | (r[7] << 32)
    if t1 < t0:
        raise ValueError("record ends before it starts")
    return unit, t0, t1


def trace_unit_busy(records) -> Dict[int, int]:
    """Busy time of each compute unit seen in the trace: the sum of the
    durations t1 - t0 of the items it ran (ticks), keyed by (xcc << 8) | cu."""
    busy: Dict[int, int] = {}
    for rec in records:
        unit, t0, t1 = _record_fields(rec)
        busy[unit] = busy.get(unit, 0) + (t1 - t0)
    return busy


def cu_imbalance(records, n_units: int) -> float:
    """Per-CU load-imbalance factor of one traced launch: load_imbalance over
    all n_units compute units of the GPU, a unit's load being its busy time
    (CUs that ran nothing count with load 0)."""
    busy = trace_unit_busy(records)
    if len(busy) > n_units:
        raise ValueError("more units in the trace than the GPU has")
    loads = list(busy.values()) + [0] * (n_units - len(busy))
    return load_imbalance(loads)


def slot_imbalance(records, slots: int) -> float:
    """The same factor over the launch's resident workgroup slots: the slowest
    slot finishes when the launch does, so the largest slot load is the span
    max(t1) - min(t0), and the mean slot load is the total item time over the
    number of slots."""
    spans = [_record_fields(rec)[1:] for rec in records]
    span = max(t1 for _, t1 in spans) - min(t0 for t0, _ in spans)
    total = sum(t1 - t0 for t0, t1 in spans)
    if total <= 0:
        raise ValueError("total item time is zero")
    return span * slots / total


def heaviest_first(counts: np.ndarray) -> np.ndarray:
    """Work items (b*Hh + h)*nB + i ordered by row count descending, ties by
    item id ascending."""
    flat = counts.reshape(-1)
    ids = np.arange(flat.shape[0])
    return np.array(sorted(ids.tolist(), key=lambda t: (-int(flat[t]), t)), dtype=np.int64)


# --------------------------------------------------------------------------
# Runtime load balancing on virtual ranks (section 3.2) and slack-aware
# budgets (section 3.3)
# --------------------------------------------------------------------------

def contiguous_placement(nheads: int, ranks: int) -> np.ndarray:
    """Ulysses head placement: head h on rank floor(h * R / nheads)."""
    return np.array([h * ranks // nheads for h in range(nheads)], dtype=np.int64)


def rank_loads(W, rank_of_head, ranks: int) -> np.ndarray:
    """L_r = sum of W_h over the heads on rank r."""
    L = np.zeros(ranks, dtype=np.int64)
    for h, r in enumerate(rank_of_head):
        L[r] += int(W[h])
    return L


def plan_objective(loads) -> Tuple[int, int]:
    """Lexicographic objective of a plan: (critical-path load max_r L_r,
    sum of squared loads).  With the total fixed, the second term orders plans
    by rank-load variance."""
    loads = [int(x) for x in loads]
    return max(loads), sum(x * x for x in loads)


def _involutions(n: int):
    """All involutions of range(n) as mate lists (mate[r] = r for fixed points)."""
    def rec(mate, r):
        while r < n and mate[r] is not None:
            r += 1
        if r == n:
            yield list(mate)
            return
        mate[r] = r
        yield from rec(mate, r + 1)
        for s in range(r + 1, n):
            if mate[s] is None:
                mate[r], mate[s] = s, r
                yield from rec(mate, r + 1)
                mate[s] = None
        mate[r] = None
    yield from rec([None] * n, 0)


def rlb_plans(W, ranks: int, topology: str):
    """Every plan of the topology: (send_to, send_head) per rank, -1 = none.
    A plan is a permutation pi of the ranks; rank r sends one of its heads to
    pi(r).  'pairs': pi an involution (swaps); 'ring': pi(r) = r + 1 mod R with
    every rank sending.  The identity plan is always included."""
    nheads = len(W)
    place = contiguous_placement(nheads, ranks)
    heads = [[h for h in range(nheads) if place[h] == r] for r in range(ranks)]
    yield [-1] * ranks, [-1] * ranks
    if topology == "pairs":
        perms = [m for m in _involutions(ranks) if any(m[r] != r for r in range(ranks))]
    elif topology == "ring":
        perms = [[(r + 1) % ranks for r in range(ranks)]] if ranks >= 2 else []
    else:
        raise ValueError(topology)
    for pi in perms:
        movers = [r for r in range(ranks) if pi[r] != r]
        for choice in itertools.product(*[heads[r] for r in movers]):
            to, hd = [-1] * ranks, [-1] * ranks
            for r, a in zip(movers, choice):
                to[r], hd[r] = pi[r], a
            yield to, hd


def apply_plan(nheads: int, ranks: int, send_to, send_head) -> np.ndarray:
    place = contiguous_placement(nheads, ranks)
    for r in range(ranks):
        if send_to[r] >= 0:
            place[send_head[r]] = send_to[r]
    return place


def rlb_plan(W, ranks: int, topology: str):
    """Brute force over every plan of the topology; the best objective, and
    one plan reaching it.  When no plan lowers the critical path the identity
    is returned (migrating without benefit only costs communication)."""
    nheads = len(W)
    ident = plan_objective(rank_loads(W, contiguous_placement(nheads, ranks), ranks))
    best, best_plan = None, None
    for to, hd in rlb_plans(W, ranks, topology):
        ob = plan_objective(rank_loads(W, apply_plan(nheads, ranks, to, hd), ranks))
        if best is None or ob < best:
            best, best_plan = ob, (to, hd)
    if not best[0] < ident[0]:
        return ident, ([-1] * ranks, [-1] * ranks)
    return best, best_plan


def sasa_budget(W, rank_of_head, ranks: int, alpha: float, head_cap: int) -> np.ndarray:
    """Per-head pair budgets: rank slack s_r = max L - L_r, extra budget
    floor(alpha * s_r) split evenly over the rank's heads in ascending head id
    (remainder to the lowest ids); each head's budget is W_h + its share,
    capped at max(head_cap, W_h)."""
    L = rank_loads(W, rank_of_head, ranks)
    lmax = int(L.max())
    out = np.array([int(x) for x in W], dtype=np.int64)
    for r in range(ranks):
        hs = [h for h in range(len(W)) if rank_of_head[h] == r]
        extra = int(math.floor(float(np.float32(alpha)) * (lmax - int(L[r]))))
        if not hs or extra <= 0:
            continue
        q, rem = divmod(extra, len(hs))
        for k, h in enumerate(hs):
            want = int(W[h]) + q + (1 if k < rem else 0)
            out[h] = min(max(want, int(W[h])), max(head_cap, int(W[h])))
    return out


# --------------------------------------------------------------------------
# Block-sparse attention (section 2: only selected block pairs are evaluated)
# --------------------------------------------------------------------------

def sparse_attention_block(qr, kr, vr, mask_row, N: int, BLK: int, scale: float,
                           qb: int) -> np.ndarray:
    """Output rows of query block qb for one (batch, head).

    qr, kr, vr: [Npad, d] arrays of that head in block order.  mask_row: bool
    [nB] selected key blocks.  Keys are the real tokens (position < N) of the
    selected blocks in ascending block order; two-pass softmax over them in
    float64.  Returns [n_real_rows, d] float64; zeros when nothing is selected.
    """
    lo, hi = qb * BLK, min((qb + 1) * BLK, N)
    q = qr[lo:hi].astype(np.float64)
    sel = np.nonzero(mask_row)[0]
    if sel.size == 0:
        return np.zeros((hi - lo, qr.shape[1]), dtype=np.float64)
    keys = np.concatenate([np.arange(j * BLK, min((j + 1) * BLK, N)) for j in sel])
    k = kr[keys].astype(np.float64)
    v = vr[keys].astype(np.float64)
    logits = (q @ k.T) * scale
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return (e @ v) / e.sum(axis=1, keepdims=True)


def sparse_attention(qr, kr, vr, mask, N: int, BLK: int, scale: float,
                     items: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Block-sparse attention over reordered tensors [B, Hh, Npad, d].

    With items=None returns the full [B, Hh, Npad, d] float64 output (pad rows
    zero).  With a list of (b, h, qb) returns {item: [rows, d] float64}."""
    B, Hh, Npad, d = qr.shape
    nB = Npad // BLK
    if items is None:
        out = np.zeros((B, Hh, Npad, d), dtype=np.float64)
        for b in range(B):
            for h in range(Hh):
                for i in range(nB):
                    lo, hi = i * BLK, min((i + 1) * BLK, N)
                    out[b, h, lo:hi] = sparse_attention_block(
                        qr[b, h], kr[b, h], vr[b, h], mask[b, h, i], N, BLK, scale, i)
        return out
    res = {}
    for (b, h, i) in items:
        res[(b, h, i)] = sparse_attention_block(qr[b, h], kr[b, h], vr[b, h],
                                                mask[b, h, i], N, BLK, scale, i)
    return res


def _selected_keys(mask_row, N: int, BLK: int) -> np.ndarray:
    sel = np.nonzero(mask_row)[0]
    if sel.size == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(j * BLK, min((j + 1) * BLK, N)) for j in sel])


def sparse_lse_block(qr, kr, mask_row, N: int, BLK: int, scale: float, qb: int) -> np.ndarray:
    """Natural log-sum-exp of the scaled scores of query block qb's real rows
    over the keys block-sparse attention uses for them (real tokens of the
    selected key blocks): lse_i = log sum_k exp(scale * q_i . k), float64
    [n_real_rows]; -inf for every row when nothing is selected."""
    lo, hi = qb * BLK, min((qb + 1) * BLK, N)
    keys = _selected_keys(mask_row, N, BLK)
    if keys.size == 0:
        return np.full(hi - lo, -np.inf)
    logits = (qr[lo:hi].astype(np.float64) @ kr[keys].astype(np.float64).T) * scale
    m = logits.max(axis=1)
    return m + np.log(np.exp(logits - m[:, None]).sum(axis=1))


def sparse_lse(qr, kr, mask, N: int, BLK: int, scale: float) -> np.ndarray:
    """sparse_lse_block over every (batch, head, query block): [B, Hh, N] f64,
    indexed by reordered query position."""
    B, Hh, Npad, _ = qr.shape
    nB = Npad // BLK
    out = np.empty((B, Hh, N), dtype=np.float64)
    for b in range(B):
        for h in range(Hh):
            for i in range(nB):
                out[b, h, i * BLK:min((i + 1) * BLK, N)] = sparse_lse_block(
                    qr[b, h], kr[b, h], mask[b, h, i], N, BLK, scale, i)
    return out


def mask_recall(lse_selected, lse_all) -> np.ndarray:
    """Share of each query's full softmax mass that its selected keys hold:
    sum_{k selected} exp(s_k) / sum_{all k} exp(s_k) = exp(lse_sel - lse_all)."""
    return np.exp(np.asarray(lse_selected, np.float64) - np.asarray(lse_all, np.float64))


# --------------------------------------------------------------------------
# Whole path
# --------------------------------------------------------------------------

def route_path(qr, kr, N, BLK, scale, top_p, topk, aug_budget=0) -> Dict[str, np.ndarray]:
    """pool -> scores -> float32 -> Top-p/Top-k route -> optional top-up ->
    workloads and heaviest-first queue."""
    qbar = pool(qr, N, BLK)
    kbar = pool(kr, N, BLK)
    S = block_scores(qbar, kbar, scale)
    S32 = scores_f32(S)
    mask, counts, margin = route(S32, top_p, topk)
    mask_aug = sasa_topup(S32, mask, aug_budget)
    counts_aug = mask_aug.sum(axis=-1).astype(np.int64)
    return dict(qbar=qbar, kbar=kbar, scores=S, scores32=S32, mask_routed=mask,
                counts_routed=counts, margin=margin, mask=mask_aug, counts=counts_aug,
                head_count=head_workload(mask_aug), queue=heaviest_first(counts_aug))


def forward(q, k, v, grid, block, top_p, topk, aug_budget=0, scale=None, order="raster"):
    """Full path on [B, N, Hh, d] inputs; returns (O [B, N, Hh, d] f64, route dict)."""
    N, BLK, nB, Npad = sizes(*grid, *block)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qr, kr, vr = (reorder(x, grid, block, order) for x in (q, k, v))
    r = route_path(qr, kr, N, BLK, scale, top_p, topk, aug_budget)
    orr = sparse_attention(qr, kr, vr, r["mask"], N, BLK, scale)
    return unreorder(orr, grid, block, order), r
