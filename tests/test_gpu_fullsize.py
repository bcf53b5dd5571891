"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (XCD schedule), against the float64 oracle.

For every full workload:
  * masks, counts, column lists, workloads and the heaviest-first queue are
    bit-exact for ALL rows when the GPU routes from the oracle's float32 scores;
  * from the GPU's own pooled scores at least 99 % of rows agree and every
    differing row is a near-tie of the cut in the oracle;
  * attention output on a sample of query blocks (heaviest, lightest, the
    ragged last block of a head, seeded random ones) is within max-abs 2e-2
    and mean-relative 5e-3 of the oracle, computed block by block;
  * the dense comparator's output on the same blocks is within the same bounds
    of the oracle with every block selected;
  * on the same blocks the sparse and dense per-query log-sum-exp are within
    5e-3 of the oracle and the mask recall exp(lse_sparse - lse_dense) within
    1e-2 (bf16-rounded probabilities are summed, each within 2^-9 relative).
"""

import numpy as np
import pytest
import torch

from adaptive_block_sparse_reorder_amd import fva as F
from adaptive_block_sparse_reorder_amd.inputs import WORKLOADS, make_qkv, small_workload
from oracle import fva_oracle as O

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_REL = 5e-3
LSE_ABS = 5e-3
RECALL_ABS = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    F.load_library()


def unpack_bitmask(bm, nB):
    b = bm.detach().cpu().numpy().view(np.uint32)
    bits = np.unpackbits(b.view(np.uint8).reshape(b.shape[0], -1), axis=1, bitorder="little")
    return bits[:, :nB].astype(bool)


def run_case(w, n_random=12):
    print(f"\n[{w.name}] generating", flush=True)
    q, k, v = make_qkv(w)
    buf = F.alloc_buffers(w.grid, w.block, w.B, w.Hh, w.d)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    print(f"[{w.name}] GPU path (own scores)", flush=True)
    F.forward(buf, qd, kd, vd, w.top_p, w.topk_floor, w.aug_budget,
              attn_flags=F.FVA_SCHED_XCD)
    torch.cuda.synchronize()
    own_mask = unpack_bitmask(buf.bitmask, w.nB)
    own_scores = buf.scores.cpu().numpy()

    print(f"[{w.name}] oracle routing", flush=True)
    qr = O.reorder(q.float().numpy(), w.grid, w.block)
    kr = O.reorder(k.float().numpy(), w.grid, w.block)
    vr = O.reorder(v.float().numpy(), w.grid, w.block)
    r = O.route_path(qr, kr, w.N, w.BLK, w.scale, w.top_p, w.topk_floor, w.aug_budget)
    ref_mask = r["mask"].reshape(-1, w.nB)

    # scores close to the oracle's, masks agree except at near-ties
    tol = 1e-5 * max(1.0, float(np.abs(r["scores"]).max()))
    delta = float(np.abs(own_scores.reshape(r["scores"].shape) - r["scores"]).max())
    assert delta <= tol
    differ = (own_mask != ref_mask).any(axis=1)
    print(f"[{w.name}] own-score mask agreement {1 - differ.mean():.5f} "
          f"({int(differ.sum())} rows, max score deviation {delta:.2e})", flush=True)
    assert differ.mean() <= 0.01
    if w.aug_budget == 0:
        # a differing row is a near-tie: either the same count with a boundary
        # score gap within the score deviation (order swap), or a cut within
        # a small CDF margin (count flip)
        S32 = r["scores32"].reshape(-1, w.nB)
        ref_counts = ref_mask.sum(axis=1)
        margin = r["margin"].reshape(-1)
        for row in np.nonzero(differ)[0]:
            n = int(ref_counts[row])
            srt = S32[row, O.route_order(S32[row][None, :])[0]].astype(np.float64)
            lo, hi = max(1, n - 2), min(w.nB - 1, n + 1)
            gap = float(np.min(srt[lo - 1:hi] - srt[lo:hi + 1]))
            assert margin[row] < 1e-4 or gap <= 2 * delta + 1e-7, (row, margin[row], gap, delta)

    print(f"[{w.name}] GPU route from oracle scores", flush=True)
    prm = F.fva_route_params(w.top_p, w.topk_floor, w.aug_budget, 0.0, 0)
    buf.scores.copy_(torch.from_numpy(r["scores32"].reshape(buf.scores.shape)))
    F.fva_route(buf.qr, buf.kr, w.B, w.Hh, w.d, buf.grid, prm, buf.mask(), buf.route_ws,
                buf.sizes.route_ws_bytes, F.FVA_ROUTE_SCORES_IN)
    torch.cuda.synchronize()
    assert np.array_equal(unpack_bitmask(buf.bitmask, w.nB), ref_mask)
    rc = buf.row_count.cpu().numpy()
    assert np.array_equal(rc, r["counts"].reshape(-1))
    ci = buf.col_idx.cpu().numpy()
    for row in np.random.default_rng(1).choice(rc.shape[0], size=256, replace=False):
        assert np.array_equal(ci[row, :rc[row]], np.nonzero(ref_mask[row])[0])
    assert np.array_equal(buf.head_count.cpu().numpy(), r["head_count"].reshape(-1))
    assert np.array_equal(buf.queue.cpu().numpy(), r["queue"])
    if w.aug_budget > 0:
        hc = r["head_count"].reshape(-1)
        routed = r["mask_routed"].reshape(w.B * w.Hh, -1).sum(-1)
        assert np.all(hc == np.maximum(routed, np.minimum(w.aug_budget, w.nB * w.nB)))

    print(f"[{w.name}] attention under every schedule, output prefilled with NaN", flush=True)
    outs = {}
    for fl in (F.FVA_SCHED_QUEUE, F.FVA_SCHED_STATIC, F.FVA_SCHED_GRID):
        buf.orr.fill_(float("nan"))
        F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, buf.grid, buf.mask(),
                          0.0, fl, buf.attn_ws, buf.sizes.attn_ws_bytes)
        torch.cuda.synchronize()
        outs[fl] = buf.orr.clone()
    nq = w.B * w.Hh * w.N
    lse_s = torch.full((nq,), float("nan"), dtype=torch.float32, device="cuda")
    lse_d = torch.full((nq,), float("nan"), dtype=torch.float32, device="cuda")
    buf.orr.fill_(float("nan"))
    F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, buf.grid, buf.mask(),
                      0.0, F.FVA_SCHED_XCD, buf.attn_ws, buf.sizes.attn_ws_bytes, lse=lse_s)
    torch.cuda.synchronize()
    # every real row written (finite), every pad row zero, every schedule bit-identical
    assert bool(torch.isfinite(buf.orr[:, :, :w.N]).all())
    assert not bool(buf.orr[:, :, w.N:].any())
    for fl, o in outs.items():
        assert torch.equal(o.view(torch.int16), buf.orr.view(torch.int16)), fl
    del outs
    assert bool(torch.isfinite(lse_s).all()) or w.topk_floor == 0
    rows = set()
    counts = r["counts"].reshape(-1)
    rows.add(int(np.argmax(counts)))
    rows.add(int(np.argmin(counts)))
    rows.add(w.nB - 1)                                   # ragged last block of head 0
    rows.add((w.B * w.Hh - 1) * w.nB + w.nB - 1)         # ... and of the last head
    rng = np.random.default_rng(7)
    rows.update(int(x) for x in rng.choice(counts.shape[0], size=n_random, replace=False))
    items = [(row // (w.Hh * w.nB), (row // w.nB) % w.Hh, row % w.nB) for row in sorted(rows)]
    ref = O.sparse_attention(qr, kr, vr, r["mask"], w.N, w.BLK, w.scale, items=items)
    got_all = buf.orr
    num = den = mx = 0.0
    for (b, h, i), o_ref in ref.items():
        lo = i * w.BLK
        got = got_all[b, h, lo:lo + o_ref.shape[0]].float().cpu().numpy()
        diff = np.abs(got - o_ref)
        mx = max(mx, float(diff.max()))
        num += float(diff.sum())
        den += float(np.abs(o_ref).sum())
    print(f"[{w.name}] {len(items)} blocks: max_abs={mx:.3e} mean_rel={num / den:.3e}",
          flush=True)
    assert mx <= MAX_ABS and num / den <= MEAN_REL

    print(f"[{w.name}] dense comparator, log-sum-exp and recall on the same blocks", flush=True)
    buf.orr.fill_(float("nan"))
    F.fva_dense_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, buf.grid, lse=lse_d)
    torch.cuda.synchronize()
    # the dense output on the sampled blocks against the oracle with every
    # block selected
    ref_dense = O.sparse_attention(qr, kr, vr, np.ones_like(r["mask"]), w.N, w.BLK, w.scale,
                                   items=items)
    num = den = mx = 0.0
    for (b, h, i), o_ref in ref_dense.items():
        lo = i * w.BLK
        got = buf.orr[b, h, lo:lo + o_ref.shape[0]].float().cpu().numpy()
        diff = np.abs(got - o_ref)
        mx = max(mx, float(diff.max()))
        num += float(diff.sum())
        den += float(np.abs(o_ref).sum())
    print(f"[{w.name}] dense {len(items)} blocks: max_abs={mx:.3e} mean_rel={num / den:.3e}",
          flush=True)
    assert mx <= MAX_ABS and num / den <= MEAN_REL
    gs = lse_s.cpu().numpy().astype(np.float64).reshape(w.B, w.Hh, w.N)
    gd = lse_d.cpu().numpy().astype(np.float64).reshape(w.B, w.Hh, w.N)
    full_row = np.ones(w.nB, dtype=bool)
    e_lse = e_rec = 0.0
    for (b, h, i) in items:
        lo, hi = i * w.BLK, min((i + 1) * w.BLK, w.N)
        ref_s = O.sparse_lse_block(qr[b, h], kr[b, h], r["mask"][b, h, i], w.N, w.BLK, w.scale, i)
        ref_d = O.sparse_lse_block(qr[b, h], kr[b, h], full_row, w.N, w.BLK, w.scale, i)
        fin = np.isfinite(ref_s)
        assert np.array_equal(np.isfinite(gs[b, h, lo:hi]), fin)
        if fin.any():
            e_lse = max(e_lse, float(np.abs(gs[b, h, lo:hi][fin] - ref_s[fin]).max()))
        e_lse = max(e_lse, float(np.abs(gd[b, h, lo:hi] - ref_d).max()))
        rec = O.mask_recall(gs[b, h, lo:hi], gd[b, h, lo:hi])
        e_rec = max(e_rec, float(np.abs(rec - O.mask_recall(ref_s, ref_d)).max()))
    print(f"[{w.name}] lse max_abs={e_lse:.2e} recall max_abs={e_rec:.2e}", flush=True)
    assert e_lse <= LSE_ABS and e_rec <= RECALL_ABS
    return r


@pytest.mark.parametrize("name", ["480p", "720p", "hetero", "long720p"])
def test_full_workload(name):
    run_case(WORKLOADS[name])


def test_largest_supported_block_count():
    # nB = 2048 blocks per head: the routing sort, queue and column lists at their maximum
    w = small_workload("max-nB", 2, 64, (16, 128, 128), (1, 8, 16), 0.9, 4, aug_budget=300000)
    assert w.nB == 2048
    run_case(w, n_random=6)


def test_rows_of_more_than_2048_blocks():
    # nB = 4100: routing takes one 1024-thread workgroup per row (four blocks
    # per thread); the near-uniform head keeps about 90 % of the blocks, so
    # attention walks column lists of more than 2048 entries in LDS chunks;
    # the top-up rewrites rows of 129 bitmask words
    w = small_workload("wide-nB", 2, 64, (4, 64, 1025), (1, 8, 8), 0.9, 4,
                       aug_budget=int(0.3 * 4100 * 4100), amp=(0.2, 3.0))
    assert w.nB == 4100
    r = run_case(w, n_random=6)
    counts = r["counts"].reshape(-1)
    assert counts.max() > 2048 and counts.min() < 2048


@pytest.mark.parametrize("top_p,topk", [(0.9, 4), (0.0, 5000), (1.0, 0), (0.5, 9000)])
def test_route_of_the_widest_rows_sampled(top_p, topk):
    # nB = 17000 (16 or more blocks per thread of the row's workgroup): route
    # from seeded float32 scores with many ties and signed zeros; sampled rows
    # bit for bit against the oracle, every count and W_h, a valid queue
    grid = F.make_grid((1, 1, 17000 * 64), (1, 1, 64))
    sz = F.fva_sizes(grid, 1, 1, 64)
    nB, rows = int(sz.nB), int(sz.rows)
    assert nB == 17000
    gen = torch.Generator(device="cuda").manual_seed(5)
    S = torch.randn((rows, nB), device="cuda", generator=gen) * 4.0
    S = torch.round(S * 16.0) / 16.0                   # many ties
    S[S == 0] = -0.0                                    # signed zeros among them
    S[::7, ::5] = 0.0
    bitmask = torch.empty((rows, int(sz.words)), dtype=torch.int32, device="cuda")
    row_count = torch.empty(rows, dtype=torch.int32, device="cuda")
    col_idx = torch.empty((rows, nB), dtype=torch.int16, device="cuda")
    head_count = torch.empty(1, dtype=torch.int32, device="cuda")
    queue = torch.empty(rows, dtype=torch.int32, device="cuda")
    ws = torch.zeros((int(sz.route_ws_bytes) + 7) // 8, dtype=torch.int64, device="cuda")
    m = F.fva_mask(S.data_ptr(), bitmask.data_ptr(), row_count.data_ptr(), col_idx.data_ptr(),
                   head_count.data_ptr(), queue.data_ptr())
    prm = F.fva_route_params(top_p, topk, 0, 0.0, 0)
    F.fva_route(None, None, 1, 1, 64, grid, prm, m, ws, int(sz.route_ws_bytes),
                F.FVA_ROUTE_SCORES_IN)
    torch.cuda.synchronize()
    rc = row_count.cpu().numpy()
    assert int(head_count.item()) == int(rc.sum())
    q = queue.cpu().numpy()
    assert np.array_equal(np.sort(q), np.arange(rows))
    assert np.array_equal(q, O.heaviest_first(rc.reshape(1, 1, -1).astype(np.int64)))
    sample = np.random.default_rng(3).choice(rows, size=24, replace=False)
    S32 = S[torch.from_numpy(sample).cuda()].cpu().numpy()
    mask, counts, _ = O.route(S32, top_p, topk)
    got = unpack_bitmask(bitmask[torch.from_numpy(sample).cuda()], nB)
    assert np.array_equal(got, mask)
    assert np.array_equal(rc[sample], counts)
    ci = col_idx[torch.from_numpy(sample).cuda()].cpu().numpy()
    for k in range(len(sample)):
        assert np.array_equal(ci[k, :counts[k]], np.nonzero(mask[k])[0])


@pytest.mark.parametrize("name", ["720p", "hetero"])
def test_per_cu_imbalance_target_at_full_size(name):
    # the balance target on one GPU: under the XCD schedule the traced launch's
    # per-CU load-imbalance factor (max over mean busy time over all CUs, the
    # oracle's definition) is at most 1.10, and so is the per-slot factor;
    # the fixed contiguous split is shown beside it for scale
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    buf = F.alloc_buffers(w.grid, w.block, w.B, w.Hh, w.d, trace=True)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    F.forward(buf, qd, kd, vd, w.top_p, w.topk_floor, w.aug_budget, attn_flags=F.FVA_SCHED_XCD)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = int(buf.sizes.rows)
    lam = {}
    for fl in (F.FVA_SCHED_STATIC, F.FVA_SCHED_XCD):
        buf.trace.zero_()
        F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, buf.grid, buf.mask(),
                          0.0, fl | F.FVA_TRACE, buf.attn_ws, buf.sizes.attn_ws_bytes, buf.trace)
        torch.cuda.synchronize()
        recs = buf.trace.cpu().numpy().view(np.uint32).reshape(-1, 8)[:rows].tolist()
        assert sorted(r[0] for r in recs) == list(range(rows))      # every item traced once
        slots = len({r[3] for r in recs})                           # resident workgroups used
        lam[fl] = (O.cu_imbalance(recs, cus), O.slot_imbalance(recs, slots))
    print(f"[{name}] lambda_cu static {lam[F.FVA_SCHED_STATIC][0]:.3f} -> XCD "
          f"{lam[F.FVA_SCHED_XCD][0]:.3f}; lambda_slot {lam[F.FVA_SCHED_STATIC][1]:.3f} -> "
          f"{lam[F.FVA_SCHED_XCD][1]:.3f}", flush=True)
    assert lam[F.FVA_SCHED_XCD][0] <= 1.10
    assert lam[F.FVA_SCHED_XCD][1] <= 1.10
