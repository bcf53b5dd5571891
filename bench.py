#!/usr/bin/env python3
"""Benchmark of the adaptive block-sparse attention hot path on one MI355X.

One step = the whole path on one synthetic batch already resident in HBM:
reorder Q (rows layout), K (k64 tiles) and V (v64 tiles) -> route (pool, scores, Top-p
cut with Top-k floor, optional top-up, heaviest-first queue) -> block-sparse
attention on the persistent queue -> inverse reorder of the output.

Prints ONE JSON line.  `value` is executed attention TFLOP/s over whole steps
(4*d*BLK^2 per selected block pair / step time).  `roofline` reports the
sparse-attention kernel against the bf16 MFMA peak, its duration measured with
HIP events on the stream it is launched on.  `cpu_baseline` times the float64
CPU oracle on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 720p]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip dense comparator and schedule traces (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--configs", default="tiny,480p,hetero,long720p",
                    help="other workloads measured after the headline one (comma list, "
                         "'' for none): per-stage ms, attention TFLOP/s, dense comparator, "
                         "imbalance per schedule, top-up ms")
    ap.add_argument("--sched", default="xcd", choices=["queue", "static", "grid", "xcd"])
    ap.add_argument("--mfma-probe", action="store_true",
                    help="run the matrix-core probe even with --no-extras")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(reference kernel for HBM byte counters)")
    return ap.parse_args()


def measured_traffic(workload, sched_name):
    """HBM bytes per launch of the sparse kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, when it was taken on this workload and
    schedule with the current kernel source; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attn_kernel_{workload}_hbm_traffic.txt")
    src = os.path.join(ROOT, "adaptive_block_sparse_reorder_amd", "csrc", "attn.hip")
    if sched_name != "xcd" or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip().split()[0] if v.strip() else ""
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if kv.get("attn_source_sha256_16") != sha:
        return None
    return float(kv["attn_hbm_bytes"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def lambda_cu(trace_u32, rows, slots=512, n_units=256):
    """Imbalance of one traced launch: the load-imbalance factor of the FVAttn
    page (papers.paperslantern.ai/papers/2607.16190, section 2: largest unit
    load over the mean unit load), taken over the GPU's CUs and over its
    resident workgroup slots.

    lambda_cu:   per-CU busy time (sum of its item durations), max over the
                 mean of all n_units CUs (a CU that ran nothing counts as 0).
                 A CU is named by XCC_ID bits 3:0 and HW_ID bits 15:8.
    lambda_slot: critical path over mean slot load, span * slots / sum of item
                 durations, with slots = resident workgroups (2 per CU here).  A
                 CU hosting one long and one short workgroup looks balanced to
                 lambda_cu but idles half its capacity; lambda_slot sees it."""
    import numpy as np
    tr = trace_u32.reshape(-1, 8)[:rows]
    t0 = tr[:, 4].astype(np.uint64) | (tr[:, 5].astype(np.uint64) << np.uint64(32))
    t1 = tr[:, 6].astype(np.uint64) | (tr[:, 7].astype(np.uint64) << np.uint64(32))
    dur = (t1 - t0).astype(np.float64)
    xcc = tr[:, 1] & 0xF
    hw = tr[:, 2]
    cu_key = (xcc.astype(np.int64) << 8) | ((hw >> 8) & 0xFF).astype(np.int64)
    keys, inv = np.unique(cu_key, return_inverse=True)
    busy = np.bincount(inv, weights=dur)
    n = max(int(n_units), len(keys))
    span = float(t1.max() - t0.min())
    return dict(lambda_cu=float(busy.max() / (busy.sum() / n)),
                lambda_slot=float(span * slots / dur.sum()), cus=int(len(keys)),
                busy_max_ms=float(busy.max()) / 1e5, busy_mean_ms=float(busy.sum() / n) / 1e5,
                span_ms=span / 1e5)


def cpu_baseline(w, q, k, v, seconds):
    """Time the float64 oracle: its full routing, then its attention on a
    seeded sample of (head, query-block) items until ~`seconds` elapse."""
    import numpy as np
    from oracle import fva_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    qr = O.reorder(q.float().numpy(), w.grid, w.block)
    kr = O.reorder(k.float().numpy(), w.grid, w.block)
    vr = O.reorder(v.float().numpy(), w.grid, w.block)
    t1 = time.perf_counter()
    r = O.route_path(qr, kr, w.N, w.BLK, w.scale, w.top_p, w.topk_floor, w.aug_budget)
    t2 = time.perf_counter()
    # a stated head subset: the lightest and the heaviest head by W_h and two
    # seeded others; their query blocks are taken round-robin across the four
    # heads, each head's in seeded order, until the time budget is spent
    rng = np.random.default_rng(0)
    hc = r["head_count"].reshape(-1)
    light, heavy = int(np.argmin(hc)), int(np.argmax(hc))
    others = [x for x in rng.permutation(hc.shape[0]).tolist() if x not in (light, heavy)][:2]
    heads = [light, heavy] + others
    orders = [rng.permutation(w.nB) for _ in heads]
    counts = r["counts"].reshape(-1)
    flops, n = 0.0, 0
    ts = time.perf_counter()
    for step in range(w.nB):
        for bh, order in zip(heads, orders):
            b, h = divmod(bh, w.Hh)
            i = int(order[step])
            O.sparse_attention(qr, kr, vr, r["mask"], w.N, w.BLK, w.scale, items=[(b, h, i)])
            flops += 4.0 * w.d * w.BLK * w.BLK * counts[bh * w.nB + i]
            n += 1
        if time.perf_counter() - ts >= seconds:
            break
    dt = time.perf_counter() - ts
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "cpu_model": cpu_model,
        "sample": (f"float64 numpy oracle, attention of {n} (head, query-block) items of the "
                   f"{w.name} workload from heads {heads} (lightest and heaviest by W_h, up to two "
                   f"seeded), round-robin over the heads in seeded query-block order "
                   f"({flops / 1e12:.3f} executed TFLOP in {dt:.1f} s); its reorder of Q,K,V took "
                   f"{t1 - t0:.1f} s and routing of all {w.B * w.Hh * w.nB} rows {t2 - t1:.1f} s "
                   f"(not in value); cores = the BLAS threads its matrix products ran on"),
        "route_density": float(r["head_count"].sum() / (w.B * w.Hh * w.nB ** 2)),
    }


def reorder_pooled(F, w, buf, qd, kd, vd, table=None):
    """Forward block organization of Q (rows) and K (k64) with their block
    means written on the way, and of V (v64)."""
    g = buf.grid
    F.fva_reorder_pool(qd, buf.qr, buf.qbar, w.B, w.Hh, w.d, g, table, F.token_strides(qd),
                       F.FVA_LAYOUT_ROWS)
    F.fva_reorder_pool(kd, buf.kr, buf.kbar, w.B, w.Hh, w.d, g, table, F.token_strides(kd),
                       F.FVA_LAYOUT_K64)
    F.fva_reorder_ex(vd, buf.vt, w.B, w.Hh, w.d, g, table, F.token_strides(vd), F.FVA_FORWARD,
                     F.FVA_LAYOUT_V64)


def config_block(name, sched_flag, cus, slots, reps=3):
    """The whole path on another workload, timed stage by stage with HIP events
    on the launch stream (median of `reps` passes after two warm passes), with
    the dense comparator, the per-CU / per-slot imbalance of every schedule
    (traced launches), the realized density and, when the workload tops heads
    up to a pair budget, the top-up's own time."""
    import numpy as np
    import torch
    from adaptive_block_sparse_reorder_amd import fva as F
    from adaptive_block_sparse_reorder_amd.inputs import WORKLOADS, make_qkv

    w = WORKLOADS[name]
    log(f"config {name}: generating inputs")
    q, k, v = make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    del q, k, v
    buf = F.alloc_buffers(w.grid, w.block, w.B, w.Hh, w.d, trace=True)
    g, m = buf.grid, buf.mask()
    stream = torch.cuda.current_stream()
    prm = F.fva_route_params(w.top_p, w.topk_floor, w.aug_budget, 0.0, 0)

    def event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def reorders():
        reorder_pooled(F, w, buf, qd, kd, vd)

    def attn(flags, trace=None):
        F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0, flags,
                          buf.attn_ws, buf.sizes.attn_ws_bytes, trace)

    log(f"config {name}: timing the path")
    for _ in range(2):
        F.forward(buf, qd, kd, vd, w.top_p, w.topk_floor, w.aug_budget, attn_flags=sched_flag)
    torch.cuda.synchronize()
    laps = []
    for _ in range(reps):
        e = [event()]
        reorders()
        e.append(event())
        F.fva_route(buf.qbar, buf.kbar, w.B, w.Hh, w.d, g, prm, m, buf.route_ws,
                    buf.sizes.route_ws_bytes, F.FVA_ROUTE_POOLED_IN)
        e.append(event())
        attn(sched_flag)
        e.append(event())
        F.fva_reorder(buf.orr, buf.out, w.B, w.Hh, w.d, g, F.token_strides(buf.out),
                      F.FVA_INVERSE)
        e.append(event())
        laps.append(e)
    torch.cuda.synchronize()
    ms = np.median([[a.elapsed_time(b) for a, b in zip(e[:-1], e[1:])] for e in laps], axis=0)
    nnz = int(buf.row_count.sum().item())
    ex = F.executed_flops(nnz, w.d, w.BLK)
    de = F.dense_equiv_flops(w.N, w.d, w.Hh, w.B)
    dens = buf.head_count.cpu().numpy().astype(np.float64) / (w.nB ** 2)
    for _ in range(2):
        F.fva_dense_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g)
    dl = []
    for _ in range(reps):
        a = event()
        F.fva_dense_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g)
        dl.append((a, event()))
    torch.cuda.synchronize()
    ms_dense = float(np.median([a.elapsed_time(b) for a, b in dl]))
    # the sparse call timed the way the dense one is (back-to-back launches of
    # the attention call alone, events around each): the speedup compares the
    # two kernels, not the dispatch gap after the routing kernels that the
    # in-path figure above carries (microseconds, visible only on tiny problems)
    sl = []
    for _ in range(reps):
        a = event()
        attn(sched_flag)
        sl.append((a, event()))
    torch.cuda.synchronize()
    ms_alone = float(np.median([a.elapsed_time(b) for a, b in sl]))
    lam = {}
    for sname, fl in (("static", F.FVA_SCHED_STATIC), ("grid", F.FVA_SCHED_GRID),
                      ("queue", F.FVA_SCHED_QUEUE), ("xcd", F.FVA_SCHED_XCD)):
        buf.trace.zero_()
        attn(fl | F.FVA_TRACE, buf.trace)
        torch.cuda.synchronize()
        lc = lambda_cu(buf.trace.cpu().numpy().view(np.uint32), int(buf.sizes.rows), slots, cus)
        lam[sname] = {"lambda_cu": round(lc["lambda_cu"], 4),
                      "lambda_slot": round(lc["lambda_slot"], 4), "cus": lc["cus"]}
    out = {
        "workload": (f"B={w.B} heads={w.Hh} d={w.d} grid={w.grid[0]}x{w.grid[1]}x{w.grid[2]} "
                     f"({w.N} tokens, {w.nB} blocks of {w.BLK}) block={w.block[0]}x{w.block[1]}x"
                     f"{w.block[2]} top_p={w.top_p} topk_floor={w.topk_floor} "
                     f"aug_budget={w.aug_budget}"),
        "rows": int(buf.sizes.rows),
        "density": {"mean": round(float(dens.mean()), 4), "min": round(float(dens.min()), 4),
                    "max": round(float(dens.max()), 4)},
        "reorder_qkv_ms": round(float(ms[0]), 4),
        "route_ms": round(float(ms[1]), 4),
        "sparse_attn_ms": round(float(ms[2]), 4),
        "unreorder_ms": round(float(ms[3]), 4),
        "step_ms": round(float(ms.sum()), 4),
        "executed_tflop": round(ex / 1e12, 4),
        "executed_tflops": round(ex / (ms[2] * 1e-3) / 1e12, 2),
        "frac": round(ex / (ms[2] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "dense_equiv_tflops": round(de / (ms[2] * 1e-3) / 1e12, 2),
        "sparse_attn_alone_ms": round(ms_alone, 4),
        "dense_ms": round(ms_dense, 4),
        "speedup_vs_dense": round(ms_dense / ms_alone, 4),
        "imbalance": lam,
    }
    if w.aug_budget > 0:
        # the same top-up as inside the routing call, on its own: route
        # without a budget, then raise every head to the budget
        prm0 = F.fva_route_params(w.top_p, w.topk_floor, 0, 0.0, 0)
        budgets = torch.full((w.B * w.Hh,), w.aug_budget, dtype=torch.int64, device="cuda")
        tl = []
        for _ in range(reps):
            F.fva_route(buf.qr, buf.kr, w.B, w.Hh, w.d, g, prm0, m, buf.route_ws,
                        buf.sizes.route_ws_bytes, 0)
            a = event()
            F.fva_topup(w.B, w.Hh, w.d, g, budgets, m, buf.route_ws, buf.sizes.route_ws_bytes)
            tl.append((a, event()))
        torch.cuda.synchronize()
        out["topup_ms"] = round(float(np.median([a.elapsed_time(b) for a, b in tl])), 4)
        F.fva_route(buf.qr, buf.kr, w.B, w.Hh, w.d, g, prm0, m, buf.route_ws,
                    buf.sizes.route_ws_bytes, 0)
        torch.cuda.synchronize()
        out["topup_pairs_added"] = nnz - int(buf.row_count.sum().item())
    del buf, qd, kd, vd
    torch.cuda.empty_cache()
    log(f"config {name}: attention {out['sparse_attn_ms']} ms, "
        f"{out['executed_tflops']} TFLOP/s, dense {out['dense_ms']} ms")
    return out


def recall_stats(lse_sel, lse_all):
    """Share of each query's full softmax mass held by its selected blocks,
    exp(lse_sel - lse_all), over every real query of every head: the mask
    coverage the FVAttn page's sections 1 and 3.3 argue about, measured as the
    attention recall that the DFSAttn abstract listed at
    thelatestinai.com/papers/2607.16190 uses for block-sparse masks."""
    import torch

    r = torch.exp(lse_sel.double() - lse_all.double())
    return {"mean": round(float(r.mean()), 5),
            "p05": round(float(torch.quantile(r.float(), 0.05)), 5),
            "min": round(float(r.min()), 5)}


def copy_reference(reorder_gbs, mib=2048, reps=10):
    """Practical HBM rate of this card: a plain device-to-device copy (torch),
    counted as bytes read plus bytes written, the reference the streaming
    kernels (reorder, pool, un-reorder) are read against."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * n / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del src, dst
    return {"what": f"torch device copy of {mib} MiB, read + write bytes", "GBs": round(gbs, 1),
            "frac_of_8TBs": round(gbs / 8000.0, 4), "reorder_over_copy": round(reorder_gbs / gbs, 4)}


def mfma_ceiling(attn_tflops, iters=2_000_000):
    """Matrix-core-only steady state of this card (libfva_probe.so): two waves
    per SIMD issuing independent 32x32x16 bf16 MFMAs on register operands,
    nothing else, for about half a second, on random normal operands and on
    constant ones.  The switching power of the data sets the clock the matrix
    cores can hold, so the rate on random operands is the practical ceiling
    of any bf16 MFMA kernel on real data; the attention kernel's rate is also
    given as a share of it.  The roofline's peak stays the published one."""
    import ctypes
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "adaptive_block_sparse_reorder_amd", "libfva_probe.so"))
    lib.fva_probe_operand_bytes.restype = ctypes.c_size_t
    lib.fva_probe_output_bytes.restype = ctypes.c_size_t
    lib.fva_probe_operand_bytes.argtypes = [ctypes.c_int32]
    lib.fva_probe_output_bytes.argtypes = [ctypes.c_int32]
    lib.fva_probe_mfma.restype = ctypes.c_int32
    lib.fva_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p]
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    nop = lib.fva_probe_operand_bytes(blocks) // 2
    out = torch.empty(lib.fva_probe_output_bytes(blocks) // 4, dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(11)
    res = {"what": "independent v_mfma_f32_32x32x16_bf16, 2 waves per SIMD, register operands, "
                   f"{iters} rounds of 4 per wave"}
    stream = torch.cuda.current_stream()
    for name, ops in (("random", torch.randn(nop, device="cuda", dtype=torch.bfloat16, generator=gen)),
                      ("constant", torch.ones(nop, device="cuda", dtype=torch.bfloat16))):
        st = lib.fva_probe_mfma(ops.data_ptr(), out.data_ptr(), blocks, iters // 10, stream.cuda_stream)
        assert st == 0, st
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.fva_probe_mfma(ops.data_ptr(), out.data_ptr(), blocks, iters, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        assert st == 0, st
        ms = e0.elapsed_time(e1)
        flop = blocks * 512 / 64 * iters * 4 * 32768.0
        res[f"{name}_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
        res[f"{name}_ms"] = round(ms, 2)
    res["attn_over_random"] = round(attn_tflops / res["random_tflops"], 4)
    return res


def gemm_reference(attn_tflops, n=8192, reps=50):
    """Practical bf16 MFMA rate of this card: the vendor GEMM (torch.matmul)
    on random normal operands.  Data-dependent power, not the issue rate, sets
    the clock it runs at, so it is the reference the attention kernel's rate is
    read against (the published peak stays the roofline's peak)."""
    import torch

    gen = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    tf = 2.0 * n ** 3 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12
    del a, b, c
    return {"library": "torch.matmul (hipBLASLt), random normal bf16 operands", "n": n,
            "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "attn_over_gemm": round(attn_tflops / tf, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU (its per-GPU share of heads); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    from adaptive_block_sparse_reorder_amd import fva as F
    from adaptive_block_sparse_reorder_amd.inputs import WORKLOADS, make_qkv

    sched_name = args.sched
    args.sched = {"queue": F.FVA_SCHED_QUEUE, "static": F.FVA_SCHED_STATIC,
                  "grid": F.FVA_SCHED_GRID, "xcd": F.FVA_SCHED_XCD}[sched_name]
    F.load_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = WORKLOADS[args.workload]
    log(f"generating {w.name} inputs")
    q, k, v = make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    buf = F.alloc_buffers(w.grid, w.block, w.B, w.Hh, w.d, trace=True)
    g = buf.grid
    stream = torch.cuda.current_stream()
    prm = F.fva_route_params(w.top_p, w.topk_floor, w.aug_budget, 0.0, 0)
    m = buf.mask()

    ev = {}

    def mark(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev.setdefault(name, []).append(e)

    def step(timed):
        if timed: mark("s0")
        reorder_pooled(F, w, buf, qd, kd, vd)
        if timed: mark("s1")
        F.fva_route(buf.qbar, buf.kbar, w.B, w.Hh, w.d, g, prm, m, buf.route_ws,
                    buf.sizes.route_ws_bytes, F.FVA_ROUTE_POOLED_IN)
        if timed: mark("s2")
        F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0,
                          args.sched, buf.attn_ws, buf.sizes.attn_ws_bytes, None)
        if timed: mark("s3")
        F.fva_reorder(buf.orr, buf.out, w.B, w.Hh, w.d, g, F.token_strides(buf.out),
                      F.FVA_INVERSE)
        if timed: mark("s4")

    log("warmup")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def avg(a, b):
        return float(np.mean([x.elapsed_time(y) for x, y in zip(ev[a], ev[b])]))

    ms_reorder, ms_route, ms_attn, ms_unre = (avg("s0", "s1"), avg("s1", "s2"),
                                              avg("s2", "s3"), avg("s3", "s4"))
    ms_step = wall * 1e3 / args.steps
    nnz = int(buf.row_count.sum().item())
    heads = buf.head_count.cpu().numpy().astype(np.float64) / (w.nB ** 2)
    ex_flop = F.executed_flops(nnz, w.d, w.BLK)
    de_flop = F.dense_equiv_flops(w.N, w.d, w.Hh, w.B)
    attn_tflops = ex_flop / (ms_attn * 1e-3) / 1e12
    # reorder: read N*Hh*d and write Npad*Hh*d bf16 for each of Q, K, V, and
    # write the float32 block means of Q and K
    reorder_bytes = 3 * 2 * w.B * w.Hh * w.d * (w.N + w.Npad) + 2 * 4 * int(buf.sizes.rows) * w.d
    unre_bytes = 2 * w.B * w.Hh * w.d * (w.N + w.N)

    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step, attention {ms_attn:.3f} ms")
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    extras = {}
    if args.no_extras and args.mfma_probe:
        extras["mfma_ceiling"] = mfma_ceiling(attn_tflops)
    if not args.no_extras:
        log("dense comparator and schedule traces")
        # dense comparator, same core
        for _ in range(2):
            F.fva_dense_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record(stream)
        for _ in range(reps):
            F.fva_dense_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_dense = e0.elapsed_time(e1) / reps
        extras["dense_ms"] = ms_dense
        extras["dense_tflops"] = de_flop / (ms_dense * 1e-3) / 1e12
        extras["speedup_vs_dense"] = ms_dense / ms_attn
        extras["gemm_reference"] = gemm_reference(attn_tflops)
        extras["mfma_ceiling"] = mfma_ceiling(attn_tflops)
        extras["torch_copy_reference"] = copy_reference(reorder_bytes / (ms_reorder * 1e-3) / 1e9)
        # mask recall: per-query log-sum-exp of the sparse and the dense kernel
        nq = w.B * w.Hh * w.N
        lse_all = torch.empty(nq, dtype=torch.float32, device="cuda")
        lse_sel = torch.empty(nq, dtype=torch.float32, device="cuda")
        F.fva_dense_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, lse=lse_all)
        F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0, args.sched,
                          buf.attn_ws, buf.sizes.attn_ws_bytes, None, lse=lse_sel)
        torch.cuda.synchronize()
        recall = {"definition": "exp(lse_sparse - lse_dense) per real query, all heads",
                  "topp_raster": recall_stats(lse_sel, lse_all)}
        # per-CU and per-slot imbalance under each schedule (2 resident
        # workgroups per CU: 64 KB of LDS each)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        slots = 2 * cus
        lam = {}
        for name, fl in (("static", F.FVA_SCHED_STATIC), ("grid", F.FVA_SCHED_GRID),
                         ("queue", F.FVA_SCHED_QUEUE), ("xcd", F.FVA_SCHED_XCD)):
            buf.trace.zero_()
            F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0,
                              fl | F.FVA_TRACE, buf.attn_ws, buf.sizes.attn_ws_bytes, buf.trace)
            torch.cuda.synchronize()
            lam[name] = lambda_cu(buf.trace.cpu().numpy().view(np.uint32), int(buf.sizes.rows),
                                  slots, cus)
        extras["lambda_cu"] = lam

    if not args.no_extras:
        # reorder + route with the router pooling Q and K itself (a second
        # read of both) against the pooling reorder the step uses
        pev = []
        for _ in range(3):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            for x, dst, lay in ((qd, buf.qr, F.FVA_LAYOUT_ROWS), (kd, buf.kr, F.FVA_LAYOUT_K64),
                                (vd, buf.vt, F.FVA_LAYOUT_V64)):
                F.fva_reorder(x, dst, w.B, w.Hh, w.d, g, F.token_strides(x), F.FVA_FORWARD, lay)
            e[1].record(stream)
            F.fva_route(buf.qr, buf.kr, w.B, w.Hh, w.d, g, prm, m, buf.route_ws,
                        buf.sizes.route_ws_bytes, 0)
            e[2].record(stream)
            pev.append(e)
        torch.cuda.synchronize()
        extras["pool_in_router"] = {
            "reorder_qkv_ms": round(float(np.median([e[0].elapsed_time(e[1]) for e in pev])), 4),
            "route_ms": round(float(np.median([e[1].elapsed_time(e[2]) for e in pev])), 4),
        }

    if not args.no_extras:
        # the same step with the tile order along a 3-D Hilbert curve
        table = F.tile_table(g, F.FVA_ORDER_HILBERT)
        ev.clear()
        for _ in range(2):
            F.forward(buf, qd, kd, vd, w.top_p, w.topk_floor, w.aug_budget, attn_flags=args.sched,
                      table=table)
        hev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        hev[0].record(stream)
        reorder_pooled(F, w, buf, qd, kd, vd, table)
        hev[1].record(stream)
        F.fva_route(buf.qbar, buf.kbar, w.B, w.Hh, w.d, g, prm, m, buf.route_ws,
                    buf.sizes.route_ws_bytes, F.FVA_ROUTE_POOLED_IN)
        hev[2].record(stream)
        F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0,
                          args.sched, buf.attn_ws, buf.sizes.attn_ws_bytes, None)
        hev[3].record(stream)
        F.fva_reorder_ex(buf.orr, buf.out, w.B, w.Hh, w.d, g, table, F.token_strides(buf.out),
                         F.FVA_INVERSE)
        hev[4].record(stream)
        torch.cuda.synchronize()
        hnnz = int(buf.row_count.sum().item())
        lse_hall = torch.empty(nq, dtype=torch.float32, device="cuda")
        F.fva_dense_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, lse=lse_hall)
        F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0, args.sched,
                          buf.attn_ws, buf.sizes.attn_ws_bytes, None, lse=lse_sel)
        torch.cuda.synchronize()
        recall["topp_hilbert"] = recall_stats(lse_sel, lse_hall)
        del lse_hall
        extras["hilbert_order"] = {
            "density_mean": round(hnnz / (w.B * w.Hh * w.nB ** 2), 4),
            "density_mean_raster": round(nnz / (w.B * w.Hh * w.nB ** 2), 4),
            "reorder_qkv_ms": round(hev[0].elapsed_time(hev[1]), 4),
            "route_ms": round(hev[1].elapsed_time(hev[2]), 4),
            "sparse_attn_ms": round(hev[2].elapsed_time(hev[3]), 4),
            "unreorder_ms": round(hev[3].elapsed_time(hev[4]), 4),
        }
        # fixed Top-k control: every row keeps the Top-p run's mean row count,
        # a uniform per-row load with the same executed work
        kfix = int(round(nnz / (w.B * w.Hh * w.nB)))
        prm_k = F.fva_route_params(0.0, kfix, 0, 0.0, 0)
        for x, dst, lay in ((qd, buf.qr, F.FVA_LAYOUT_ROWS), (kd, buf.kr, F.FVA_LAYOUT_K64),
                            (vd, buf.vt, F.FVA_LAYOUT_V64)):
            F.fva_reorder(x, dst, w.B, w.Hh, w.d, g, F.token_strides(x), F.FVA_FORWARD, lay)
        F.fva_route(buf.qr, buf.kr, w.B, w.Hh, w.d, g, prm_k, m, buf.route_ws,
                    buf.sizes.route_ws_bytes, 0)
        fk = {"topk": kfix}
        for name, fl in (("static", F.FVA_SCHED_STATIC), ("queue", F.FVA_SCHED_QUEUE),
                         ("xcd", F.FVA_SCHED_XCD)):
            buf.trace.zero_()
            k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            k0.record(stream)
            F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0,
                              fl | F.FVA_TRACE, buf.attn_ws, buf.sizes.attn_ws_bytes, buf.trace)
            k1.record(stream)
            torch.cuda.synchronize()
            lc = lambda_cu(buf.trace.cpu().numpy().view(np.uint32), int(buf.sizes.rows), slots,
                           cus)
            fk[name] = {"lambda_cu": round(lc["lambda_cu"], 4),
                        "lambda_slot": round(lc["lambda_slot"], 4),
                        "attn_ms_traced": round(k0.elapsed_time(k1), 3)}
        F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0, args.sched,
                          buf.attn_ws, buf.sizes.attn_ws_bytes, None, lse=lse_sel)
        torch.cuda.synchronize()
        recall["topk_fixed_raster"] = recall_stats(lse_sel, lse_all)
        extras["fixed_topk_control"] = fk
        # quality-efficiency points: Top-p at several p (floor as configured)
        # and, for each, a fixed Top-k with the same executed work
        pareto = []
        for p_cut in (0.8, 0.9, 0.95, 0.98):
            for policy in ("top_p", "top_k"):
                if policy == "top_p":
                    prm_x = F.fva_route_params(p_cut, w.topk_floor, 0, 0.0, 0)
                else:
                    prm_x = F.fva_route_params(0.0, kmatch, 0, 0.0, 0)
                F.fva_route(buf.qr, buf.kr, w.B, w.Hh, w.d, g, prm_x, m, buf.route_ws,
                            buf.sizes.route_ws_bytes, 0)
                x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                x0.record(stream)
                F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0,
                                  args.sched, buf.attn_ws, buf.sizes.attn_ws_bytes, None,
                                  lse=lse_sel)
                x1.record(stream)
                torch.cuda.synchronize()
                xnnz = int(buf.row_count.sum().item())
                if policy == "top_p":
                    kmatch = int(round(xnnz / (w.B * w.Hh * w.nB)))
                rs = recall_stats(lse_sel, lse_all)
                pareto.append({"policy": policy,
                               "param": p_cut if policy == "top_p" else kmatch,
                               "density": round(xnnz / (w.B * w.Hh * w.nB ** 2), 4),
                               "recall_mean": rs["mean"], "recall_p05": rs["p05"],
                               "attn_ms": round(x0.elapsed_time(x1), 3)})
        recall["pareto_raster"] = pareto
        # restore the raster-order Top-p state for what follows
        step(False)
        torch.cuda.synchronize()

    # runtime load balancing on 8 virtual ranks (fewer when there are fewer
    # heads) from the realized workloads
    vranks = min(8, len(buf.head_count))
    hc = buf.head_count.cpu().numpy().astype(np.int64).tolist()
    rlb = {}
    for name, topo in (("pairs", F.FVA_RLB_PAIRS), ("ring", F.FVA_RLB_RING)):
        _, _, roh, st = F.fva_rlb_plan(hc, vranks, topo)
        rlb[name] = {"lambda_before": round(st.lambda_before, 4),
                     "lambda_after": round(st.lambda_after, 4),
                     "migrations": int(st.migrations), "solve_us": round(st.solve_us, 1)}
        if name == "pairs":
            roh_pairs = roh
    rlb["ranks"] = vranks
    extras["rlb_virtual_ranks"] = rlb
    # slack-aware augmentation after balancing (alpha 0.5), applied on the device
    budgets, rank_after = F.fva_sasa_budget(hc, vranks, roh_pairs, 0.5, w.nB * w.nB)
    dev_budgets = torch.tensor(budgets, dtype=torch.int64, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    F.fva_topup(w.B, w.Hh, w.d, g, dev_budgets, m, buf.route_ws, buf.sizes.route_ws_bytes)
    e1.record(stream)
    torch.cuda.synchronize()
    if not args.no_extras:
        F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, g, m, 0.0, args.sched,
                          buf.attn_ws, buf.sizes.attn_ws_bytes, None, lse=lse_sel)
        torch.cuda.synchronize()
        recall["topp_raster_after_sasa"] = recall_stats(lse_sel, lse_all)
        extras["mask_recall"] = recall
    extras["sasa_alpha_0.5"] = {
        "topup_ms": round(e0.elapsed_time(e1), 4),
        "pairs_added": int(sum(budgets) - sum(hc)),
        "rank_max_after": int(max(rank_after)),
        "density_after": round(float(buf.head_count.sum().item()) / (w.Hh * w.B * w.nB ** 2), 4),
    }

    if not args.no_extras and args.configs:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        extras["configs"] = {c: config_block(c, args.sched, cus, 2 * cus)
                             for c in args.configs.split(",") if c and c != w.name}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu oracle baseline")
        cpu = cpu_baseline(w, q, k, v, args.cpu_seconds)

    out = {
        "metric": "sparse-attn ms & executed TFLOP/s (% bf16 MFMA peak) at 720p Wan shape, 1 GPU",
        "value": round(ex_flop / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={w.B} heads={w.Hh} d={w.d} grid={w.grid[0]}x{w.grid[1]}x"
                        f"{w.grid[2]} ({w.N} tokens, {w.nB} blocks of {w.BLK}) block="
                        f"{w.block[0]}x{w.block[1]}x{w.block[2]} top_p={w.top_p} "
                        f"topk_floor={w.topk_floor} aug_budget={w.aug_budget}",
            "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "mfma", "kernel": f"attn_kernel (sparse, {sched_name} schedule)",
            "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(w.name, sched_name),
        },
        "cpu_baseline": cpu,
        "breakdown": {
            "sparse_attn_ms": round(ms_attn, 4),
            "executed_tflop": round(ex_flop / 1e12, 3),
            "dense_equiv_tflop": round(de_flop / 1e12, 3),
            "executed_tflops": round(attn_tflops, 2),
            "dense_equiv_tflops": round(de_flop / (ms_attn * 1e-3) / 1e12, 2),
            "density": {"mean": float(heads.mean()), "min": float(heads.min()),
                        "max": float(heads.max())},
            "stages": ("reorder_qkv: Q and K reordered with their block means, V reordered; "
                       "route: block scores, Top-p/Top-k cut, mask, top-up, queue"),
            "reorder_qkv_ms": round(ms_reorder, 4),
            "reorder_qkv_GBs": round(reorder_bytes / (ms_reorder * 1e-3) / 1e9, 1),
            "route_ms": round(ms_route, 4),
            "unreorder_ms": round(ms_unre, 4),
            "unreorder_GBs": round(unre_bytes / (ms_unre * 1e-3) / 1e9, 1),
            **{k2: (round(v2, 4) if isinstance(v2, float) else v2) for k2, v2 in extras.items()},
        },
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
