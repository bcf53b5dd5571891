"""Thin ctypes binding of libfva (include/fva.h), same names as the C ABI.

Argument marshalling only: torch tensors are passed as device pointers and
torch's current HIP stream is used unless a stream handle is given.  Every
step of the path runs in the HIP kernels of libfva.so; there is no fallback,
and loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import math
import os
import re
from dataclasses import dataclass
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfva.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "fva.h")

FVA_OK = 0
FVA_ERR_INVALID_ARG = -1
FVA_ERR_UNSUPPORTED = -2
FVA_ERR_WORKSPACE = -3
FVA_ERR_HIP = -4

FVA_ROUTE_SCORES_IN = 0x1
FVA_ROUTE_POOLED_IN = 0x2
FVA_SCHED_QUEUE = 0x0
FVA_SCHED_STATIC = 0x1
FVA_SCHED_GRID = 0x2
FVA_SCHED_XCD = 0x3
FVA_TRACE = 0x10
FVA_FORWARD = 0
FVA_INVERSE = 1
FVA_LAYOUT_ROWS = 0
FVA_LAYOUT_V64 = 1
FVA_LAYOUT_K64 = 2
FVA_ORDER_RASTER = 0
FVA_ORDER_HILBERT = 1
FVA_RLB_PAIRS = 0
FVA_RLB_RING = 1
FVA_RLB_MAX_PAIR_RANKS = 12


class fva_grid(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "W", "bt", "bh", "bw")]


class fva_sizes_t(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("Npad", ctypes.c_int64), ("BLK", ctypes.c_int32),
                ("nB", ctypes.c_int32), ("words", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("route_ws_bytes", ctypes.c_size_t),
                ("attn_ws_bytes", ctypes.c_size_t), ("trace_bytes", ctypes.c_size_t)]


class fva_route_params(ctypes.Structure):
    _fields_ = [("top_p", ctypes.c_float), ("topk_floor", ctypes.c_int32),
                ("aug_budget", ctypes.c_int64), ("scale", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


class fva_mask(ctypes.Structure):
    _fields_ = [("scores", ctypes.c_void_p), ("bitmask", ctypes.c_void_p),
                ("row_count", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("head_count", ctypes.c_void_p), ("queue", ctypes.c_void_p)]


class fva_rlb_stats(ctypes.Structure):
    _fields_ = [("max_before", ctypes.c_int64), ("max_after", ctypes.c_int64),
                ("mean", ctypes.c_double), ("lambda_before", ctypes.c_double),
                ("lambda_after", ctypes.c_double), ("solve_us", ctypes.c_double),
                ("migrations", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class FvaError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: status {status}: {detail}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfva.so once; raise when it is missing (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m adaptive_block_sparse_reorder_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                          ctypes.c_float)
    lib.fva_sizes.argtypes = [ctypes.POINTER(fva_grid), I32, I32, I32, ctypes.POINTER(fva_sizes_t)]
    lib.fva_reorder.argtypes = [P, P, I32, I32, I32, ctypes.POINTER(fva_grid),
                                ctypes.POINTER(ctypes.c_int64), I32, I32, P]
    lib.fva_route.argtypes = [P, P, I32, I32, I32, ctypes.POINTER(fva_grid),
                              ctypes.POINTER(fva_route_params), ctypes.POINTER(fva_mask), P, SZ,
                              I32, P]
    lib.fva_route_flags.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), P]
    lib.fva_sparse_attn.argtypes = [P, P, P, P, I32, I32, I32, ctypes.POINTER(fva_grid),
                                    ctypes.POINTER(fva_mask), F, I32, P, SZ, P, P, P]
    lib.fva_dense_attn.argtypes = [P, P, P, P, I32, I32, I32, ctypes.POINTER(fva_grid), F, P, P]
    lib.fva_sparse_attn_noalloc.argtypes = [P, P, P, P, I32, I32, I32, ctypes.POINTER(fva_grid),
                                            ctypes.POINTER(fva_mask), F, I32, P, P, P]
    lib.fva_reorder_ex.argtypes = [P, P, I32, I32, I32, ctypes.POINTER(fva_grid), P,
                                   ctypes.POINTER(ctypes.c_int64), I32, I32, P]
    lib.fva_reorder_pool.argtypes = [P, P, P, I32, I32, I32, ctypes.POINTER(fva_grid), P,
                                     ctypes.POINTER(I64), I32, P]
    lib.fva_tile_order_bytes.argtypes = [ctypes.POINTER(fva_grid), ctypes.POINTER(ctypes.c_size_t)]
    lib.fva_tile_order.argtypes = [ctypes.POINTER(fva_grid), I32, P, SZ, P]
    lib.fva_tile_table_status.argtypes = [P, ctypes.POINTER(ctypes.c_int32), P]
    PI32 = ctypes.POINTER(ctypes.c_int32)
    PI64 = ctypes.POINTER(ctypes.c_int64)
    lib.fva_rlb_plan.argtypes = [PI32, I32, I32, I32, PI32, PI32, PI32,
                                 ctypes.POINTER(fva_rlb_stats)]
    lib.fva_sasa_budget.argtypes = [PI32, I32, I32, PI32, F, I64, PI64, PI64]
    lib.fva_topup.argtypes = [I32, I32, I32, ctypes.POINTER(fva_grid), P,
                              ctypes.POINTER(fva_mask), P, SZ, P]
    for fn in ("fva_sizes", "fva_reorder", "fva_route", "fva_route_flags", "fva_sparse_attn",
               "fva_dense_attn", "fva_rlb_plan", "fva_sasa_budget", "fva_topup",
               "fva_reorder_ex", "fva_reorder_pool", "fva_tile_order_bytes", "fva_tile_order",
               "fva_tile_table_status", "fva_sparse_attn_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.fva_status_string.argtypes = [ctypes.c_int]
    lib.fva_status_string.restype = ctypes.c_char_p
    lib.fva_last_error.argtypes = []
    lib.fva_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the entry points declared in include/fva.h."""
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fva_[a-z_]+)\s*\(", src)))


def _check(st: int, fn: str):
    if st != FVA_OK:
        lib = load_library()
        raise FvaError(st, fn, lib.fva_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_grid(grid: Sequence[int], block: Sequence[int]) -> fva_grid:
    return fva_grid(*[int(x) for x in grid], *[int(x) for x in block])


def fva_sizes(grid: fva_grid, B: int, Hh: int, d: int) -> fva_sizes_t:
    lib = load_library()
    out = fva_sizes_t()
    _check(lib.fva_sizes(ctypes.byref(grid), B, Hh, d, ctypes.byref(out)), "fva_sizes")
    return out


def fva_reorder(src, dst, B: int, Hh: int, d: int, grid: fva_grid, strides: Sequence[int],
                direction: int = FVA_FORWARD, layout: int = FVA_LAYOUT_ROWS, stream=None):
    lib = load_library()
    st = (ctypes.c_int64 * 3)(*[int(s) for s in strides])
    _check(lib.fva_reorder(_ptr(src), _ptr(dst), B, Hh, d, ctypes.byref(grid), st, direction,
                           layout, _stream(stream)), "fva_reorder")


def fva_reorder_ex(src, dst, B: int, Hh: int, d: int, grid: fva_grid, table,
                   strides: Sequence[int], direction: int = FVA_FORWARD,
                   layout: int = FVA_LAYOUT_ROWS, stream=None):
    lib = load_library()
    st = (ctypes.c_int64 * 3)(*[int(s) for s in strides])
    _check(lib.fva_reorder_ex(_ptr(src), _ptr(dst), B, Hh, d, ctypes.byref(grid), _ptr(table), st,
                              direction, layout, _stream(stream)), "fva_reorder_ex")


def fva_reorder_pool(src, dst, pooled, B: int, Hh: int, d: int, grid: fva_grid, table,
                     strides: Sequence[int], layout: int = FVA_LAYOUT_ROWS, stream=None):
    """Forward reorder into `layout` (rows or k64) that also writes the float32
    block means [B*Hh, nB, d] into `pooled`."""
    lib = load_library()
    st = (ctypes.c_int64 * 3)(*[int(s) for s in strides])
    _check(lib.fva_reorder_pool(_ptr(src), _ptr(dst), _ptr(pooled), B, Hh, d, ctypes.byref(grid),
                                _ptr(table), st, layout, _stream(stream)), "fva_reorder_pool")


def fva_tile_order_bytes(grid: fva_grid) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.fva_tile_order_bytes(ctypes.byref(grid), ctypes.byref(n)), "fva_tile_order_bytes")
    return int(n.value)


def fva_tile_order(grid: fva_grid, order: int, table, table_bytes: int, stream=None):
    lib = load_library()
    _check(lib.fva_tile_order(ctypes.byref(grid), order, _ptr(table), table_bytes,
                              _stream(stream)), "fva_tile_order")


def fva_tile_table_status(table, stream=None) -> int:
    lib = load_library()
    v = ctypes.c_int32(0)
    _check(lib.fva_tile_table_status(_ptr(table), ctypes.byref(v), _stream(stream)),
           "fva_tile_table_status")
    return int(v.value)


TILE_TABLE_HEADER_WORDS = 12


def tile_table(grid: fva_grid, order: int = FVA_ORDER_HILBERT, device="cuda", stream=None):
    """Allocate (torch) and fill a device tile table."""
    import torch
    nbytes = fva_tile_order_bytes(grid)
    t = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device=device)
    fva_tile_order(grid, order, t, nbytes, stream)
    return t


def fva_route(qr, kr, B: int, Hh: int, d: int, grid: fva_grid, params: fva_route_params,
              mask: fva_mask, ws, ws_bytes: int, flags: int = 0, stream=None):
    lib = load_library()
    _check(lib.fva_route(_ptr(qr), _ptr(kr), B, Hh, d, ctypes.byref(grid), ctypes.byref(params),
                         ctypes.byref(mask), _ptr(ws), ws_bytes, flags, _stream(stream)),
           "fva_route")


def fva_route_flags(ws, stream=None) -> int:
    lib = load_library()
    v = ctypes.c_uint32(0)
    _check(lib.fva_route_flags(_ptr(ws), ctypes.byref(v), _stream(stream)), "fva_route_flags")
    return int(v.value)


def fva_sparse_attn(qr, kr, vt, out, B: int, Hh: int, d: int, grid: fva_grid, mask: fva_mask,
                    scale: float = 0.0, flags: int = FVA_SCHED_QUEUE, ws=None, ws_bytes: int = 0,
                    trace=None, stream=None, lse=None):
    """lse: optional float32 device tensor of B*Hh*N entries (per-query
    log-sum-exp of the scaled scores over the keys used)."""
    lib = load_library()
    _check(lib.fva_sparse_attn(_ptr(qr), _ptr(kr), _ptr(vt), _ptr(out), B, Hh, d,
                               ctypes.byref(grid), ctypes.byref(mask), scale, flags, _ptr(ws),
                               ws_bytes, _ptr(trace), _ptr(lse), _stream(stream)),
           "fva_sparse_attn")


FVA_NOALLOC_ATTN_WS_MAX = 1 << 20


def fva_sparse_attn_noalloc(qr, kr, vt, out, B: int, Hh: int, d: int, grid: fva_grid,
                            mask: fva_mask, scale: float = 0.0, flags: int = FVA_SCHED_QUEUE,
                            trace=None, stream=None, lse=None):
    """fva_sparse_attn with the library's own static workspace (no caller
    workspace, no allocation)."""
    lib = load_library()
    _check(lib.fva_sparse_attn_noalloc(_ptr(qr), _ptr(kr), _ptr(vt), _ptr(out), B, Hh, d,
                                       ctypes.byref(grid), ctypes.byref(mask), scale, flags,
                                       _ptr(trace), _ptr(lse), _stream(stream)),
           "fva_sparse_attn_noalloc")


def fva_dense_attn(qr, kr, vt, out, B: int, Hh: int, d: int, grid: fva_grid, scale: float = 0.0,
                   stream=None, lse=None):
    lib = load_library()
    _check(lib.fva_dense_attn(_ptr(qr), _ptr(kr), _ptr(vt), _ptr(out), B, Hh, d,
                              ctypes.byref(grid), scale, _ptr(lse), _stream(stream)),
           "fva_dense_attn")


def fva_rlb_plan(head_count, ranks: int, topology: int = FVA_RLB_PAIRS):
    """Host planner.  head_count: sequence of per-head workloads W_h.
    Returns (send_to, send_head, rank_of_head, stats)."""
    lib = load_library()
    W = [int(x) for x in head_count]
    n = len(W)
    hc = (ctypes.c_int32 * n)(*W)
    to = (ctypes.c_int32 * ranks)()
    hd = (ctypes.c_int32 * ranks)()
    roh = (ctypes.c_int32 * n)()
    st = fva_rlb_stats()
    _check(lib.fva_rlb_plan(hc, n, ranks, topology, to, hd, roh, ctypes.byref(st)),
           "fva_rlb_plan")
    return list(to), list(hd), list(roh), st


def fva_sasa_budget(head_count, ranks: int, rank_of_head, alpha: float, head_cap: int):
    """Host budgets.  Returns (head_budget, rank_load_after) as lists."""
    lib = load_library()
    W = [int(x) for x in head_count]
    n = len(W)
    hc = (ctypes.c_int32 * n)(*W)
    roh = (ctypes.c_int32 * n)(*[int(x) for x in rank_of_head])
    hb = (ctypes.c_int64 * n)()
    rl = (ctypes.c_int64 * ranks)()
    _check(lib.fva_sasa_budget(hc, n, ranks, roh, float(alpha), int(head_cap), hb, rl),
           "fva_sasa_budget")
    return list(hb), list(rl)


def fva_topup(B: int, Hh: int, d: int, grid: fva_grid, head_budget, mask: fva_mask, ws,
              ws_bytes: int, stream=None):
    """Device top-up with per-head budgets (head_budget: device int64 [B*Hh])."""
    lib = load_library()
    _check(lib.fva_topup(B, Hh, d, ctypes.byref(grid), _ptr(head_budget), ctypes.byref(mask),
                         _ptr(ws), ws_bytes, _stream(stream)), "fva_topup")


# --------------------------------------------------------------------------
# Device buffers for one problem (allocation through torch: plumbing only)
# --------------------------------------------------------------------------

@dataclass
class Buffers:
    grid: fva_grid
    sizes: fva_sizes_t
    B: int
    Hh: int
    d: int
    qr: object
    kr: object
    vt: object
    orr: object
    out: object
    scores: object
    bitmask: object
    row_count: object
    col_idx: object
    head_count: object
    queue: object
    route_ws: object
    attn_ws: object
    trace: object
    qbar: object = None
    kbar: object = None

    def mask(self) -> fva_mask:
        return fva_mask(self.scores.data_ptr(), self.bitmask.data_ptr(),
                        self.row_count.data_ptr(), self.col_idx.data_ptr(),
                        self.head_count.data_ptr(), self.queue.data_ptr())


def alloc_buffers(grid: Sequence[int], block: Sequence[int], B: int, Hh: int, d: int,
                  device="cuda", trace: bool = False) -> Buffers:
    import torch
    g = make_grid(grid, block)
    sz = fva_sizes(g, B, Hh, d)
    bf = torch.bfloat16
    rows, nB = int(sz.rows), int(sz.nB)

    def dev(n, dt):
        return torch.empty(n, dtype=dt, device=device)

    # workspaces are allocated as 256-byte-aligned int64 storage
    def ws(nbytes):
        return torch.zeros((nbytes + 7) // 8, dtype=torch.int64, device=device)

    return Buffers(
        grid=g, sizes=sz, B=B, Hh=Hh, d=d,
        qr=dev((B, Hh, sz.Npad, d), bf), kr=dev((B, Hh, sz.Npad // 64, d // 8, 64, 8), bf),
        vt=dev((B, Hh, sz.Npad // 64, 8, d, 8), bf), orr=dev((B, Hh, sz.Npad, d), bf),
        out=dev((B, int(sz.N), Hh, d), bf),
        scores=dev((rows, nB), torch.float32), bitmask=dev((rows, int(sz.words)), torch.int32),
        row_count=dev((rows,), torch.int32), col_idx=dev((rows, nB), torch.int16),
        head_count=dev((B * Hh,), torch.int32), queue=dev((rows,), torch.int32),
        route_ws=ws(sz.route_ws_bytes), attn_ws=ws(sz.attn_ws_bytes),
        trace=ws(sz.trace_bytes) if trace else None,
        qbar=dev((rows, d), torch.float32), kbar=dev((rows, d), torch.float32))


def token_strides(x) -> Sequence[int]:
    """Element strides (b, n, h) of a token-major [B, N, Hh, d] tensor."""
    assert x.stride(3) == 1
    return (x.stride(0), x.stride(1), x.stride(2))


def forward(buf: Buffers, q, k, v, top_p: float, topk_floor: int, aug_budget: int = 0,
            scale: float = 0.0, route_flags: int = 0, attn_flags: int = FVA_SCHED_XCD,
            stream=None, table=None, lse=None):
    """One pass of the hot path: reorder Q (rows) and K (k64) with their block
    means, V (v64) -> route from the means -> block-sparse attention -> inverse
    reorder (with FVA_ROUTE_SCORES_IN in route_flags: plain reorders, routing
    from buf.scores as given).  Inputs [B, N, Hh, d] bf16 on the device;
    the result lands in buf.out.  `table`: a device tile table from
    fva_tile_order (None = raster tile order).  `lse`: optional float32 device
    tensor of B*Hh*N entries for each query's log-sum-exp (reordered positions)."""
    g, B, Hh, d = buf.grid, buf.B, buf.Hh, buf.d
    pool = not (route_flags & FVA_ROUTE_SCORES_IN)
    if pool:
        # Q and K are pooled while they are reordered; the router reads the means
        fva_reorder_pool(q, buf.qr, buf.qbar, B, Hh, d, g, table, token_strides(q),
                         FVA_LAYOUT_ROWS, stream)
        fva_reorder_pool(k, buf.kr, buf.kbar, B, Hh, d, g, table, token_strides(k),
                         FVA_LAYOUT_K64, stream)
    else:
        fva_reorder_ex(q, buf.qr, B, Hh, d, g, table, token_strides(q), FVA_FORWARD,
                       FVA_LAYOUT_ROWS, stream)
        fva_reorder_ex(k, buf.kr, B, Hh, d, g, table, token_strides(k), FVA_FORWARD,
                       FVA_LAYOUT_K64, stream)
    fva_reorder_ex(v, buf.vt, B, Hh, d, g, table, token_strides(v), FVA_FORWARD,
                   FVA_LAYOUT_V64, stream)
    prm = fva_route_params(top_p, topk_floor, aug_budget, scale, 0)
    m = buf.mask()
    if pool:
        fva_route(buf.qbar, buf.kbar, B, Hh, d, g, prm, m, buf.route_ws,
                  buf.sizes.route_ws_bytes, route_flags | FVA_ROUTE_POOLED_IN, stream)
    else:
        fva_route(buf.qr, buf.kr, B, Hh, d, g, prm, m, buf.route_ws, buf.sizes.route_ws_bytes,
                  route_flags, stream)
    fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, B, Hh, d, g, m, scale, attn_flags,
                    buf.attn_ws, buf.sizes.attn_ws_bytes,
                    buf.trace if (attn_flags & FVA_TRACE) else None, stream, lse=lse)
    fva_reorder_ex(buf.orr, buf.out, B, Hh, d, g, table, token_strides(buf.out), FVA_INVERSE,
                   FVA_LAYOUT_ROWS, stream)
    return buf.out


def executed_flops(row_count_sum: int, d: int, BLK: int) -> float:
    """Executed MFMA work of the sparse kernel: QK^T and PV over every
    selected block pair, padded keys included: 4*d*BLK^2 per pair."""
    return 4.0 * d * BLK * BLK * row_count_sum


def dense_equiv_flops(N: int, d: int, Hh: int, B: int = 1) -> float:
    return 4.0 * N * N * d * Hh * B
