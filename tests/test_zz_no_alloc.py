"""fva_sparse_attn_noalloc: the attention entry point that takes its workspace
from the library's own static device array instead of a caller buffer.  It
runs the same kernels as fva_sparse_attn, so its outputs (and log-sum-exp and
trace) must be bit-identical to that entry point's on the same mask, for every
schedule; checked on two problems in a row, the second smaller, so the second
call reuses the array the first one left behind.  The size limit is checked
on the host before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

from adaptive_block_sparse_reorder_amd import fva as F
from adaptive_block_sparse_reorder_amd.inputs import make_qkv, small_workload

SCHEDS = (F.FVA_SCHED_XCD, F.FVA_SCHED_QUEUE, F.FVA_SCHED_STATIC, F.FVA_SCHED_GRID)


def _workloads():
    # first call: 816 rows (more than the resident workgroups, so the XCD plan
    # and the queue counter live in the array); second call: 66 rows
    big = small_workload("noalloc-big", 8, 128, (3, 33, 131), (1, 8, 16), 0.9, 2,
                         amp=(0.2, 3.0, 1.2, 2.4, 0.6, 4.0, 1.8, 0.1))
    small = small_workload("noalloc-small", 3, 64, (3, 13, 19), (1, 8, 8), 0.8, 1)
    return big, small


def _prepared(w):
    q, k, v = make_qkv(w)
    buf = F.alloc_buffers(w.grid, w.block, w.B, w.Hh, w.d, trace=True)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    g = buf.grid
    for x, dst, lay in ((qd, buf.qr, F.FVA_LAYOUT_ROWS), (kd, buf.kr, F.FVA_LAYOUT_K64),
                        (vd, buf.vt, F.FVA_LAYOUT_V64)):
        F.fva_reorder(x, dst, w.B, w.Hh, w.d, g, F.token_strides(x), F.FVA_FORWARD, lay)
    prm = F.fva_route_params(w.top_p, w.topk_floor, w.aug_budget, 0.0, 0)
    F.fva_route(buf.qr, buf.kr, w.B, w.Hh, w.d, g, prm, buf.mask(), buf.route_ws,
                buf.sizes.route_ws_bytes, 0)
    return buf


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_point_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    F.load_library()
    for w in _workloads():
        buf = _prepared(w)
        nq = w.B * w.Hh * w.N
        print(f"{w.name}: rows={int(buf.sizes.rows)} attn_ws_bytes={int(buf.sizes.attn_ws_bytes)}",
              flush=True)
        assert buf.sizes.attn_ws_bytes <= F.FVA_NOALLOC_ATTN_WS_MAX
        for fl in SCHEDS:
            ref_lse = torch.full((nq,), float("nan"), dtype=torch.float32, device="cuda")
            buf.orr.fill_(float("nan"))
            buf.trace.zero_()
            F.fva_sparse_attn(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, buf.grid,
                              buf.mask(), 0.0, fl | F.FVA_TRACE, buf.attn_ws,
                              buf.sizes.attn_ws_bytes, buf.trace, lse=ref_lse)
            torch.cuda.synchronize()
            ref = buf.orr.clone()
            ref_rows = buf.trace.view(torch.int32).reshape(-1, 8)[:buf.sizes.rows, 0].clone()
            got_lse = torch.full((nq,), float("nan"), dtype=torch.float32, device="cuda")
            buf.orr.fill_(float("nan"))
            buf.trace.zero_()
            F.fva_sparse_attn_noalloc(buf.qr, buf.kr, buf.vt, buf.orr, w.B, w.Hh, w.d, buf.grid,
                                      buf.mask(), 0.0, fl | F.FVA_TRACE, buf.trace, lse=got_lse)
            torch.cuda.synchronize()
            assert torch.equal(buf.orr.view(torch.int16), ref.view(torch.int16)), (w.name, fl)
            assert torch.equal(got_lse.view(torch.int32), ref_lse.view(torch.int32)), (w.name, fl)
            rows = buf.trace.view(torch.int32).reshape(-1, 8)[:buf.sizes.rows, 0]
            assert sorted(rows.cpu().tolist()) == list(range(int(buf.sizes.rows))), (w.name, fl)
            assert torch.equal(rows, ref_rows), (w.name, fl)
            assert bool(torch.isfinite(buf.orr[:, :, :w.N]).all())
        del buf
        torch.cuda.empty_cache()


def test_noalloc_refuses_problems_beyond_its_array():
    # host-side check, before anything touches the device: 200 heads of 2048
    # blocks need 1.6 MB of workspace, more than the static array holds
    lib = F.load_library()
    g = F.make_grid((16, 128, 128), (1, 8, 16))
    s = F.fva_sizes(g, 1, 200, 128)
    assert s.nB == 2048 and s.attn_ws_bytes > F.FVA_NOALLOC_ATTN_WS_MAX
    m = F.fva_mask(256, 256, 256, 256, 256, 256)
    st = lib.fva_sparse_attn_noalloc(256, 256, 256, 256, 1, 200, 128, ctypes.byref(g),
                                     ctypes.byref(m), 0.0, F.FVA_SCHED_QUEUE, None, None, None)
    assert st == F.FVA_ERR_UNSUPPORTED
    assert b"workspace" in lib.fva_last_error()
    # the ordinary argument checks come first
    st = lib.fva_sparse_attn_noalloc(None, 256, 256, 256, 1, 2, 64, ctypes.byref(g),
                                     ctypes.byref(m), 0.0, F.FVA_SCHED_QUEUE, None, None, None)
    assert st == F.FVA_ERR_INVALID_ARG
    st = lib.fva_sparse_attn_noalloc(256, 256, 256, 256, 1, 2, 64, ctypes.byref(g),
                                     ctypes.byref(m), 0.0, 0x40, None, None, None)
    assert st == F.FVA_ERR_INVALID_ARG
