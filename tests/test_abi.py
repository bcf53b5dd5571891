"""The C-ABI library loads and exports every entry point include/fva.h
declares; host-side sizing and validation (no GPU needed: nothing here
launches a kernel)."""

import ctypes
import os

import pytest

from adaptive_block_sparse_reorder_amd import fva as F
from adaptive_block_sparse_reorder_amd.inputs import WORKLOADS


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(F.LIB_PATH):
        from adaptive_block_sparse_reorder_amd import build
        build.build(verbose=False)
    return F.load_library()


def test_exports_every_declared_symbol(lib):
    names = F.header_functions()
    assert set(names) >= {"fva_sizes", "fva_reorder", "fva_route", "fva_sparse_attn",
                          "fva_dense_attn", "fva_status_string", "fva_last_error"}
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("name,N,Npad,nB,words", [
    ("tiny", 1280, 1280, 20, 1), ("480p", 32760, 32768, 256, 8),
    ("720p", 75600, 75648, 591, 19), ("hetero", 75600, 75648, 591, 19),
    ("long720p", 111600, 111616, 872, 28)])
def test_sizes_match_workloads(lib, name, N, Npad, nB, words):
    w = WORKLOADS[name]
    s = F.fva_sizes(F.make_grid(w.grid, w.block), w.B, w.Hh, w.d)
    assert (s.N, s.Npad, s.nB, s.words, s.BLK) == (N, Npad, nB, words, w.BLK)
    assert s.rows == w.B * w.Hh * nB
    assert s.trace_bytes == 32 * s.rows
    assert s.attn_ws_bytes >= 256 + 4 * s.rows
    # route workspace: status word + pooled q, k (float32) + per-head thresholds
    assert s.route_ws_bytes >= 256 + 2 * 4 * s.rows * w.d + 8 * w.Hh


def test_derived_floor_and_budget():
    assert WORKLOADS["720p"].topk_floor == 48          # ceil(0.08 * 591)
    assert WORKLOADS["long720p"].aug_budget == 190096  # 25 % of 872^2 pairs


def test_validation_errors_before_launch(lib):
    g = F.make_grid((5, 16, 16), (1, 8, 8))
    out = F.fva_sizes_t()
    assert lib.fva_sizes(ctypes.byref(g), 1, 2, 96, ctypes.byref(out)) == F.FVA_ERR_UNSUPPORTED
    assert b"head dim" in lib.fva_last_error()
    bad = F.make_grid((5, 16, 16), (1, 4, 8))       # 32-token blocks
    assert lib.fva_sizes(ctypes.byref(bad), 1, 2, 64, ctypes.byref(out)) == F.FVA_ERR_UNSUPPORTED
    neg = F.make_grid((0, 16, 16), (1, 8, 8))
    assert lib.fva_sizes(ctypes.byref(neg), 1, 2, 64, ctypes.byref(out)) == F.FVA_ERR_INVALID_ARG
    big = F.make_grid((64, 256, 128), (1, 8, 8))    # 32768 blocks: past int16 column indices
    assert lib.fva_sizes(ctypes.byref(big), 1, 2, 64, ctypes.byref(out)) == F.FVA_ERR_UNSUPPORTED
    assert b"32767" in lib.fva_last_error()
    most = F.make_grid((1, 1, 32767 * 64), (1, 1, 64))  # the largest block count
    assert lib.fva_sizes(ctypes.byref(most), 1, 2, 64, ctypes.byref(out)) == F.FVA_OK
    assert out.nB == 32767 and out.words == 1024
    st = (ctypes.c_int64 * 3)(1280 * 2 * 64, 2 * 64, 64)
    # null pointers
    assert lib.fva_reorder(None, None, 1, 2, 64, ctypes.byref(g), st, 0, 0, None) == \
        F.FVA_ERR_INVALID_ARG
    # misaligned stride
    st2 = (ctypes.c_int64 * 3)(1280 * 2 * 64, 2 * 64, 63)
    assert lib.fva_reorder(16, 32, 1, 2, 64, ctypes.byref(g), st2, 0, 0, None) == \
        F.FVA_ERR_INVALID_ARG
    # the inverse writes the token-major layout only
    assert lib.fva_reorder(16, 32, 1, 2, 64, ctypes.byref(g), st, 1, 1, None) == \
        F.FVA_ERR_INVALID_ARG
    # route: workspace too small, negative floor, bad flags
    m = F.fva_mask(16, 16, 16, 16, 16, 16)
    prm = F.fva_route_params(0.9, 2, 0, 0.0, 0)
    assert lib.fva_route(16, 16, 1, 2, 64, ctypes.byref(g), ctypes.byref(prm), ctypes.byref(m),
                         256, 8, 0, None) == F.FVA_ERR_WORKSPACE
    prm2 = F.fva_route_params(0.9, -1, 0, 0.0, 0)
    assert lib.fva_route(16, 16, 1, 2, 64, ctypes.byref(g), ctypes.byref(prm2), ctypes.byref(m),
                         256, 1 << 30, 0, None) == F.FVA_ERR_INVALID_ARG
    assert lib.fva_route(16, 16, 1, 2, 64, ctypes.byref(g), ctypes.byref(prm), ctypes.byref(m),
                         256, 1 << 30, 0x8, None) == F.FVA_ERR_INVALID_ARG
    m0 = F.fva_mask(16, 0, 16, 16, 16, 16)
    assert lib.fva_route(16, 16, 1, 2, 64, ctypes.byref(g), ctypes.byref(prm), ctypes.byref(m0),
                         256, 1 << 30, 0, None) == F.FVA_ERR_INVALID_ARG
    # attention: bad schedule flag, missing workspace, trace without buffer
    big_ws = 1 << 20
    assert lib.fva_sparse_attn(16, 16, 16, 16, 1, 2, 64, ctypes.byref(g), ctypes.byref(m), 0.0,
                               0x4, 256, big_ws, None, None, None) == F.FVA_ERR_INVALID_ARG
    assert lib.fva_sparse_attn(16, 16, 16, 16, 1, 2, 64, ctypes.byref(g), ctypes.byref(m), 0.0,
                               0, None, 0, None, None, None) == F.FVA_ERR_WORKSPACE
    assert lib.fva_sparse_attn(16, 16, 16, 16, 1, 2, 64, ctypes.byref(g), ctypes.byref(m), 0.0,
                               0, 256, 64, None, None, None) == F.FVA_ERR_WORKSPACE
    assert lib.fva_sparse_attn(16, 16, 16, 16, 1, 2, 64, ctypes.byref(g), ctypes.byref(m), 0.0,
                               F.FVA_TRACE, 256, big_ws, None, None, None) == F.FVA_ERR_INVALID_ARG
    # a log-sum-exp buffer must be 4-byte aligned
    assert lib.fva_sparse_attn(16, 16, 16, 16, 1, 2, 64, ctypes.byref(g), ctypes.byref(m), 0.0,
                               0, 256, big_ws, None, 18, None) == F.FVA_ERR_INVALID_ARG
    assert lib.fva_dense_attn(16, 16, 16, 16, 1, 2, 64, ctypes.byref(g), 0.0, 18, None) == \
        F.FVA_ERR_INVALID_ARG
    # the XCD schedule caps the number of heads
    many = F.make_grid((2, 8, 8), (1, 8, 8))
    assert lib.fva_sparse_attn(256, 256, 256, 256, 1, 5000, 64, ctypes.byref(many),
                               ctypes.byref(m), 0.0, F.FVA_SCHED_XCD, 256, 1 << 30, None,
                               None, None) == F.FVA_ERR_UNSUPPORTED
    assert lib.fva_dense_attn(16, 16, 0, 16, 1, 2, 64, ctypes.byref(g), 0.0, None, None) == \
        F.FVA_ERR_INVALID_ARG
    assert lib.fva_status_string(F.FVA_ERR_WORKSPACE) == b"FVA_ERR_WORKSPACE"


def test_tile_table_sizes_and_limits(lib):
    # the documented layout: a 12-word header {ntiles, order, status, T, H, W,
    # bt, bh, bw, 0, 0, 0}, ntiles raster ids, ntiles + 1 starts
    g = F.make_grid((3, 13, 19), (1, 8, 8))          # 3 x 2 x 3 = 18 tiles, clipped in y and x
    nbytes = ctypes.c_size_t(0)
    assert lib.fva_tile_order_bytes(ctypes.byref(g), ctypes.byref(nbytes)) == F.FVA_OK
    need = nbytes.value
    assert need == 48 + 4 * 18 + 4 * 19
    assert lib.fva_tile_order_bytes(ctypes.byref(g), None) == F.FVA_ERR_INVALID_ARG
    # heavy clipping: 15000 frames of a 1 x 17 strip with 1x8x16 tiles give 30000
    # tiles but only 1993 blocks, past the tile table's 8192-tile capacity
    many = F.make_grid((15000, 1, 17), (1, 8, 16))
    s = F.fva_sizes(many, 1, 1, 64)
    assert s.nB == 1993
    assert lib.fva_tile_order_bytes(ctypes.byref(many), ctypes.byref(nbytes)) == \
        F.FVA_ERR_UNSUPPORTED
    assert lib.fva_tile_order(ctypes.byref(many), F.FVA_ORDER_HILBERT, 256, 1 << 20, None) == \
        F.FVA_ERR_UNSUPPORTED
    st = (ctypes.c_int64 * 3)(64, 64, 64)
    assert lib.fva_reorder_ex(256, 512, 1, 1, 64, ctypes.byref(many), 1024, st, F.FVA_FORWARD,
                              F.FVA_LAYOUT_ROWS, None) == F.FVA_ERR_UNSUPPORTED
    # table too small, unknown order, misaligned table: rejected before any launch
    assert lib.fva_tile_order(ctypes.byref(g), F.FVA_ORDER_HILBERT, 256, need - 4, None) == \
        F.FVA_ERR_WORKSPACE
    assert lib.fva_tile_order(ctypes.byref(g), 7, 256, 1 << 20, None) == F.FVA_ERR_INVALID_ARG
    assert lib.fva_tile_order(ctypes.byref(g), F.FVA_ORDER_HILBERT, 264, 1 << 20, None) == \
        F.FVA_ERR_INVALID_ARG
    # a misaligned table is refused by the reorder and the status read too
    assert lib.fva_reorder_ex(256, 512, 1, 1, 64, ctypes.byref(g), 1028, st, F.FVA_FORWARD,
                              F.FVA_LAYOUT_ROWS, None) == F.FVA_ERR_INVALID_ARG
    out = ctypes.c_int32(0)
    assert lib.fva_tile_table_status(None, ctypes.byref(out), None) == F.FVA_ERR_INVALID_ARG
    assert lib.fva_tile_table_status(1028, ctypes.byref(out), None) == F.FVA_ERR_INVALID_ARG
    assert lib.fva_tile_table_status(1024, None, None) == F.FVA_ERR_INVALID_ARG


def test_probe_library_exports_and_checks_arguments():
    # the benchmark's matrix-core probe: a library of its own, every symbol its
    # header declares exported, bad arguments refused before any launch
    import re
    path = os.path.join(os.path.dirname(F.LIB_PATH), "libfva_probe.so")
    if not os.path.exists(path):
        from adaptive_block_sparse_reorder_amd import build
        build.build(verbose=False)
    lib = ctypes.CDLL(path)
    hdr = open(os.path.join(os.path.dirname(F.HEADER), "fva_probe.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = sorted(set(re.findall(r"\b(fva_probe_[a-z_]+)\s*\(", hdr)))
    assert names == ["fva_probe_mfma", "fva_probe_operand_bytes", "fva_probe_output_bytes"]
    for n in names:
        assert hasattr(lib, n), n
    lib.fva_probe_operand_bytes.restype = ctypes.c_size_t
    lib.fva_probe_output_bytes.restype = ctypes.c_size_t
    assert lib.fva_probe_operand_bytes(2) == 2 * 512 * 32
    assert lib.fva_probe_output_bytes(2) == 2 * 512 * 4
    assert lib.fva_probe_operand_bytes(0) == 0
    f = lib.fva_probe_mfma
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert f(None, 256, 1, 1, None) == -1
    assert f(256, 256, 0, 1, None) == -1
    assert f(256, 256, 1, 0, None) == -1
    assert f(264, 256, 1, 1, None) == -1
