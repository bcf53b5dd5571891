"""The C ABI from a plain C11 program (tests/c_consumer.c).

CPU: the program, and with it include/fva.h, compiles as C11 with warnings as
errors.  GPU: the program's pass over the tiny workload (reorder, route from
its own pooled scores, XCD-scheduled attention, inverse reorder) gives the
oracle's masks and output within the attention bar, and the same bits as the
Python binding's pass on the same inputs."""

import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "adaptive_block_sparse_reorder_amd")
SRC = os.path.join(ROOT, "tests", "c_consumer.c")


def _compile(tmp_path, link):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are missing")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include")]
    if link:
        exe = tmp_path / "c_consumer"
        cmd += [SRC, "-o", str(exe), "-L", LIB_DIR, "-lfva", f"-Wl,-rpath,{LIB_DIR}",
                "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    else:
        exe = tmp_path / "c_consumer.o"
        cmd += ["-c", SRC, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_header_and_caller_compile_as_c(tmp_path):
    _compile(tmp_path, link=False)


@pytest.mark.gpu
def test_c_program_runs_the_path(tmp_path):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from adaptive_block_sparse_reorder_amd import fva as F
    from adaptive_block_sparse_reorder_amd.inputs import WORKLOADS, make_qkv
    from oracle import fva_oracle as O

    F.load_library()
    exe = _compile(tmp_path, link=True)
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w)
    inp = tmp_path / "qkv.bin"
    with open(inp, "wb") as f:
        for x in (q, k, v):
            f.write(x.contiguous().view(torch.int16).numpy().tobytes())
    outp = tmp_path / "out.bin"
    args = [str(exe), str(inp), str(outp), *map(str, w.grid), *map(str, w.block), str(w.B),
            str(w.Hh), str(w.d), repr(w.top_p), str(w.topk_floor)]
    print("running", " ".join(args[3:]), flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout, r.stderr)

    raw = outp.read_bytes()
    tok = w.B * w.N * w.Hh * w.d * 2
    rows = w.B * w.Hh * w.nB
    words = (w.nB + 31) // 32
    assert len(raw) == tok + rows * 4 + rows * words * 4
    out_c = np.frombuffer(raw[:tok], dtype=np.int16).reshape(w.B, w.N, w.Hh, w.d)
    counts = np.frombuffer(raw[tok:tok + rows * 4], dtype=np.int32)
    bm = np.frombuffer(raw[tok + rows * 4:], dtype=np.uint32).reshape(rows, words)

    o_ref, ref = O.forward(q.float().numpy(), k.float().numpy(), v.float().numpy(), w.grid,
                           w.block, w.top_p, w.topk_floor, 0)
    mask = np.zeros((rows, w.nB), dtype=bool)
    for j in range(w.nB):
        mask[:, j] = (bm[:, j // 32] >> np.uint32(j % 32)) & 1
    assert np.array_equal(mask, ref["mask"].reshape(rows, w.nB))
    assert np.array_equal(counts, ref["counts"].reshape(-1))
    got = torch.from_numpy(out_c.copy()).view(torch.bfloat16).float().numpy()
    diff = np.abs(got - o_ref)
    assert diff.max() <= 2e-2 and diff.sum() / np.abs(o_ref).sum() <= 5e-3

    # the Python binding's pass on the same inputs gives the same bits
    buf = F.alloc_buffers(w.grid, w.block, w.B, w.Hh, w.d)
    F.forward(buf, q.cuda(), k.cuda(), v.cuda(), w.top_p, w.topk_floor, 0)
    torch.cuda.synchronize()
    assert np.array_equal(buf.out.cpu().view(torch.int16).numpy(), out_c)
