"""Seeded synthetic workloads for adaptive block-sparse video attention.

This module holds no arithmetic of the method itself.  It only names the
workload shapes and draws the Q/K/V tensors that both the CPU oracle and the
HIP path consume, so that the two can be compared on identical inputs.

Workload shapes follow the FVAttn pages (papers.paperslantern.ai/papers/2607.16190,
section 1 and the abstract): step-distilled Wan2.x image-to-video attention at
480p and 720p latent sizes.  Real Wan activations need trained weights that are
not available, so Q and K are drawn as Gaussian noise plus a per-head-scaled 3-D
sinusoidal position term over the (t, y, x) latent grid; the positional term
makes nearby tokens similar, which is what gives block routing its structure.
The amplitude a_h of that term controls how concentrated a head's attention is
(large a_h -> few dominant key blocks, small a_h -> near-uniform attention).

Layout of every generated tensor: [B, N, Hh, d] bf16, N in raster (t, y, x)
order, i.e. the token-major layout a DiT hands to attention.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hh: int
    d: int
    grid: Tuple[int, int, int]            # (T, H, W) latent grid
    block: Tuple[int, int, int]           # (bt, bh, bw) video-aware block shape
    top_p: float
    topk_floor: int                       # absolute key-block count
    aug_budget: int = 0                   # SASA-style per-head pair budget, 0 = off
    amp: Optional[Tuple[float, ...]] = None   # fixed per-head amplitudes, else U[0, 3]
    seed: int = 0

    @property
    def N(self) -> int:
        T, H, W = self.grid
        return T * H * W

    @property
    def BLK(self) -> int:
        bt, bh, bw = self.block
        return bt * bh * bw

    @property
    def nB(self) -> int:
        return -(-self.N // self.BLK)

    @property
    def Npad(self) -> int:
        return self.nB * self.BLK

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def _nb(grid, block):
    N = grid[0] * grid[1] * grid[2]
    blk = block[0] * block[1] * block[2]
    return -(-N // blk)


def _pct_blocks(frac, grid, block):
    # "k % of key blocks" -> absolute count, rounded up
    return int(math.ceil(frac * _nb(grid, block) - 1e-9))


def _pct_pairs(frac, grid, block):
    nb = _nb(grid, block)
    return int(math.ceil(frac * nb * nb - 1e-9))


_G720 = (21, 45, 80)
_B720 = (1, 8, 16)
_GLONG = (31, 45, 80)
_BLONG = (2, 8, 8)

WORKLOADS = {
    # 2 heads, d 64, 5x16x16 grid, 1x8x8 blocks (20 blocks), fixed amplitudes
    "tiny": Workload("tiny", 1, 2, 64, (5, 16, 16), (1, 8, 8), 0.9, 2, amp=(0.5, 2.5)),
    # 480p-like: 21x30x52 grid (32760 tokens, 8 pad), 1x8x16 blocks
    "480p": Workload("480p", 1, 40, 128, (21, 30, 52), (1, 8, 16), 0.9, 4),
    # 720p-like: 21x45x80 grid (75600 tokens, 48 pad), floor = 8 % of key blocks
    "720p": Workload("720p", 1, 40, 128, _G720, _B720, 0.95,
                     _pct_blocks(0.08, _G720, _B720)),
    # heterogeneity stress: 20 near-uniform heads then 20 concentrated heads
    "hetero": Workload("hetero", 1, 40, 128, _G720, _B720, 0.95, 4,
                       amp=tuple([0.2] * 20 + [4.0] * 20)),
    # long 720p: 31x45x80 grid, 2x8x8 blocks, per-head top-up to 25 % of pairs
    "long720p": Workload("long720p", 1, 40, 128, _GLONG, _BLONG, 0.9, 4,
                         aug_budget=_pct_pairs(0.25, _GLONG, _BLONG)),
}


def small_workload(name, Hh, d, grid, block, top_p, topk_floor, aug_budget=0,
                   amp=None, seed=0) -> Workload:
    """A reduced workload for parity tests (ragged grids, several tiles)."""
    return Workload(name, 1, Hh, d, tuple(grid), tuple(block), top_p, topk_floor,
                    aug_budget, None if amp is None else tuple(amp), seed)


def sinusoid_3d(T: int, H: int, W: int, d: int) -> torch.Tensor:
    """[T*H*W, d] fp32 3-D sinusoidal position term in raster (t, y, x) order.

    d/2 frequency pairs are split between the axes (x and y get floor(F/3),
    t the rest); per axis a, frequency k uses omega = 10000^(-k/F_a); the
    channels are [sin t, cos t, sin y, cos y, sin x, cos x] blocks.
    """
    F = d // 2
    fy = fx = F // 3
    ft = F - fy - fx
    t = torch.arange(T, dtype=torch.float64)
    y = torch.arange(H, dtype=torch.float64)
    x = torch.arange(W, dtype=torch.float64)

    def axis(pos, f):
        om = 10000.0 ** (-torch.arange(f, dtype=torch.float64) / f)
        ang = pos[:, None] * om[None, :]
        return torch.sin(ang), torch.cos(ang)

    st, ct = axis(t, ft)
    sy, cy = axis(y, fy)
    sx, cx = axis(x, fx)
    tt = torch.cat([st, ct], 1)[:, None, None, :].expand(T, H, W, 2 * ft)
    yy = torch.cat([sy, cy], 1)[None, :, None, :].expand(T, H, W, 2 * fy)
    xx = torch.cat([sx, cx], 1)[None, None, :, :].expand(T, H, W, 2 * fx)
    return torch.cat([tt, yy, xx], -1).reshape(T * H * W, d).to(torch.float32)


def amplitudes(w: Workload, g: torch.Generator) -> torch.Tensor:
    if w.amp is not None:
        assert len(w.amp) == w.Hh
        return torch.tensor(w.amp, dtype=torch.float32)
    return torch.rand(w.Hh, generator=g, dtype=torch.float32) * 3.0


def make_qkv(w: Workload, seed: Optional[int] = None):
    """Q, K, V as [B, N, Hh, d] bf16 CPU tensors, drawn in a fixed order:
    amplitudes (when random), Q noise, K noise, V."""
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    a = amplitudes(w, g)
    T, H, W = w.grid
    pe = sinusoid_3d(T, H, W, w.d)                     # [N, d]
    shape = (w.B, w.N, w.Hh, w.d)
    out = []
    for _ in range(2):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        x.add_(a[None, None, :, None] * pe[None, :, None, :])
        out.append(x.to(torch.bfloat16))
        del x
    v = torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return out[0], out[1], v


def make_random(shape: Sequence[int], seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(dtype)
