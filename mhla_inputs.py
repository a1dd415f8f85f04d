"""Seeded synthetic inputs for the MHLA forward (workload table + generators).

This module is shared by the oracle side and the GPU side, so it holds none of
the operator's arithmetic: it only draws Q, K, V and the coefficient matrix,
rounds to bf16 where a workload asks for it, and describes the token grids.

Workloads (shapes follow the image/video settings discussed in "MHLA:
Restoring Expressivity of Linear Attention via Token-Level Multi-Head",
§5.1-§5.3; the data are N(0,1) stand-ins for ImageNet / DiT / Wan latents,
no dataset or trained weight is involved):

  tiny      fp32  B1  H1  N64    (8x8 grid, 4x4 blocks, M=4)       d16 relu
  deit_t    bf16  B64 H3  N196   (14x14 grid, 7x7 blocks, M=4)     d64 elu+1
  dit_xl2   bf16  B32 H16 N256   (16x16 grid, 4x4 blocks, M=16)    d72 relu
  hires     bf16  B4  H16 N4096  (64x64 grid, 8x8 blocks, M=64)    d64 relu
  video     bf16  B1  H24 N32768 (8x64x64 grid, 1x8x8 blocks, M=512) d64 elu+1
  lm_causal bf16  B16 H16 N2048  (1-D, chunks of 64, M=32)         d64 elu+1,
            chunkwise causal form without the normaliser (§5.4: context 2048,
            M = 32; the paper drops the denominator for language modelling)

Draw order per workload (numpy PCG64, seed = 20260 + index): Q, K, V as
standard normal fp32 [B,H,N,d] in C order, then the coefficient logits [H,M,M]
as standard normal fp64.  W = row-softmax(logits) in fp64, stored fp32; the
DeiT-shaped workload adds 2.0 to the diagonal logits first.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

PHI_RELU = 0
PHI_ELU1 = 1
DTYPE_F32 = 0
DTYPE_BF16 = 1
FLAG_NO_NORM = 1   # option bits, the values of the C ABI's MHLA_FLAG_*
FLAG_CAUSAL = 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    H: int
    d: int
    grid: Tuple[int, int, int]   # (T, Hg, Wg); unused leading dims are 1
    block: Tuple[int, int, int]  # (bt, bh, bw)
    phi: int
    dtype: int
    diag_boost: float = 0.0
    flags: int = 0

    @property
    def norm(self) -> bool:
        return not (self.flags & FLAG_NO_NORM)

    @property
    def causal(self) -> bool:
        return bool(self.flags & FLAG_CAUSAL)

    @property
    def nb(self) -> int:
        return self.block[0] * self.block[1] * self.block[2]

    @property
    def N(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def M(self) -> int:
        return ((self.grid[0] // self.block[0]) * (self.grid[1] // self.block[1])
                * (self.grid[2] // self.block[2]))

    @property
    def ndim(self) -> int:
        if self.grid[0] > 1 or self.block[0] > 1:
            return 3
        if self.grid[1] > 1 or self.block[1] > 1:
            return 2
        return 1

    @property
    def seed(self) -> int:
        return 20260 + self.index

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == DTYPE_F32 else 2

    def algorithmic_bytes(self) -> int:
        """Q, K, V read + Y written (input dtype) + W read (fp32)."""
        qkvy = 4 * self.B * self.H * self.N * self.d * self.elt_bytes
        return qkvy + self.H * self.M * self.M * 4

    def algorithmic_flops(self) -> int:
        """B*H*(4*N*d^2 + 2*M^2*d^2): summaries + readout + mixing.  The causal
        form mixes only the lower triangle (M^2 d^2) and adds its own chunk's
        masked token pairs (two products over nb^2/2 pairs: 2*N*nb*d)."""
        d2 = self.d * self.d
        if self.causal:
            return self.B * self.H * (4 * self.N * d2 + self.M * self.M * d2
                                      + 2 * self.N * self.nb * self.d)
        return self.B * self.H * (4 * self.N * d2 + 2 * self.M * self.M * d2)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny", 0, 1, 1, 16, (1, 8, 8), (1, 4, 4), PHI_RELU, DTYPE_F32),
        Workload("deit_t", 1, 64, 3, 64, (1, 14, 14), (1, 7, 7), PHI_ELU1, DTYPE_BF16,
                 diag_boost=2.0),
        Workload("dit_xl2", 2, 32, 16, 72, (1, 16, 16), (1, 4, 4), PHI_RELU, DTYPE_BF16),
        Workload("hires", 3, 4, 16, 64, (1, 64, 64), (1, 8, 8), PHI_RELU, DTYPE_BF16),
        Workload("video", 4, 1, 24, 64, (8, 64, 64), (1, 8, 8), PHI_ELU1, DTYPE_BF16),
        Workload("lm_causal", 5, 16, 16, 64, (1, 1, 2048), (1, 1, 64), PHI_ELU1, DTYPE_BF16,
                 flags=FLAG_NO_NORM | FLAG_CAUSAL),
    ]
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def row_softmax(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


@dataclasses.dataclass
class Inputs:
    """One seeded draw.  For bf16 workloads q/k/v hold the uint16 bf16 bits;
    for fp32 workloads they hold float32.  `*_f64` give the exact values as fp64."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    w: np.ndarray  # float32 [H, M, M]

    def as_f64(self, x: np.ndarray) -> np.ndarray:
        if self.wl.dtype == DTYPE_BF16:
            return bf16_bits_to_f32(x).astype(np.float64)
        return x.astype(np.float64)

    @property
    def q_f64(self):
        return self.as_f64(self.q)

    @property
    def k_f64(self):
        return self.as_f64(self.k)

    @property
    def v_f64(self):
        return self.as_f64(self.v)

    @property
    def w_f64(self):
        return self.w.astype(np.float64)


def make_inputs(wl: Workload, seed: Optional[int] = None, B: Optional[int] = None,
                H: Optional[int] = None) -> Inputs:
    """Draw the workload's inputs.  B/H may be reduced for quick tests (the draw
    then covers only the smaller shape; it is not a slice of the full draw)."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    shape = (B, H, wl.N, wl.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    logits = rng.standard_normal((H, wl.M, wl.M))
    if wl.diag_boost:
        logits = logits + wl.diag_boost * np.eye(wl.M)[None]
    w = row_softmax(logits).astype(np.float32)
    if wl.dtype == DTYPE_BF16:
        q, k, v = bf16_round_bits(q), bf16_round_bits(k), bf16_round_bits(v)
    return Inputs(dataclasses.replace(wl, B=B, H=H), q, k, v, w)


def make_upstream_grad(wl: Workload, B: Optional[int] = None, H: Optional[int] = None,
                       seed: Optional[int] = None) -> np.ndarray:
    """Upstream gradient G = dL/dY for the backward pass: standard normal of the
    output's shape, drawn from its own stream (PCG64, seed = workload seed +
    50000), rounded to bf16 bits for bf16 workloads (fp32 otherwise)."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    rng = np.random.Generator(np.random.PCG64((wl.seed if seed is None else seed) + 50000))
    g = rng.standard_normal((B, H, wl.N, wl.d), dtype=np.float32)
    return bf16_round_bits(g) if wl.dtype == DTYPE_BF16 else g


def custom_workload(B: int, H: int, d: int, grid, block, phi: int, dtype: int,
                    name: str = "custom", index: int = 100, flags: int = 0) -> Workload:
    g = tuple(int(x) for x in grid)
    b = tuple(int(x) for x in block)
    g = (1,) * (3 - len(g)) + g
    b = (1,) * (3 - len(b)) + b
    return Workload(name, index, B, H, d, g, b, phi, dtype, flags=flags)
