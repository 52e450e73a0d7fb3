"""Seeded synthetic workloads for 3D-RoPE video-DiT attention.

This module only draws and stores numbers: it holds the workload shapes
and the seeded generators that both the oracle tests and the HIP path use.
It contains none of the method's arithmetic (no norm, rotation, softmax or
state update), so importing it couples neither side to the other.

Recipe (used everywhere): ``numpy.random.default_rng(seed)`` (PCG64); tensors
are drawn in the order q, k, v, each ``standard_normal(shape)`` in C order of
the ``[B, L, H, D]`` layout, float64 -> float32, then (for bf16 workloads)
float32 -> bfloat16 with round-to-nearest-even.  Values come back as float64
arrays holding exactly the rounded numbers, plus the raw bf16 bit patterns.
The default seed of a workload is 1000 + its number.

The "structured" variant replaces each tensor by a 3-tap box average along
t, h and w of the latent grid, so neighbouring tokens correlate the way the
pages observe for real video latents (Kaleido review, "The pith": attention
maps with spatial tiles and temporal diagonals).  It is used for parity only.
"""
from __future__ import annotations

import dataclasses

from typing import Optional

import numpy as np


# ---------------------------------------------------------------- bfloat16 --

def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------- workloads --

@dataclasses.dataclass(frozen=True)
class Workload:
    number: int
    name: str
    mode: str                 # "full" | "ring" | "rolling" | "hybrid"
    dtype: str                # "bf16" | "f32"
    grid: tuple               # (T, H, W) latent grid of the whole sequence
    heads: int
    kv_heads: int
    head_dim: int
    pairs: tuple              # RoPE channel pairs per axis (t, h, w)
    theta: float = 10000.0
    # ring: query tokens [q0, q0+Lq); key chunks as (start, length) in the grid
    q_range: Optional[tuple] = None
    kv_chunks: Optional[tuple] = None
    # rolling: window of n_slots frames, frames streamed
    n_slots: int = 0
    n_frames: int = 0
    # hybrid: tokens per chunk
    chunk_tokens: int = 0
    # rolling: per-head RMSNorm of keys and values, queries rotated only
    kv_norm: bool = False
    # hybrid: keys before each chunk that join its softmax window
    overlap_tokens: int = 0

    @property
    def tokens(self) -> int:
        T, H, W = self.grid
        return T * H * W

    @property
    def seed(self) -> int:
        return 1000 + self.number


WORKLOADS = {
    1: Workload(1, "tiny_full_f32", "full", "f32", (3, 4, 6), 2, 2, 64, (12, 10, 10)),
    2: Workload(2, "wan1.3b_full_32760", "full", "bf16", (21, 30, 52), 12, 12, 128, (22, 21, 21)),
    3: Workload(3, "wan14b_ring_shard_15600x2", "ring", "bf16", (20, 30, 52), 10, 10, 128, (22, 21, 21),
                q_range=(0, 15600), kv_chunks=((0, 15600), (15600, 15600))),
    4: Workload(4, "rolling_decode_2040x5", "rolling", "bf16", (1, 34, 60), 16, 16, 64, (12, 10, 10),
                n_slots=5, n_frames=64),
    5: Workload(5, "hybrid_chunk_12090", "hybrid", "bf16", (31, 15, 26), 24, 24, 128, (22, 21, 21),
                chunk_tokens=1170),
    # FlashDecoder-XL decode at 720p: 45 x 80 latent tokens per frame, 24 query
    # heads in 3 KV groups, head dim 1536 / 24 = 64, window of 2 frames, KV-norm
    6: Workload(6, "flashdecoder_xl_rolling_720p_3600x2", "rolling", "bf16", (1, 45, 80), 24, 3, 64,
                (12, 10, 10), n_slots=2, n_frames=16, kv_norm=True),
    # its temporal refinement: steps of r_t = 4 sub-frames, window 2 steps = 8 sub-frames
    7: Workload(7, "flashdecoder_xl_refine_720p_4x3600x2", "rolling", "bf16", (4, 45, 80), 24, 3, 64,
                (12, 10, 10), n_slots=2, n_frames=6, kv_norm=True),
    # the chunk-hybrid with MobileWan's chunk of T_c = 4 latent frames and a
    # softmax overlap of T_o = 2 frames (390 tokens per frame)
    8: Workload(8, "hybrid_overlap_12090_c4_o2", "hybrid", "bf16", (31, 15, 26), 24, 24, 128, (22, 21, 21),
                chunk_tokens=4 * 390, overlap_tokens=2 * 390),
}


def poly_phi_coefficients(head_dim: int) -> tuple:
    """Synthetic coefficients (a0..a3, b0..b3) of degree-3 feature maps phi_q,
    phi_k for the chunk-hybrid's linear term (the pages give the degree, not
    the learned values).  In y = x / R with R = sqrt(head_dim) (1 + 2^-7), the
    largest element of a row RMS-normalised with gain 1 (and rounded to
    bf16), they are 1 + y/2 + y^2/4 + y^3/8 and 1 - y/3 + y^2/5 + y^3/10, both
    between 0.6 and 1.9 on [-1, 1]; returned as float32-representable
    numbers in powers of x."""
    R = float(np.sqrt(head_dim)) * (1.0 + 2.0 ** -7)
    py = (1.0, 1 / 2, 1 / 4, 1 / 8, 1.0, -1 / 3, 1 / 5, 1 / 10)
    c = [py[i] / R ** (i % 4) for i in range(8)]
    return tuple(float(np.float32(x)) for x in c)


def hybrid_flops(w: "Workload") -> float:
    """Matmul FLOPs of the chunk-hybrid's softmax part: each chunk's queries
    against its window (its own keys plus the overlap before them)."""
    total = 0.0
    for c0 in range(0, w.tokens, w.chunk_tokens):
        c1 = min(w.tokens, c0 + w.chunk_tokens)
        total += flops_full(c1 - c0, c1 - max(0, c0 - w.overlap_tokens), w.heads, w.head_dim)
    return total


def flops_full(Lq: int, Lkv: int, heads: int, D: int, B: int = 1) -> float:
    """Matmul FLOPs of exact attention: QK^T plus PV, 2 FLOP per multiply-add."""
    return 4.0 * B * heads * Lq * Lkv * D


@dataclasses.dataclass
class Tensor:
    """A drawn tensor: exact float64 values and, for bf16, the raw bits."""
    values: np.ndarray
    bits: Optional[np.ndarray]
    dtype: str


def _box3(x: np.ndarray, grid: tuple) -> np.ndarray:
    # 3-tap box average along each grid axis (edges replicate); input [B,L,H,D]
    B, L, Hh, D = x.shape
    T, H, W = grid
    g = x.reshape(B, T, H, W, Hh, D)
    for ax in (1, 2, 3):
        if g.shape[ax] < 2:
            continue
        pad = [(0, 0)] * g.ndim
        pad[ax] = (1, 1)
        p = np.pad(g, pad, mode="edge")
        n = g.shape[ax]
        sl = lambda a, b: tuple(slice(a, b) if i == ax else slice(None) for i in range(g.ndim))
        g = (p[sl(0, n)] + p[sl(1, n + 1)] + p[sl(2, n + 2)]) / 3.0
    # restore unit variance so the structured field has the same scale
    g = g / max(g.std(), 1e-30)
    return g.reshape(B, L, Hh, D)


def draw(shape, rng: np.random.Generator, dtype: str, structured_grid: Optional[tuple] = None) -> Tensor:
    x = rng.standard_normal(shape)
    if structured_grid is not None:
        x = _box3(x, structured_grid)
    x32 = x.astype(np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Tensor(bf16_bits_to_f64(bits), bits, dtype)
    return Tensor(x32.astype(np.float64), None, dtype)


def draw_qkv(shape_q, shape_k, seed: int, dtype: str, structured_grid: Optional[tuple] = None):
    """Draw q, k, v in that order from one generator."""
    rng = np.random.default_rng(seed)
    q = draw(shape_q, rng, dtype, structured_grid)
    k = draw(shape_k, rng, dtype, structured_grid)
    v = draw(shape_k, rng, dtype, structured_grid)
    return q, k, v


def workload_inputs(w: Workload, seed: Optional[int] = None, structured: bool = False):
    """Raw (pre-norm, pre-rotation) q, k, v for a workload, over its whole grid.

    Rolling workloads draw [n_frames, L_step, H, D] per tensor, step-major
    (L_step = tokens of the per-step grid).
    """
    seed = w.seed if seed is None else seed
    if w.mode == "rolling":
        L = w.tokens
        shape = (w.n_frames, L, w.heads, w.head_dim)
        shape_k = (w.n_frames, L, w.kv_heads, w.head_dim)
        sg = None
        return draw_qkv(shape, shape_k, seed, w.dtype, sg)
    shape = (1, w.tokens, w.heads, w.head_dim)
    shape_k = (1, w.tokens, w.kv_heads, w.head_dim)
    return draw_qkv(shape, shape_k, seed, w.dtype, w.grid if structured else None)


def sample_rows(n_total: int, n_sample: int, seed: int) -> np.ndarray:
    """Seeded sorted sample of row indices (used for full-size spot checks)."""
    rng = np.random.default_rng(seed)
    n_sample = min(n_sample, n_total)
    return np.sort(rng.choice(n_total, size=n_sample, replace=False))


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [
    "Workload", "WORKLOADS", "Tensor", "draw", "draw_qkv", "workload_inputs",
    "f32_to_bf16_bits", "bf16_bits_to_f64", "flops_full", "hybrid_flops", "sample_rows", "ceil_div",
    "poly_phi_coefficients",
]

