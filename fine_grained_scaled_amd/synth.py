"""Seeded synthetic operands with the pages' workload shapes and statistics.

This module only draws random numbers and rounds them to BF16; it holds none
of the quantization or GEMM arithmetic, so both the GPU path and the CPU
oracle can be fed from it.

Recipe (every stream is numpy's default generator seeded with
``SeedSequence([seed, tag, chunk])``, where chunk is a fixed 512-row block
index so any row range can be regenerated on its own):
  activations  N(0, 1) in float32, with round(0.001 * cols) outlier channels
               (tag OUTLIER, chosen uniformly without replacement, the same
               channels for every row) multiplied by 50 before BF16 rounding;
  weights      N(0, 0.02) (sigma = 0.02);
  gradients    Student-t with 3 degrees of freedom scaled to std 1e-3,
               i.e. t3 * 1e-3 / sqrt(3);
  expert counts Multinomial(tokens, p_r proportional to r^-1.1), r = 1..experts.
Values are rounded to BF16 with round-to-nearest-even (torch's conversion).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TAG_A, TAG_W, TAG_DY, TAG_OUTLIER, TAG_COUNTS, TAG_RHT, TAG_SR = 1, 2, 3, 4, 5, 6, 7
CHUNK_ROWS = 512


def _rng(seed: int, tag: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tag, *extra]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (nearest-even) and return the bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def outlier_channels(cols: int, seed: int = 0) -> np.ndarray:
    k = int(round(0.001 * cols))
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(seed, TAG_OUTLIER, cols).choice(cols, size=k, replace=False))


def _draw(kind: str, seed: int, tag: int, cols: int, chunk: int, n_rows: int, sigma: float):
    g = _rng(seed, tag, chunk)
    if kind == "normal":
        v = g.standard_normal((n_rows, cols), dtype=np.float32)
        if sigma != 1.0:
            v *= np.float32(sigma)
        return v
    if kind == "t3":
        return (g.standard_t(3, size=(n_rows, cols)) * (1e-3 / math.sqrt(3.0))).astype(np.float32)
    raise ValueError(kind)


def _matrix(kind, rows, cols, seed, tag, sigma=1.0, row_range=None, outliers=False, threads=8):
    r0, r1 = (0, rows) if row_range is None else row_range
    out = np.empty((r1 - r0, cols), dtype=np.uint16)
    chans = outlier_channels(cols, seed) if outliers else None
    chunks = list(range(r0 // CHUNK_ROWS, (r1 + CHUNK_ROWS - 1) // CHUNK_ROWS))

    def work(ch):
        c0 = ch * CHUNK_ROWS
        n = min(CHUNK_ROWS, rows - c0)
        v = _draw(kind, seed, tag, cols, ch, n, sigma)
        if chans is not None and len(chans):
            v[:, chans] *= np.float32(50.0)
        lo, hi = max(r0, c0), min(r1, c0 + n)
        out[lo - r0:hi - r0] = f32_to_bf16_bits(v[lo - c0:hi - c0])

    if len(chunks) > 1 and threads > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, chunks))
    else:
        for ch in chunks:
            work(ch)
    return out


def activations(rows, cols, seed=0, outliers=True, row_range=None, tag=TAG_A):
    """BF16 bits ~ N(0, 1) with x50 outlier channels."""
    return _matrix("normal", rows, cols, seed, tag, 1.0, row_range, outliers)


def weights(rows, cols, seed=0, sigma=0.02, row_range=None, tag=TAG_W):
    """BF16 bits ~ N(0, sigma)."""
    return _matrix("normal", rows, cols, seed, tag, sigma, row_range)


def gradients(rows, cols, seed=0, row_range=None, tag=TAG_DY):
    """BF16 bits ~ Student-t(3) scaled to std 1e-3."""
    return _matrix("t3", rows, cols, seed, tag, 1.0, row_range)


def normal_gradients(rows, cols, seed=0, row_range=None, tag=TAG_DY):
    """BF16 bits ~ N(0, 1) (gradients distributed like the activations)."""
    return _matrix("normal", rows, cols, seed, tag, 1.0, row_range)


def expert_counts(tokens=32768, experts=256, alpha=1.1, seed=0) -> np.ndarray:
    """Per-expert row counts ~ Multinomial(tokens, p_r ~ r^-alpha)."""
    p = np.arange(1, experts + 1, dtype=np.float64) ** (-alpha)
    p /= p.sum()
    return _rng(seed, TAG_COUNTS).multinomial(tokens, p).astype(np.int64)


def derived_seed(seed: int, tag: int) -> int:
    """A 64-bit seed for the Hadamard signs (TAG_RHT) or SR words (TAG_SR)."""
    return int(np.random.SeedSequence([seed, tag]).generate_state(1, dtype=np.uint64)[0])


def to_torch_bf16(bits: np.ndarray):
    """Reinterpret BF16 bit patterns as a torch bfloat16 CPU tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
