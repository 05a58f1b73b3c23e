"""Shared test helpers: tolerance checks and layout marshalling between the
oracle's natural layouts and the C ABI's layouts (no method arithmetic)."""
import numpy as np


def gemm_within_fp32_bound(c, c_ref, s_ref):
    """|C - C_ref| <= 1e-5 * S + 1e-6 elementwise; returns (ok, worst ratio)."""
    c = np.asarray(c, dtype=np.float64)
    err = np.abs(c - c_ref)
    bound = 1e-5 * s_ref + 1e-6
    bad = ~(err <= bound)
    return (not bad.any()), float((err / bound).max()) if err.size else 0.0


def _bf16_round(x64):
    import torch
    return torch.from_numpy(np.asarray(x64, dtype=np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def _bf16_ulp(v):
    """Spacing of BF16 numbers at |v| (2^(e-7) for normal v)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def gemm_within_bf16_bound(c_bf16_as_f64, c_ref, s_ref):
    """Within 1 BF16 ulp of bf16_RNE(C_ref), or, where cancellation makes
    C_ref small, within 1e-5*S + 1e-6 + half a BF16 ulp of C_ref."""
    r = _bf16_round(c_ref)
    c = np.asarray(c_bf16_as_f64, dtype=np.float64)
    ok1 = np.abs(c - r) <= _bf16_ulp(r)
    ok2 = np.abs(c - c_ref) <= 1e-5 * s_ref + 1e-6 + 0.5 * _bf16_ulp(c_ref)
    ok = ok1 | ok2
    return bool(ok.all()), int((~ok).sum())


def tile_scales_to_abi(s_rows_by_kb):
    """oracle [rows][K/128] -> ABI [K/128][rows]."""
    return np.ascontiguousarray(np.asarray(s_rows_by_kb).T)


def sample_rows(rows, tile=128, seed=0):
    """Rows {0, 127, one hashed} of every 128-row tile (clipped to rows)."""
    g = np.random.default_rng(seed)
    out = []
    for r0 in range(0, rows, tile):
        r1 = min(r0 + tile, rows)
        out += [r0, r1 - 1, int(g.integers(r0, r1))]
    return np.unique(np.array(out))
