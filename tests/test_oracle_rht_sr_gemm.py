"""Pins of the oracle's random Hadamard transform, stochastic rounding and
GEMM reference.

The random 16x16 Hadamard transforms of gradient inputs and the stochastic
rounding come from "NVIDIA developed a method to train neural networks at
4-bit", section "How it works".  The GEMM with block scales and FP32
promotion of partial sums comes from "Can you explain the role of FP8
precision in DeepSeek-V3 training", sections "Mixed precision framework"
(GEMMs in FP8) and "Increasing accumulation precision".
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
from fine_grained_scaled_amd import synth


def _rht_matrix(seed):
    """Columns of the transform, from the oracle applied to unit vectors."""
    eye = np.eye(16, dtype=np.float32)
    return oracle.rht_rows(eye, seed).T.astype(np.float64)   # T[:, j] = rht(e_j)


@pytest.mark.parametrize("seed", [0, 1, 0xDEADBEEF, 2**63 + 12345])
def test_rht_is_quarter_sylvester_times_signs(seed):
    t = _rht_matrix(seed)
    d = oracle.rht_signs(seed).astype(np.float64)
    assert set(np.unique(d)) <= {-1.0, 1.0}
    h = scipy.linalg.hadamard(16).astype(np.float64)           # library Sylvester H16
    assert np.array_equal(t, 0.25 * h @ np.diag(d))
    assert np.array_equal(h @ h.T, 16 * np.eye(16))            # H H^T = 16 I
    assert np.array_equal(t @ t.T, np.eye(16))                 # orthonormal, exactly


def test_rht_signs_depend_on_seed():
    seen = {tuple(oracle.rht_signs(s)) for s in range(64)}
    assert len(seen) > 32
    assert any(-1.0 in s for s in seen) and any(1.0 in s for s in seen)


def test_rht_butterfly_vs_dense_fp64_and_dot_products():
    g = np.random.default_rng(0)
    x = g.standard_normal((200, 64)).astype(np.float32) * np.float32(3.0)
    y = g.standard_normal((200, 64)).astype(np.float32)
    seed = 77
    tx = oracle.rht_rows(x, seed).astype(np.float64)
    ty = oracle.rht_rows(y, seed).astype(np.float64)
    t = _rht_matrix(seed)
    for c in range(0, 64, 16):
        dense = x[:, c:c + 16].astype(np.float64) @ t.T
        bound = 4 * 2.0 ** -24 * np.abs(x[:, c:c + 16].astype(np.float64)).sum(axis=1, keepdims=True)
        assert np.all(np.abs(tx[:, c:c + 16] - dense) <= bound)
    dots = (x.astype(np.float64) * y).sum(axis=1)
    dots_t = (tx * ty).sum(axis=1)
    scale = (np.abs(x).astype(np.float64) * np.abs(y)).sum(axis=1)
    assert np.all(np.abs(dots - dots_t) <= 1e-5 * scale)


INTERVALS = [(0.0, 0.5), (0.5, 1.0), (1.0, 1.5), (1.5, 2.0), (2.0, 3.0), (3.0, 4.0), (4.0, 6.0)]


@pytest.mark.parametrize("lo,hi", INTERVALS)
def test_sr_unbiased(lo, hi):
    """Over 10^6 trials mean(SR(y)) = y within 5 sigma, and P(up) = p."""
    n = 1_000_000
    tab = oracle.e2m1_decode_table()
    for frac in (0.1, 0.5, 0.83):
        y = np.float32(lo + frac * (hi - lo))
        p = (float(y) - lo) / (hi - lo)
        words = oracle.sr_words(0xABCDEF, np.arange(n, dtype=np.uint64) + 7 * 2**32)
        for sign in (1.0, -1.0):
            codes = oracle.e2m1_encode(np.full(n, sign * y, dtype=np.float32), words)
            vals = tab[codes]
            up = np.mean(np.abs(vals) == hi)
            sigma = math.sqrt(p * (1 - p) / n)
            assert abs(up - p) <= 5 * sigma
            assert abs(vals.mean() - sign * float(y)) <= 5 * (hi - lo) * sigma + 1e-12
            assert np.all((np.abs(vals) == lo) | (np.abs(vals) == hi))


def test_sr_keeps_representable_values():
    tab = oracle.e2m1_decode_table()
    vals = tab.astype(np.float32)
    words = oracle.sr_words(5, np.arange(16, dtype=np.uint64))
    for w in (0, 0xFFFFFFFF):
        assert np.array_equal(tab[oracle.e2m1_encode(vals, np.full(16, w, np.uint32))], tab)
    assert np.array_equal(tab[oracle.e2m1_encode(vals, words)], tab)


# FP32 bit patterns across every E2M1 interval: plain fractions of a step,
# values just above a grid point or just below the next, values with low
# mantissa bits below 1 (where p * 2^22 is not an integer), the smallest
# subnormal, and 3.4 (an inexact FP32 value)
SR_BITS = [0x3DCCCCCD, 0x3E800001, 0x3EFFFFFF, 0x3F000001, 0x3F000003, 0x3F2AAAAB, 0x3F7FFFFF,
           0x3F800001, 0x3FA00000, 0x3FD55555, 0x3FFFFFFF, 0x40200001, 0x4059999A, 0x409FFFFF,
           0x40A00000, 0x40BFFFFF, 0x3A83126F, 0x00000001]
SR_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


@pytest.mark.parametrize("bits", SR_BITS)
def test_sr_up_count_over_all_variates(bits):
    """Over every one of the 2^22 values of the variate (r >> 10; the low 10
    bits of r random), SR rounds y up for exactly floor(p * 2^22) of them,
    p = (|y| - lo) / (hi - lo) taken in exact rational arithmetic.  For
    |y| >= 1 that count is p * 2^22 itself, so the mean of SR(y) over the
    variates is y exactly; below 1 it falls short of y by less than 2^-22
    of the grid step and never exceeds it."""
    y = np.array([bits], dtype=np.uint32).view(np.float32)[0]
    yq = Fraction(float(y))
    lo = max(Fraction(v) for v in SR_GRID if Fraction(v) <= yq)
    hi = min(Fraction(v) for v in SR_GRID if Fraction(v) > yq)
    p = (yq - lo) / (hi - lo)
    expect = math.floor(p * 2**22)
    g = np.random.default_rng(bits)
    k = np.arange(1 << 22, dtype=np.uint32)
    r = (k << np.uint32(10)) | g.integers(0, 1024, k.size, dtype=np.uint64).astype(np.uint32)
    tab = oracle.e2m1_decode_table()
    for sign in (1.0, -1.0):
        vals = tab[oracle.e2m1_encode(np.full(k.size, sign * y, dtype=np.float32), r)].astype(np.float64)
        assert np.all((np.abs(vals) == float(lo)) | (np.abs(vals) == float(hi)))
        assert int(np.sum(np.abs(vals) == float(hi))) == expect
        mean = Fraction(int(round(abs(vals).sum() * 2)), 2 * 2**22)     # vals are multiples of 1/2
        if yq >= 1:
            assert mean == yq
        else:
            assert 0 <= yq - mean < (hi - lo) / 2**22


def test_sr_decision_uses_the_high_22_bits_monotonically():
    """The low 10 bits of r never change a code, the all-ones word never
    rounds up, and a smaller variate rounds up wherever a larger one does."""
    g = np.random.default_rng(3)
    y = (g.uniform(0.0, 6.0, 200_000) * g.choice([1.0, 1e-3], 200_000)).astype(np.float32)
    r = g.integers(0, 2**32, y.size, dtype=np.uint64).astype(np.uint32)
    base = oracle.e2m1_encode(y, r)
    low = g.integers(0, 1024, y.size, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(oracle.e2m1_encode(y, r ^ low), base)
    down = oracle.e2m1_encode(y, np.full(y.size, 0xFFFFFFFF, np.uint32))
    tab = oracle.e2m1_decode_table()
    assert np.all(np.abs(tab[down]) <= np.abs(y))                     # all-ones: the lower neighbour
    smaller = ((r >> np.uint32(10)) // np.uint32(3)) << np.uint32(10)
    up = base != down
    assert np.all(oracle.e2m1_encode(y, smaller)[up] == base[up])
    assert 0.2 < up.mean() < 0.8


def test_sr_words_uniform_and_seeded():
    n = 1 << 20
    idx = np.arange(n, dtype=np.uint64)
    w = oracle.sr_words(2024, idx)
    counts = np.bincount((w >> 24).astype(np.int64), minlength=256)
    chi2 = ((counts - n / 256) ** 2 / (n / 256)).sum()
    assert chi2 < 400          # 255 dof: mean 255, sd ~22.6
    w2 = oracle.sr_words(2025, idx)
    assert np.mean(w == w2) < 1e-3
    w3 = oracle.sr_words(2024, idx + np.uint64(2**32))      # high index bits matter
    assert np.mean(w == w3) < 1e-3


# ------------------------------------------------------------ GEMM --------
def test_gemm_ref_vs_exact_rationals():
    g = np.random.default_rng(1)
    for (m, n, k) in [(1, 1, 1), (3, 5, 7), (8, 8, 256), (2, 7, 130)]:
        a = g.standard_normal((m, k)) * 10.0 ** g.integers(-3, 3, (m, k))
        b = g.standard_normal((n, k))
        c, s = oracle.gemm_ref(a, b)
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(float(a[i, t])) * Fraction(float(b[j, t])) for t in range(k))
                sabs = sum(abs(Fraction(float(a[i, t])) * Fraction(float(b[j, t]))) for t in range(k))
                assert abs(Fraction(float(c[i, j])) - exact) <= Fraction(1, 10**15) * sabs
                assert abs(Fraction(float(s[i, j])) - sabs) <= Fraction(1, 10**15) * sabs


def test_gemm_ref_transpose_and_grouped():
    g = np.random.default_rng(2)
    a = g.standard_normal((20, 64))
    b = g.standard_normal((12, 64))
    c, s = oracle.gemm_ref(a, b)
    ct, st = oracle.gemm_ref(b, a)
    assert np.allclose(c.T, ct, rtol=1e-14, atol=0) and np.allclose(s.T, st, rtol=1e-14)
    cg, sg = oracle.grouped_gemm_ref(a, [b], [0, 20])
    assert np.array_equal(cg, c) and np.array_equal(sg, s)
    b2 = g.standard_normal((12, 64))
    cg2, _ = oracle.grouped_gemm_ref(a, [b, b2, b], [0, 7, 7, 20])  # empty middle group
    assert np.array_equal(cg2[:7], oracle.gemm_ref(a[:7], b)[0])
    assert np.array_equal(cg2[7:], oracle.gemm_ref(a[7:], b)[0])


def test_quantized_gemm_close_to_bf16_gemm():
    """End to end: dequantized 1x128 x 128x128 operands reproduce the BF16
    product to within the quantization error (a few percent of S)."""
    a = synth.activations(64, 512, seed=3)
    b = synth.weights(96, 512, seed=3)
    qa, sa = oracle.quant_e4m3(a, "tile")
    qb, sb = oracle.quant_e4m3(b, "block")
    ah = oracle.dequant_e4m3(qa, sa, "tile")
    bh = oracle.dequant_e4m3(qb, sb, "block")
    c, s = oracle.gemm_ref(ah, bh)
    c_true, s_true = oracle.gemm_ref(oracle.bf16_bits_to_f32(a), oracle.bf16_bits_to_f32(b))
    assert np.all(np.abs(c - c_true) <= 0.13 * s_true)
    assert np.sqrt(np.mean((c - c_true) ** 2)) < 0.05 * np.sqrt(np.mean(s_true ** 2))


def test_nvfp4_sampled_rows_match_whole_tensor():
    """Quantizing sampled rows under the whole tensor's scale, with the SR
    index base of each row, reproduces those rows of the whole-tensor
    quantization (row-wise and column-wise, RHT and SR on)."""
    from fine_grained_scaled_amd import synth
    bits = synth.gradients(64, 96, seed=31)
    for colwise in (False, True):
        q, s, ts = oracle.quant_nvfp4(bits, colwise=colwise, rht=True, rht_seed=5, stochastic=True, sr_seed=77)
        vals = oracle.nvfp4_operand_values(bits, colwise=colwise, rht=True, rht_seed=5)
        assert oracle.nvfp4_tensor_scale(vals) == ts
        for r in (0, 7, vals.shape[0] - 1):
            if colwise:      # quantized row r = source column r; elements run down the source rows
                base, cs = r, bits.shape[1]
            else:
                base, cs = r * bits.shape[1], 1
            qr, sr = oracle.quant_nvfp4_rows(vals[r:r + 1], ts, stochastic=True, sr_seed=77,
                                             idx_base=base, idx_cs=cs)
            assert np.array_equal(qr[0], q[r]) and np.array_equal(sr[0], s[r])
