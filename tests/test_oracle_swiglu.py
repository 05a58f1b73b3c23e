"""Pins of the oracle's SwiGLU activation and of its one-step FP64 -> BF16
rounding (the activation sits between the two expert GEMMs of a DeepSeek-V3
MoE layer; its BF16 output is what the second GEMM's quantizer reads).

Pins used: every BF16 number maps to itself, every midpoint between two
neighbours goes to the even one and one FP64 ulp either side of it to the
nearer one (a brute-force walk over the whole BF16 grid), the overflow
threshold; SwiGLU against scipy's logistic function and the identity
silu(g) - silu(-g) = g.
"""
import numpy as np
from scipy.special import expit

import oracle
from fine_grained_scaled_amd import synth


def _bf16_values():
    bits = np.arange(0, 0x7F80, dtype=np.uint32)          # +0 .. largest finite
    return bits, (bits << 16).view(np.float32).astype(np.float64)


def test_f64_to_bf16_grid_midpoints_and_overflow():
    bits, vals = _bf16_values()
    assert np.array_equal(oracle.f64_to_bf16(vals), bits.astype(np.uint16))
    assert np.array_equal(oracle.f64_to_bf16(-vals), (bits | 0x8000).astype(np.uint16))
    mid = (vals[:-1] + vals[1:]) / 2                       # exact in FP64
    even = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:]).astype(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16(mid), even)
    assert np.array_equal(oracle.f64_to_bf16(np.nextafter(mid, 0)), bits[:-1].astype(np.uint16))
    assert np.array_equal(oracle.f64_to_bf16(np.nextafter(mid, np.inf)), bits[1:].astype(np.uint16))
    top = vals[-1]
    half_ulp = 2.0 ** 119
    assert oracle.f64_to_bf16([top + half_ulp])[0] == 0x7F80              # ties away from the odd max
    assert oracle.f64_to_bf16([np.nextafter(top + half_ulp, 0)])[0] == 0x7F7F
    assert oracle.f64_to_bf16([np.inf])[0] == 0x7F80 and oracle.f64_to_bf16([-np.inf])[0] == 0xFF80
    assert (int(oracle.f64_to_bf16([np.nan])[0]) & 0x7FFF) > 0x7F80


def test_swiglu_against_logistic_and_identity():
    inter = 256
    gu = synth.activations(64, 2 * inter, seed=3)
    h = oracle.swiglu_f64(gu, inter)
    v = oracle.bf16_bits_to_f32(gu).astype(np.float64)
    g, u = v[:, :inter], v[:, inter:]
    ref = g * expit(g) * u
    assert np.allclose(h, ref, rtol=1e-14, atol=1e-300)
    neg = np.concatenate([synth.f32_to_bf16_bits(-oracle.bf16_bits_to_f32(gu[:, :inter])),
                          gu[:, inter:]], axis=1)
    sg = oracle.swiglu_f64(np.concatenate([gu[:, :inter], np.full_like(gu[:, inter:], 0x3F80)], axis=1), inter)
    sn = oracle.swiglu_f64(np.concatenate([neg[:, :inter], np.full_like(gu[:, inter:], 0x3F80)], axis=1), inter)
    assert np.allclose(sg - sn, g, rtol=1e-13, atol=1e-13)                # silu(g) - silu(-g) = g
    z = np.zeros((2, 2 * inter), np.uint16)
    assert not oracle.swiglu_f64(z, inter).any()
    hb = oracle.swiglu_bf16(gu, inter)
    assert np.array_equal(hb, oracle.f64_to_bf16(h))
