"""Pins of the oracle's MoE weight-gradient pieces: the per-expert transposed
1x128 quantization and the per-expert wgrad product.

"Can you explain the role of FP8 precision in DeepSeek-V3 training",
sections "Fine-grained quantization" (1x128 tiles along the contraction,
each scaled from its own amax), "Online quantization" and "Mixed precision
framework" (the expert GEMMs run in FP8).  For the weight gradient of expert
g the contraction runs over the tokens routed to it, so its tiles hold
tokens of that expert only.

Pins used: the closed-form scale computed here from the tokens present,
torch's float8 cast and a brute-force argmin as independent rounding
routines, locality across an expert boundary, power-of-two invariance, the
reduction to the dense column-wise quantization when every boundary is a
multiple of 128, and exact integer arithmetic for the products.
"""
import numpy as np
import torch

import oracle
from fine_grained_scaled_amd import synth

F32 = np.float32


def _torch_e4m3(y):
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


OFFS = [0, 0, 130, 131, 300, 300, 428]     # empty, 130 (ragged), 1, 169, empty, 128


def test_grouped_colwise_closed_form():
    """Every tile's scale is fl32(amax / 448) over the tokens of its group
    present in it; codes are torch's RNE cast of fl32(x / scale); one column
    against the brute-force argmin as well."""
    from test_oracle_codecs import _brute_e4m3
    x = synth.gradients(428, 256, seed=21)
    xf = oracle.bf16_bits_to_f32(x)
    res = oracle.quant_e4m3_grouped_colwise(x, OFFS)
    assert len(res) == len(OFFS) - 1
    for g, (q, s) in enumerate(res):
        r0, r1 = OFFS[g], OFFS[g + 1]
        m = r1 - r0
        assert q.shape == (256, m) and s.shape == (256, (m + 127) // 128)
        for t in range(0, m, 128):
            seg = xf[r0 + t:min(r0 + t + 128, r1)].T          # [C x tokens of the tile]
            want_s = (np.abs(seg).max(axis=1).astype(F32) / F32(448.0)).astype(F32)
            assert np.array_equal(s[:, t // 128].view(np.uint32), want_s.view(np.uint32))
            y = seg / want_s[:, None]
            assert np.array_equal(q[:, t:t + seg.shape[1]], _torch_e4m3(y))
            assert np.array_equal(q[7, t:t + seg.shape[1]], _brute_e4m3(y[7]))


def test_grouped_colwise_tiles_stay_in_group():
    """An outlier in the last token of one expert changes that expert's last
    tile only; the next expert's first tile (which a dense 128-row tiling
    would share with it) is untouched."""
    x = synth.gradients(428, 128, seed=22)
    base = oracle.quant_e4m3_grouped_colwise(x, OFFS)
    y = x.copy()
    y[129, 5] = synth.f32_to_bf16_bits(np.array([3.0e3], F32))[0]   # last token of group 1
    hit = oracle.quant_e4m3_grouped_colwise(y, OFFS)
    for g in range(len(OFFS) - 1):
        (q0, s0), (q1, s1) = base[g], hit[g]
        if g != 1:
            assert np.array_equal(q0, q1) and np.array_equal(s0, s1)
            continue
        assert np.array_equal(q0[:, :128], q1[:, :128]) and np.array_equal(s0[:, 0], s1[:, 0])
        assert s1[5, 1] != s0[5, 1]
        assert np.array_equal(np.delete(s0[:, 1], 5), np.delete(s1[:, 1], 5))


def test_grouped_colwise_power_of_two_invariance():
    """Scaling one expert's tokens by 2^5 scales its scales by 2^5 exactly
    and changes no code anywhere."""
    x = synth.gradients(428, 128, seed=23)
    base = oracle.quant_e4m3_grouped_colwise(x, OFFS)
    xf = oracle.bf16_bits_to_f32(x).copy()
    xf[131:300] *= F32(32.0)
    res = oracle.quant_e4m3_grouped_colwise(synth.f32_to_bf16_bits(xf), OFFS)
    for g in range(len(OFFS) - 1):
        assert np.array_equal(base[g][0], res[g][0])
        want = base[g][1] * F32(32.0) if g == 3 else base[g][1]
        assert np.array_equal(res[g][1], want.astype(F32))


def test_grouped_colwise_aligned_groups_are_dense_colwise():
    """With every boundary a multiple of 128 the expert tiles coincide with
    the dense column-wise tiles, so the groups concatenate to it."""
    offs = [0, 256, 256, 384, 768]
    x = synth.gradients(768, 256, seed=24)
    res = oracle.quant_e4m3_grouped_colwise(x, offs)
    qd, sd = oracle.quant_e4m3(x, "tile", colwise=True)
    assert np.array_equal(np.concatenate([q for q, _ in res], axis=1), qd)
    assert np.array_equal(np.concatenate([s for _, s in res], axis=1), sd)


def test_grouped_wgrad_ref_exact_integers():
    """Integer-valued operands make every FP64 sum exact: C_g equals the
    token loop, an empty group is exactly zero, and the groups add up to the
    product over all tokens."""
    g = np.random.default_rng(5)
    counts = [3, 0, 5, 1]
    a_groups = [g.integers(-8, 9, (4, c)).astype(np.float64) for c in counts]
    b_groups = [g.integers(-8, 9, (3, c)).astype(np.float64) for c in counts]
    c, s = oracle.grouped_wgrad_ref(a_groups, b_groups)
    assert c.shape == (4, 4, 3)
    for k, cnt in enumerate(counts):
        for i in range(4):
            for j in range(3):
                want = sum(a_groups[k][i, t] * b_groups[k][j, t] for t in range(cnt))
                want_s = sum(abs(a_groups[k][i, t] * b_groups[k][j, t]) for t in range(cnt))
                assert c[k, i, j] == want and s[k, i, j] == want_s
    assert not c[1].any() and not s[1].any()
    dense, _ = oracle.gemm_ref(np.concatenate(a_groups, axis=1), np.concatenate(b_groups, axis=1))
    assert np.array_equal(c.sum(axis=0), dense)


def test_gather_rowwise_equivariance_and_invalid_rows():
    """1x128 row tiles are per row, so quantizing gathered rows equals
    gathering the quantized rows; an index outside x gives a zero row
    (scale 1, zero codes), and the grouped column-wise codes of a gather
    equal those of the explicitly permuted matrix."""
    x = synth.activations(50, 256, seed=25)
    g = np.random.default_rng(6)
    idx = g.integers(0, 50, 90)
    idx[[3, 40]] = [-1, 50]
    gx = oracle.gather_rows(x, idx)
    qg, sg = oracle.quant_e4m3(gx, "tile")
    qx, sx = oracle.quant_e4m3(x, "tile")
    ok = (idx >= 0) & (idx < 50)
    assert np.array_equal(qg[ok], qx[idx[ok]]) and np.array_equal(sg[ok], sx[idx[ok]])
    assert not qg[~ok].any() and np.all(sg[~ok] == 1.0)
    offs = [0, 30, 30, 90]
    res = oracle.quant_e4m3_grouped_colwise(x, offs, row_index=idx)
    perm = np.where(ok[:, None], x[np.clip(idx, 0, 49)], 0).astype(np.uint16)
    ref = oracle.quant_e4m3_grouped_colwise(perm, offs)
    for (q0, s0), (q1, s1) in zip(res, ref):
        assert np.array_equal(q0, q1) and np.array_equal(s0, s1)
