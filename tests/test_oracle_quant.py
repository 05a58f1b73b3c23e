"""Pins of the oracle's quantizers.

1x128 activation tiles and 128x128 weight blocks, each scaled on its own
from its current amax: "Can you explain the role of FP8 precision in
DeepSeek-V3 training", sections "Fine-grained quantization" and "Online
quantization".  Per-tensor scaling and MXFP8 blocks of 32: "Accelerating FP8
training performance with the NVIDIA NeMo framework".  NVFP4 with a 16-element
E4M3 scale and an FP32 tensor scale: "NVIDIA developed a method to train
neural networks at 4-bit", section "How it works".

Pins used: the closed-form scale, brute-force argmin codes, torch's float8
cast as an independent rounding routine, invariants that hold for any
correct quantizer (the block maximum lands on +-448 / +-6, power-of-two
scale invariance, block locality, transpose invariance), special blocks,
and a worked NVFP4 example computed by hand.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

F32 = np.float32


def _bf16(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _f32(bits):
    return oracle.bf16_bits_to_f32(bits)


def _torch_e4m3(y):
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _blocks(rows, cols, br, bc):
    for r0 in range(0, rows, br):
        for c0 in range(0, cols, bc):
            yield slice(r0, min(r0 + br, rows)), slice(c0, min(c0 + bc, cols))


@pytest.mark.parametrize("mode,shape", [("tile", (37, 384)), ("tile", (5, 200)),
                                        ("block", (300, 260)), ("tensor", (64, 300))])
def test_fp32_scaled_closed_form_and_codes(mode, shape):
    """scale == fl32(amax / 448) bit for bit; codes == torch's RNE cast of
    fl32(x / scale) (never above 448 here, so torch's overflow rule is moot)."""
    rows, cols = shape
    x = synth.activations(rows, cols, seed=11)
    q, s = oracle.quant_e4m3(x, mode)
    xf = _f32(x)
    br, bc = {"tile": (1, 128), "block": (128, 128), "tensor": (rows, cols)}[mode]
    for bi, (rs, cs) in enumerate(_blocks(rows, cols, br, bc)):
        amax = F32(np.max(np.abs(xf[rs, cs])))
        want_s = amax / F32(448.0)
        got_s = s.reshape(-1)[bi]
        assert np.float32(got_s).tobytes() == np.float32(want_s).tobytes()
        y = xf[rs, cs] / want_s
        assert np.abs(y).max() < 449.0
        assert np.array_equal(q[rs, cs], _torch_e4m3(y))


def test_tile_codes_bruteforce_small():
    from test_oracle_codecs import _brute_e4m3
    x = synth.activations(3, 256, seed=2)
    q, s = oracle.quant_e4m3(x, "tile")
    xf = _f32(x)
    for r in range(3):
        for t in range(2):
            y = xf[r, t * 128:(t + 1) * 128] / s[r, t]
            assert np.array_equal(q[r, t * 128:(t + 1) * 128], _brute_e4m3(y))


@pytest.mark.parametrize("mode", ["tile", "block", "tensor"])
def test_block_max_maps_to_448(mode):
    """Invariant: every finite non-zero block whose scale is normal holds
    +-448 (code 0x7E / 0xFE): the block's amax divided by amax/448 rounds to 448."""
    x = synth.activations(256, 512, seed=3)
    q, s = oracle.quant_e4m3(x, mode)
    rows, cols = x.shape
    br, bc = {"tile": (1, 128), "block": (128, 128), "tensor": (rows, cols)}[mode]
    for rs, cs in _blocks(rows, cols, br, bc):
        codes = q[rs, cs] & 0x7F
        assert codes.max() == 0x7E


@pytest.mark.parametrize("mode", ["tile", "block", "tensor"])
def test_power_of_two_scale_invariance(mode):
    x = synth.activations(130, 384, seed=4, outliers=False)
    q0, s0 = oracle.quant_e4m3(x, mode)
    for k in (-20, -3, 5, 30):
        xk = _bf16(_f32(x) * F32(2.0 ** k))        # exact: powers of two
        qk, sk = oracle.quant_e4m3(xk, mode)
        assert np.array_equal(qk, q0)
        assert np.array_equal(sk, (s0 * F32(2.0 ** k)).astype(np.float32))


@pytest.mark.parametrize("mode", ["tile", "block"])
def test_block_locality(mode):
    """Perturbing one block (an outlier) leaves every other block bit-identical."""
    x = synth.activations(256, 512, seed=5)
    q0, s0 = oracle.quant_e4m3(x, mode)
    y = x.copy()
    y[130, 300] = _bf16([1.0e4])[0]
    q1, s1 = oracle.quant_e4m3(y, mode)
    br, bc = (1, 128) if mode == "tile" else (128, 128)
    hit = (130 // br, 300 // bc)
    for bi, (rs, cs) in enumerate(_blocks(256, 512, br, bc)):
        idx = (rs.start // br, cs.start // bc)
        same = np.array_equal(q0[rs, cs], q1[rs, cs]) and s0[idx] == s1[idx]
        assert same == (idx != hit)


@pytest.mark.parametrize("mode", ["block", "tensor"])
def test_transpose_invariance(mode):
    x = synth.activations(256, 384, seed=6)
    q, s = oracle.quant_e4m3(x, mode)
    qt, st = oracle.quant_e4m3(x, mode, colwise=True)
    assert np.array_equal(qt, q.T)
    assert np.array_equal(st, s.T)


def test_colwise_tile_is_rowwise_of_transpose():
    x = synth.activations(256, 200, seed=7)
    qt, st = oracle.quant_e4m3(x, "tile", colwise=True)
    q2, s2 = oracle.quant_e4m3(np.ascontiguousarray(x.T), "tile")
    assert np.array_equal(qt, q2) and np.array_equal(st, s2)
    assert qt.shape == (200, 256) and st.shape == (200, 2)


def test_special_blocks():
    x = synth.activations(4, 512, seed=8)
    x[0, 0:128] = _bf16(np.zeros(128))                 # zero tile
    x[0, 0:128:2] = _bf16(-np.zeros(64))               # with negative zeros
    x[1, 128] = _bf16([np.nan])[0]                     # NaN tile
    x[2, 300] = _bf16([np.inf])[0]                     # Inf tile
    x[3, 400] = _bf16([-np.inf])[0]
    q, s = oracle.quant_e4m3(x, "tile")
    assert s[0, 0] == 1.0
    assert np.array_equal(q[0, 0:128:2], np.full(64, 0x80, np.uint8))
    assert np.array_equal(q[0, 1:128:2], np.zeros(64, np.uint8))
    for r, t in ((1, 1), (2, 2), (3, 3)):
        assert math.isnan(s[r, t])
        assert np.all(q[r, t * 128:(t + 1) * 128] == 0x7F)
    # the other tiles of those rows are untouched
    q_clean, s_clean = oracle.quant_e4m3(synth.activations(4, 512, seed=8), "tile")
    assert np.array_equal(q[1, :128], q_clean[1, :128]) and s[1, 0] == s_clean[1, 0]


def test_ragged_edge_tiles():
    """A partial edge tile uses the elements present."""
    x = synth.activations(3, 200, seed=9)
    q, s = oracle.quant_e4m3(x, "tile")
    assert s.shape == (3, 2)
    xf = _f32(x)
    amax = np.abs(xf[:, 128:]).max(axis=1).astype(np.float32)
    assert np.array_equal(s[:, 1], amax / F32(448.0))


def test_dequant_error_bound():
    """|x - dec(q) * s| <= 2^-4 |x| + 2^-10 s (half an E4M3 step, normal and
    subnormal range), plus one FP32 rounding of x / s."""
    x = synth.activations(64, 1024, seed=10)
    for mode in ("tile", "block", "tensor"):
        q, s = oracle.quant_e4m3(x, mode)
        xh = oracle.dequant_e4m3(q, s, mode)
        xf = _f32(x).astype(np.float64)
        rows, cols = x.shape
        sfull = xh.copy()
        br, bc = {"tile": (1, 128), "block": (128, 128), "tensor": (rows, cols)}[mode]
        for bi, (rs, cs) in enumerate(_blocks(rows, cols, br, bc)):
            sfull[rs, cs] = s.reshape(-1)[bi]
        err = np.abs(xh - xf)
        assert np.all(err <= 2.0 ** -4 * np.abs(xf) * (1 + 2.0 ** -20) + 2.0 ** -10 * sfull)


# ---------------------------------------------------------------- MXFP8 ----
def test_mx_golden_scales():
    import os
    pts = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "mx_scales.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            a, b = line.split()[:2]
            pts.append((float(a), int(b)))
    for amax, want in pts:
        blk = np.zeros((1, 32), dtype=np.float32)
        blk[0, 7] = -amax
        blk[0, 8] = amax / 4
        bits = _bf16(blk)
        assert _f32(bits)[0, 7] == -amax, amax     # fixture values are BF16-exact
        q, s = oracle.quant_mx(bits)
        assert s[0, 0] == want, (amax, s[0, 0], want)


def test_mx_codes_and_range():
    """Codes equal torch's RNE cast of x * 2^-e (exact power-of-two scaling);
    the block maximum decodes into [224, 448] (amax * 2^-e is in (224, 448])."""
    x = synth.activations(64, 512, seed=12)
    q, s = oracle.quant_mx(x)
    xf = _f32(x)
    tab = oracle.e4m3_decode_table()
    for r in range(64):
        for b in range(16):
            e = int(s[r, b]) - 127
            y = np.ldexp(xf[r, b * 32:(b + 1) * 32], -e).astype(np.float32)
            assert np.array_equal(q[r, b * 32:(b + 1) * 32], _torch_e4m3(y))
            m = np.abs(tab[q[r, b * 32:(b + 1) * 32]]).max()
            assert 224.0 <= m <= 448.0
            amax = np.abs(xf[r, b * 32:(b + 1) * 32]).max()
            assert amax <= 448.0 * 2.0 ** e and amax > 448.0 * 2.0 ** (e - 1)


def test_mx_special_and_scale_invariance():
    x = synth.activations(2, 128, seed=13, outliers=False)
    x[0, 0:32] = _bf16(np.zeros(32))
    x[1, 32] = _bf16([np.nan])[0]
    q, s = oracle.quant_mx(x)
    assert s[0, 0] == 127 and np.all(q[0, :32] == 0)
    assert s[1, 1] == 0xFF and np.all(q[1, 32:64] == 0x7F)
    q0, s0 = oracle.quant_mx(synth.activations(8, 256, seed=14))
    q1, s1 = oracle.quant_mx(_bf16(_f32(synth.activations(8, 256, seed=14)) * F32(2.0 ** 9)))
    assert np.array_equal(q0, q1) and np.array_equal(s1.astype(int), s0.astype(int) + 9)


def test_mx_colwise_is_rowwise_of_transpose():
    x = synth.activations(96, 64, seed=15)
    qt, st = oracle.quant_mx(x, colwise=True)
    q2, s2 = oracle.quant_mx(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q2) and np.array_equal(st, s2) and st.shape == (64, 3)


# ---------------------------------------------------------------- NVFP4 ----
def test_nvfp4_worked_example():
    """Hand-computed: tensor amax 2688 -> s_t = 1.
    block 0: amax 2688 -> s_b = E4M3(448) = 0x7E, d = 448:
             2688/448 = 6 -> 0x7; 1000/448 = 2.23 -> 2 (0x4); -500/448 = -1.12 -> -1 (0xA)
    block 1: amax 7 -> 7/6 = 1.1667 -> E4M3 1.125 (0x39), d = 1.125:
             7/1.125 = 6.22 saturates -> 0x7; 3.5/1.125 = 3.11 -> 3 (0x5);
             -1.75/1.125 = -1.556 -> -1.5 (0xB); 0.25/1.125 = 0.22 -> 0 (0x0)
    block 2: all zero -> s_b = 0, codes 0."""
    v = np.zeros((1, 48), dtype=np.float32)
    v[0, 0], v[0, 1], v[0, 2] = 2688, 1000, -500
    v[0, 16], v[0, 17], v[0, 18], v[0, 19] = 7, 3.5, -1.75, 0.25
    q, s, st = oracle.quant_nvfp4(_bf16(v))
    assert st == 1.0
    assert list(s[0]) == [0x7E, 0x39, 0x00]
    codes = oracle.unpack_e2m1(q, 48)[0]
    assert list(codes[0:4]) == [0x7, 0x4, 0xA, 0x0]
    assert list(codes[16:21]) == [0x7, 0x5, 0xB, 0x0, 0x0]
    assert np.all(codes[32:] == 0)
    assert q[0, 0] == (0x4 << 4) | 0x7                # element 2j low nibble


def test_nvfp4_block_max_maps_to_6_under_rne():
    """Invariant: with a normal E4M3 block scale, RNE sends the block maximum
    to +-6 (|y_max| lies within [6/(1+2^-4), 6/(1-2^-4)])."""
    x = synth.activations(32, 512, seed=16)
    q, s, st = oracle.quant_nvfp4(x)
    codes = oracle.unpack_e2m1(q, 512)
    for r in range(32):
        for b in range(32):
            if (s[r, b] & 0x7F) >= 0x08:
                assert (codes[r, b * 16:(b + 1) * 16] & 0x7).max() == 0x7


def test_nvfp4_scale_invariance_and_zero():
    x = synth.activations(16, 256, seed=17)
    q0, s0, t0 = oracle.quant_nvfp4(x)
    q1, s1, t1 = oracle.quant_nvfp4(_bf16(_f32(x) * F32(2.0 ** -7)))
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1) and t1 == t0 * F32(2.0 ** -7)
    qz, sz, tz = oracle.quant_nvfp4(_bf16(np.zeros((2, 32))))
    assert tz == 1.0 and np.all(qz == 0) and np.all(sz == 0)
    xn = x.copy()
    xn[3, 5] = _bf16([np.inf])[0]
    qn, sn, tn = oracle.quant_nvfp4(xn)
    assert math.isnan(tn) and np.all(qn == 0) and np.all(sn == 0x7F)


def test_nvfp4_dequant_bound():
    """Relative error of an RNE NVFP4 element is at most half an E2M1 step
    (1/4 of the value's binade, i.e. <= 25% of |x| above 0.5 d) plus the
    zero-flush region below 0.25 d."""
    x = synth.activations(16, 256, seed=18, outliers=False)
    q, s, st = oracle.quant_nvfp4(x)
    xh = oracle.dequant_nvfp4(q, s, st, 256)
    xf = _f32(x).astype(np.float64)
    d = np.repeat(oracle.e4m3_decode_table()[s], 16, axis=1) * float(st)
    err = np.abs(xh - xf)
    assert np.all(err <= np.maximum(0.25 * np.abs(xf), 0.25 * d) * (1 + 1e-6) + 0.5 * d * (np.abs(xf) > 6 * d))


def test_nvfp4_colwise_rne_is_rowwise_of_transpose_and_rht_cancels():
    x = synth.activations(64, 48, seed=19)
    qt, st_, tt = oracle.quant_nvfp4(x, colwise=True)
    q2, s2, t2 = oracle.quant_nvfp4(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q2) and np.array_equal(st_, s2) and tt == t2
    # the same sign vector on both operands: T^T T = I, so the product of
    # transformed operands equals the product of the originals (FP64)
    a = _f32(synth.activations(64, 32, seed=20)).T.astype(np.float64)   # [32 x 64]
    b = _f32(synth.activations(64, 16, seed=21)).T.astype(np.float64)   # [16 x 64]
    ra = oracle.rht_rows(a.astype(np.float32), 99).astype(np.float64)
    rb = oracle.rht_rows(b.astype(np.float32), 99).astype(np.float64)
    ref = a @ b.T
    assert np.allclose(ra @ rb.T, ref, rtol=0, atol=1e-5 * (np.abs(a) @ np.abs(b).T).max())


def test_nvfp4_sr_index_is_source_position():
    """SR words are keyed by the element's linear index in the source tensor
    (row * cols + col), whatever the orientation."""
    rows, cols = 32, 48
    v = np.full((rows, cols), 0.75, dtype=np.float32)   # every y = 0.75*... same p
    v[0, 0] = 2688.0 * 0.75 / 6.0 * 6                   # fixes s_t
    x = _bf16(v)
    seed = 0x1234_5678_9ABC_DEF0
    q, s, st = oracle.quant_nvfp4(x, colwise=True, stochastic=True, sr_seed=seed)
    codes = oracle.unpack_e2m1(q, rows)                  # [cols x rows]
    qr, sr, str_ = oracle.quant_nvfp4(x, stochastic=True, sr_seed=seed)
    codes_r = oracle.unpack_e2m1(qr, cols)               # [rows x cols]
    # positions whose block scale and tensor scale coincide in both
    # orientations see the same y, hence the same word gives the same code
    assert st == str_
    same_scale = 0
    for c in range(1, cols):
        for r in range(16, rows):
            if s[c, r // 16] == sr[r, c // 16]:
                same_scale += 1
                assert codes[c, r] == codes_r[r, c]
    assert same_scale > 100
