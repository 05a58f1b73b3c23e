"""GPU parity of NVFP4 quantization (E2M1 codes two per byte, E4M3 scale per
16 elements, FP32 tensor scale; optional random 16x16 Hadamard transform
along the quantized dimension; RNE or stochastic rounding) against the CPU
oracle, bit for bit on packed codes, scale bytes and tensor scales.

"NVIDIA developed a method to train neural networks at 4-bit", section
"How it works": NVFP4, random Hadamard transforms of gradient inputs,
stochastic rounding.
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import sample_rows

pytestmark = pytest.mark.gpu

RHT_SEED = synth.derived_seed(0, synth.TAG_RHT)
SR_SEED = synth.derived_seed(0, synth.TAG_SR)


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def _bits_f32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _check(fgs, bits, rht_mask, stochastic, rowwise=True, colwise=True, rht_seed=RHT_SEED, sr_seed=SR_SEED,
           workspace=None):
    x = synth.to_torch_bf16(bits).to("cuda")
    r = fgs.quantize_nvfp4(x, rowwise=rowwise, colwise=colwise, rht_mask=rht_mask, rht_seed=rht_seed,
                           stochastic=stochastic, sr_seed=sr_seed, workspace=workspace)
    torch.cuda.synchronize()
    ts = r.tensor_scale.cpu().numpy()
    for side, on in ((0, rowwise), (1, colwise)):
        if not on:
            continue
        q, s, t = oracle.quant_nvfp4(bits, colwise=bool(side), rht=bool(rht_mask >> side & 1), rht_seed=rht_seed,
                                     stochastic=stochastic, sr_seed=sr_seed)
        gq = (r.q if side == 0 else r.qT).cpu().numpy()
        gs = (r.scales if side == 0 else r.scalesT).cpu().numpy()
        assert _bits_f32(ts[side]) == _bits_f32(t), f"tensor scale {side}: {ts[side]!r} vs {t!r}"
        assert np.array_equal(gs, s), f"side {side} scales differ at {np.argwhere(gs != s)[:5]}"
        assert np.array_equal(gq, q), f"side {side} codes differ at {np.argwhere(gq != q)[:5]}"


@pytest.mark.parametrize("rht_mask", [0, 1, 2, 3])
@pytest.mark.parametrize("stochastic", [False, True])
def test_nvfp4_parity_small(fgs, rht_mask, stochastic):
    bits = synth.gradients(256, 384, seed=41) if stochastic else synth.activations(256, 384, seed=42)
    _check(fgs, bits, rht_mask, stochastic)


@pytest.mark.parametrize("shape,row,col", [((384, 160), True, False), ((128, 200), False, True),
                                           ((1, 128), True, False), ((128, 128), True, True)])
def test_nvfp4_ragged_shapes(fgs, shape, row, col):
    bits = synth.weights(*shape, seed=43)
    _check(fgs, bits, 3 if (row and col) else (1 if row else 2), True, rowwise=row, colwise=col)


def test_nvfp4_rne_ties_and_saturation(fgs):
    """Tensor amax 2688 makes s_t = 1; a block with amax 6 gets s_b = 1 and
    d = 1, so its values land exactly on the E2M1 midpoints (ties to the even
    code) and on representable points; a block with a small E4M3 scale
    overshoots 6 and saturates."""
    rows, cols = 128, 256
    f = np.zeros((rows, cols), dtype=np.float32)
    f[0, 0] = 2688.0
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 0.1, 5.9])
    f[1, 16:32] = mids
    f[2, 32:48] = -mids
    f[3, 48:64] = np.resize([6.0, 6.1, -6.3, 0.0, -0.0, 5.99, 1e-3, -1e-3], 16)
    f[4, 64:80] = np.linspace(-1.2, 1.2, 16)
    f[5:, 128:] = synth.f32_to_bf16_bits(np.ones(1)).astype(np.float32)[0] * 0 + np.resize(
        np.linspace(-3, 3, 37), (rows - 5, 128))
    bits = synth.f32_to_bf16_bits(f)
    _check(fgs, bits, 0, False)
    _check(fgs, bits, 0, True)


def test_nvfp4_special_values(fgs):
    """Zero tensor (s_t = 1, all-zero codes), a NaN or Inf anywhere (s_t NaN,
    scale bytes 0x7F, codes 0), and a tensor of tiny values."""
    rows, cols = 128, 256
    _check(fgs, synth.f32_to_bf16_bits(np.zeros((rows, cols), np.float32)), 3, True)
    for bad in (np.nan, np.inf, -np.inf):
        f = oracle.bf16_bits_to_f32(synth.activations(rows, cols, seed=44)).copy()
        f[5, 17] = bad
        _check(fgs, synth.f32_to_bf16_bits(f), 3, True)
    tiny = np.ldexp(oracle.bf16_bits_to_f32(synth.activations(rows, cols, seed=45)), -120)
    _check(fgs, synth.f32_to_bf16_bits(tiny), 3, False)


def _mixed_class_tensor():
    """BF16 bits of a 256 x 256 tensor with amax near 2^-12 whose ordinary
    blocks sit beside blocks of the kernel's careful path: row blocks and
    16 x 16 squares (careful in both orientations) with amax just under
    2^-30 (nonzero scale byte, pre-scaled quotient), scales that round to
    zero, and zeros."""
    g = np.random.default_rng(77)
    f = (g.standard_normal((256, 256)) * 2.0 ** -14).astype(np.float32)
    for r, c, lg in [(3, 16, -31.5), (3, 48, -31.0), (40, 0, -33.0), (77, 112, None), (130, 32, -31.2),
                     (200, 240, -29.5), (255, 128, -45.0)]:
        f[r, c:c + 16] = 0.0 if lg is None else g.standard_normal(16) * 2.0 ** lg
    for r, c, lg in [(96, 64, -31.3), (16, 208, -40.0), (160, 160, None)]:
        f[r:r + 16, c:c + 16] = 0.0 if lg is None else g.standard_normal((16, 16)) * 2.0 ** lg
    return synth.f32_to_bf16_bits(f)


def test_nvfp4_mixed_block_classes_are_covered():
    """The fixture really holds blocks with amax below 2^-30 and a nonzero
    scale byte, blocks whose scale byte is 0 with a nonzero amax, and
    ordinary blocks, in the same 128 x 128 tiles (oracle, no transform)."""
    bits = _mixed_class_tensor()
    f = oracle.bf16_bits_to_f32(bits)
    _, s, _ = oracle.quant_nvfp4(bits, colwise=False, rht=False, rht_seed=RHT_SEED, stochastic=False,
                                 sr_seed=SR_SEED)
    amax = np.abs(f).reshape(256, 16, 16).max(axis=2)
    assert np.any((amax < 2.0 ** -30) & (amax > 0) & (s != 0))
    assert np.any((amax > 0) & (s == 0))
    assert np.sum(amax >= 2.0 ** -30) > 3000


@pytest.mark.parametrize("rht_mask", [0, 3])
@pytest.mark.parametrize("stochastic", [False, True])
def test_nvfp4_mixed_block_classes(fgs, rht_mask, stochastic):
    """Waves that hold one careful-path block take the careful path for all
    their blocks, the other waves the fast one: codes, scale bytes and
    tensor scales stay bit-exact in both orientations."""
    _check(fgs, _mixed_class_tensor(), rht_mask, stochastic)


def test_nvfp4_determinism(fgs):
    bits = synth.gradients(512, 512, seed=46)
    x = synth.to_torch_bf16(bits).to("cuda")
    a = fgs.quantize_nvfp4(x, colwise=True, rht_mask=2, rht_seed=RHT_SEED, stochastic=True, sr_seed=SR_SEED)
    b = fgs.quantize_nvfp4(x, colwise=True, rht_mask=2, rht_seed=RHT_SEED, stochastic=True, sr_seed=SR_SEED)
    torch.cuda.synchronize()
    assert torch.equal(a.q, b.q) and torch.equal(a.qT, b.qT) and torch.equal(a.tensor_scale, b.tensor_scale)


def test_nvfp4_sr_seed_changes_codes(fgs):
    bits = synth.gradients(256, 256, seed=47)
    x = synth.to_torch_bf16(bits).to("cuda")
    a = fgs.quantize_nvfp4(x, stochastic=True, sr_seed=1)
    b = fgs.quantize_nvfp4(x, stochastic=True, sr_seed=2)
    torch.cuda.synchronize()
    assert not torch.equal(a.q, b.q)
    assert torch.equal(a.scales, b.scales)


def test_nvfp4_wgrad_gradient_full_size_sampled(fgs):
    """12B-hybrid-like wgrad operand: dY 8192 x 20480 (Student-t gradients),
    column-wise along the 8192 tokens with the random Hadamard transform and
    stochastic rounding, row-wise plain RNE; sampled rows of each output
    against the oracle under the whole tensor's scale."""
    M, N = 8192, 20480
    bits = synth.gradients(M, N, seed=0)
    x = synth.to_torch_bf16(bits).to("cuda")
    r = fgs.quantize_nvfp4(x, rowwise=True, colwise=True, rht_mask=2, rht_seed=RHT_SEED,
                           stochastic=True, sr_seed=SR_SEED)
    torch.cuda.synchronize()
    ts = r.tensor_scale.cpu().numpy()
    # row-wise: no transform, stochastic rounding
    vals = oracle.nvfp4_operand_values(bits)
    t0 = oracle.nvfp4_tensor_scale(vals)
    assert _bits_f32(ts[0]) == _bits_f32(t0)
    for row in sample_rows(M)[::7]:
        q, s = oracle.quant_nvfp4_rows(vals[row:row + 1], t0, True, SR_SEED, idx_base=int(row) * N)
        assert np.array_equal(r.q[int(row)].cpu().numpy(), q[0])
        assert np.array_equal(r.scales[int(row)].cpu().numpy(), s[0])
    del vals
    # column-wise: transform along the tokens
    valsT = oracle.nvfp4_operand_values(bits, colwise=True, rht=True, rht_seed=RHT_SEED)
    t1 = oracle.nvfp4_tensor_scale(valsT)
    assert _bits_f32(ts[1]) == _bits_f32(t1)
    for c in sample_rows(N, seed=3)[::11]:
        q, s = oracle.quant_nvfp4_rows(valsT[c:c + 1], t1, True, SR_SEED, idx_base=int(c), idx_cs=N)
        assert np.array_equal(r.qT[int(c)].cpu().numpy(), q[0])
        assert np.array_equal(r.scalesT[int(c)].cpu().numpy(), s[0])


@pytest.mark.parametrize("ws_bytes", [8, 24, 4096])
def test_nvfp4_workspace_sizes(fgs, ws_bytes):
    """The tensor-amax pass keeps two partials per workgroup in the
    workspace; any size from one slot pair up gives the oracle's result (an
    8-byte workspace runs one amax workgroup over every tile).  The
    workspace starts as garbage: no pass may rely on it being cleared."""
    bits = synth.gradients(768, 1024, seed=44)
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
    _check(fgs, bits, 2, True, workspace=ws)
