"""GPU parity of MXFP8 quantization (E4M3 codes, one E8M0 scale per 32
elements; row-wise and column-wise/transposed outputs) against the CPU
oracle, bit for bit on codes and scale bytes.

"Accelerating FP8 training performance with the NVIDIA NeMo framework":
MXFP8 scales blocks of 32 values.
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def _check(fgs, bits, rowwise=True, colwise=True):
    x = synth.to_torch_bf16(bits).to("cuda")
    r = fgs.quantize_mx(x, rowwise=rowwise, colwise=colwise)
    torch.cuda.synchronize()
    if rowwise:
        q, s = oracle.quant_mx(bits)
        gq, gs = r.q.cpu().numpy(), r.scales.cpu().numpy()
        assert np.array_equal(gs, s), f"row scales differ at {np.argwhere(gs != s)[:5]}"
        assert np.array_equal(gq, q), f"row codes differ at {np.argwhere(gq != q)[:5]}"
    if colwise:
        q, s = oracle.quant_mx(bits, colwise=True)
        gq, gs = r.qT.cpu().numpy(), r.scalesT.cpu().numpy()
        assert np.array_equal(gs, s), f"col scales differ at {np.argwhere(gs != s)[:5]}"
        assert np.array_equal(gq, q), f"col codes differ at {np.argwhere(gq != q)[:5]}"


@pytest.mark.parametrize("shape,row,col", [((256, 512), True, True), ((384, 160), True, True),
                                           ((128, 96), True, True), ((300, 64), True, False),
                                           ((128, 40 * 8), False, True), ((1, 32), True, False)])
def test_mx_parity_small(fgs, shape, row, col):
    bits = synth.activations(*shape, seed=11)
    _check(fgs, bits, row, col)


def test_mx_special_values(fgs):
    """Zero, NaN and Inf blocks; amax on both sides of the 1.75 * 2^E
    boundary (BF16 mantissa field 0x60 / 0x61); subnormal, tiny (e clamped to
    -127) and huge (e = 120) blocks; exact E4M3 ties after scaling."""
    rows, cols = 128, 512
    f = oracle.bf16_bits_to_f32(synth.activations(rows, cols, seed=12, outliers=False)).copy()
    f[0, 0:32] = 0.0
    f[0, 0:32:5] = -0.0
    f[1, 32] = np.nan
    f[2, 64] = np.inf
    f[3, 96] = -np.inf
    f[4, 0:32] = 1.75 * np.linspace(-1, 1, 32)                      # amax = 1.75 (field 0x60)
    f[5, 0:32] = 1.7578125 * np.linspace(-1, 1, 32)                 # field 0x61
    f[6, 32:64] = np.ldexp(np.arange(32) % 5 - 2, -133)             # BF16 subnormals
    f[7, 64:96] = np.ldexp(np.linspace(-1, 1, 32), -120)            # e clamps to -127
    f[8, 96:128] = np.ldexp(np.linspace(-1.9, 1.9, 32), 127)        # e = 120
    f[9, 128:160] = np.resize([448.0, 1.0625, 1.1875, 2 ** -10, 3 * 2 ** -10, -240.0, 232.0, 0.5], 32)
    f[10, 160:192] = np.resize([3.0e38, -1.0e-30, 1.0, 65504.0], 32)
    f[40:48, 200:205] = 5.0e4                                        # column outliers
    bits = synth.f32_to_bf16_bits(f)
    _check(fgs, bits)


def test_mx_llama405b_full_size_sampled(fgs):
    """Llama-3.1-405B shapes, one GPU's share: X 4096 x 16384 row-wise and
    column-wise, checked on sampled rows / columns."""
    M, K = 4096, 16384
    bits = synth.activations(M, K, seed=0, outliers=False)
    x = synth.to_torch_bf16(bits).to("cuda")
    r = fgs.quantize_mx(x, rowwise=True, colwise=True)
    torch.cuda.synchronize()
    rs = sample_rows(M)
    q, s = oracle.quant_mx(bits[rs])
    idx = torch.from_numpy(rs).cuda()
    assert np.array_equal(r.q[idx].cpu().numpy(), q)
    assert np.array_equal(r.scales[idx].cpu().numpy(), s)
    cs = sample_rows(K, seed=2)
    qt, st = oracle.quant_mx(np.ascontiguousarray(bits[:, cs]), colwise=True)
    cidx = torch.from_numpy(cs).cuda()
    assert np.array_equal(r.qT[cidx].cpu().numpy(), qt)
    assert np.array_equal(r.scalesT[cidx].cpu().numpy(), st)


def test_mx_determinism(fgs):
    bits = synth.weights(512, 1024, seed=13)
    x = synth.to_torch_bf16(bits).to("cuda")
    a = fgs.quantize_mx(x, colwise=True)
    b = fgs.quantize_mx(x, colwise=True)
    torch.cuda.synchronize()
    assert torch.equal(a.q, b.q) and torch.equal(a.qT, b.qT)
    assert torch.equal(a.scales, b.scales) and torch.equal(a.scalesT, b.scalesT)
