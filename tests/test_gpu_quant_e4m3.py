"""GPU parity of online FP32-scaled E4M3 quantization (1x128 tiles, 128x128
blocks, per-tensor; row-wise and column-wise/transposed outputs) against the
CPU oracle, bit for bit on codes and scales.

"Can you explain the role of FP8 precision in DeepSeek-V3 training",
sections "Fine-grained quantization" and "Online quantization";
"Accelerating FP8 training performance with the NVIDIA NeMo framework"
(per-tensor scaling).
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

pytestmark = pytest.mark.gpu

from _helpers import sample_rows  # noqa: E402


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def _dev(bits):
    return synth.to_torch_bf16(bits).to("cuda")


def _bf16(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _check(fgs, bits, mode, rowwise, colwise):
    x = _dev(bits)
    r = fgs.quantize_blockwise(x, mode, rowwise=rowwise, colwise=colwise)
    torch.cuda.synchronize()
    if rowwise:
        q, s = oracle.quant_e4m3(bits, mode)
        gq, gs = r.q.cpu().numpy(), r.scales.cpu().numpy()
        if mode == "tile":
            gs = gs.T
        assert np.array_equal(gq, q), f"row codes differ at {np.argwhere(gq != q)[:5]}"
        assert np.array_equal(gs.reshape(s.shape).view(np.uint32), s.view(np.uint32)), "row scales differ"
    if colwise:
        q, s = oracle.quant_e4m3(bits, mode, colwise=True)
        gq, gs = r.qT.cpu().numpy(), r.scalesT.cpu().numpy()
        if mode == "tile":
            gs = gs.T
        assert np.array_equal(gq, q), f"col codes differ at {np.argwhere(gq != q)[:5]}"
        assert np.array_equal(gs.reshape(s.shape).view(np.uint32), s.view(np.uint32)), "col scales differ"


@pytest.mark.parametrize("mode", ["tile", "block", "tensor"])
@pytest.mark.parametrize("shape,row,col", [((384, 512), True, True), ((300, 384), True, False),
                                           ((256, 200), False, True), ((128, 128), True, True),
                                           ((1, 128), True, False)])
def test_quant_parity_small(fgs, mode, shape, row, col):
    bits = synth.activations(*shape, seed=3)
    _check(fgs, bits, mode, row, col)


@pytest.mark.parametrize("mode", ["tile", "block", "tensor"])
def test_quant_special_values(fgs, mode):
    """Zero, NaN, +-Inf, all-subnormal and tiny (< 2^-64) blocks, exact E4M3
    ties (amax 448 -> scale 1 -> quotients on midpoints), huge outliers."""
    rows, cols = 256, 512
    v = synth.activations(rows, cols, seed=4).copy()
    f = oracle.bf16_bits_to_f32(v).copy()
    f[0, 0:128] = 0.0
    f[0, 0:128:3] = -0.0
    f[1, 128] = np.nan
    f[2, 300] = np.inf
    f[3, 400] = -np.inf
    f[4, 0:128] = np.ldexp(np.arange(128) % 7 - 3, -133)           # BF16 subnormals
    f[5, 128:256] = np.ldexp(np.linspace(-1, 1, 128), -70)          # amax < 2^-64
    f[6, 256:384] = np.ldexp(np.linspace(-1, 1, 128), -63)          # amax just above
    mids = np.array([1.0625, 1.1875, 2 ** -10, 3 * 2 ** -10, 5 * 2 ** -10, 0.96875, 248.0, 432.0])
    f[7, 0:128] = np.resize(np.concatenate([mids, -mids]), 128)
    f[7, 5] = 448.0
    f[8, 384:512] = np.resize([3.0e38, -1.0e-30, 1.0, 65504.0], 128)
    f[130:140, 130:135] = 1.0e4                                     # outlier patch
    bits = _bf16(f)
    if mode == "tensor":
        # one non-finite element makes the whole tensor NaN-scaled; test
        # that separately from the finite special cases
        fin = f.copy()
        fin[1, 128] = fin[2, 300] = fin[3, 400] = 0.0
        _check(fgs, _bf16(fin), mode, True, True)
        tiny = np.ldexp(synth.activations(128, 256, seed=9).view(np.int16).astype(np.float64) / 32768.0, -80)
        _check(fgs, _bf16(tiny), mode, True, True)
        zeros = np.zeros((128, 128))
        zeros[::2] = -0.0
        _check(fgs, _bf16(zeros), mode, True, True)
    _check(fgs, bits, mode, True, True)


def test_quant_tile_full_size_sampled(fgs):
    """Llama-3-8B activation shape (8192 x 4096, outlier channels), dual
    output, checked on sampled rows (row-wise tiles) and sampled columns
    (column-wise tiles)."""
    M, K = 8192, 4096
    bits = synth.activations(M, K, seed=0)
    x = _dev(bits)
    r = fgs.quantize_blockwise(x, "tile", rowwise=True, colwise=True)
    torch.cuda.synchronize()
    rs = sample_rows(M)
    q, s = oracle.quant_e4m3(bits[rs], "tile")
    assert np.array_equal(r.q[torch.from_numpy(rs).cuda()].cpu().numpy(), q)
    assert np.array_equal(r.scales[:, torch.from_numpy(rs).cuda()].cpu().numpy().T, s)
    cs = sample_rows(K, seed=1)
    qt, st = oracle.quant_e4m3(np.ascontiguousarray(bits[:, cs]), "tile", colwise=True)
    assert np.array_equal(r.qT[torch.from_numpy(cs).cuda()].cpu().numpy(), qt)
    assert np.array_equal(r.scalesT[:, torch.from_numpy(cs).cuda()].cpu().numpy().T, st)


@pytest.mark.parametrize("mode", ["block", "tensor"])
def test_quant_block_tensor_full_size(fgs, mode):
    """Llama-3-8B weight shape (6144 x 4096) with transposed codes."""
    N, K = 6144, 4096
    bits = synth.weights(N, K, seed=0)
    _check(fgs, bits, mode, True, True)


def test_quant_determinism(fgs):
    bits = synth.activations(1024, 1024, seed=5)
    x = _dev(bits)
    a = fgs.quantize_blockwise(x, "tile", colwise=True)
    b = fgs.quantize_blockwise(x, "tile", colwise=True)
    torch.cuda.synchronize()
    assert torch.equal(a.q, b.q) and torch.equal(a.qT, b.qT)
    assert torch.equal(a.scales, b.scales) and torch.equal(a.scalesT, b.scalesT)


def test_quant_strided_input(fgs):
    """A row stride larger than cols (a column slice of a wider tensor)."""
    bits = synth.activations(256, 640, seed=6)
    x = _dev(bits)[:, 128:512]
    r = fgs.quantize_blockwise(x, "tile", colwise=True)
    torch.cuda.synchronize()
    sub = np.ascontiguousarray(bits[:, 128:512])
    q, s = oracle.quant_e4m3(sub, "tile")
    qt, st = oracle.quant_e4m3(sub, "tile", colwise=True)
    assert np.array_equal(r.q.cpu().numpy(), q) and np.array_equal(r.scales.cpu().numpy().T, s)
    assert np.array_equal(r.qT.cpu().numpy(), qt) and np.array_equal(r.scalesT.cpu().numpy().T, st)


@pytest.mark.parametrize("ws_bytes", [4, 12, 4096])
def test_tensor_mode_workspace_sizes(fgs, ws_bytes):
    """The per-tensor amax pass keeps one partial per workgroup in the
    workspace; any size from one slot up gives the oracle's codes and scale
    (a 4-byte workspace runs one amax workgroup over every tile).  The
    workspace starts as garbage: no pass may rely on it being cleared."""
    bits = synth.activations(1024, 1536, seed=11)
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
    r = fgs.quantize_blockwise(_dev(bits), "tensor", rowwise=True, colwise=True, workspace=ws)
    torch.cuda.synchronize()
    q, s = oracle.quant_e4m3(bits, "tensor")
    qt, _ = oracle.quant_e4m3(bits, "tensor", colwise=True)
    assert np.array_equal(r.q.cpu().numpy(), q)
    assert np.array_equal(r.qT.cpu().numpy(), qt)
    assert r.scales.cpu().numpy().view(np.uint32)[0] == np.asarray(s, dtype=np.float32).reshape(-1).view(np.uint32)[0]
