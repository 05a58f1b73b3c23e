"""GPU parity of the GEMM epilogue that quantizes its BF16 output in 1x128
tiles for the next layer: the BF16 C is within one BF16 ulp of the oracle's
FP64 product (as for the plain GEMM), and the codes and scales are exactly
the oracle's 1x128 quantization of that BF16 C (the integer decisions taken
on the same BF16 values on both sides).

"Can you explain the role of FP8 precision in DeepSeek-V3 training",
sections "Fine-grained quantization" and "Online quantization" (the
activation tiles of the next layer, scaled from their own amax).
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import gemm_within_bf16_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def _e4m3_operand(fgs, bits, mode):
    q, s = oracle.quant_e4m3(bits, mode)
    s_abi = np.ascontiguousarray(s.T) if mode == "tile" else (s if mode == "block" else s.reshape(1))
    code = {"tensor": 0, "tile": 1, "block": 2}[mode]
    return fgs.Operand(torch.from_numpy(q).cuda(), torch.from_numpy(s_abi).cuda(), code), \
        oracle.dequant_e4m3(q, s, mode)


def _bits(c):
    return c.cpu().view(torch.int16).numpy().view(np.uint16)


def _check_codes(qq, c_bits, rows=None):
    qr, sr = oracle.quant_e4m3(c_bits, "tile")
    q = qq.q.cpu().numpy()
    s = qq.scales.cpu().numpy().T
    if rows is not None:
        q, s, qr, sr = q[rows], s[rows], qr[rows], sr[rows]
    assert np.array_equal(q, qr)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))


@pytest.mark.parametrize("amode,bmode", [("tile", "block"), ("tile", "tile"), ("tensor", "tensor")])
@pytest.mark.parametrize("M,N,K", [(520, 384, 384), (257, 768, 256), (1, 128, 128)])
def test_fp8out_dense(fgs, amode, bmode, M, N, K):
    A, ah = _e4m3_operand(fgs, synth.activations(M, K, seed=M), amode)
    B, bh = _e4m3_operand(fgs, synth.weights(N, K, seed=N), bmode)
    qq, c = fgs.gemm_block_scaled_fp8out(A, B)
    torch.cuda.synchronize()
    cref, sref = oracle.gemm_ref(ah, bh)
    ok, nbad = gemm_within_bf16_bound(c.float().cpu().numpy().astype(np.float64), cref, sref)
    assert ok, f"{nbad} BF16 outputs outside one ulp"
    _check_codes(qq, _bits(c))
    # without the BF16 output: the same codes
    qq2, c2 = fgs.gemm_block_scaled_fp8out(A, B, bf16_out=False)
    torch.cuda.synchronize()
    assert c2 is None
    assert torch.equal(qq2.q, qq.q) and torch.equal(qq2.scales.view(torch.int32), qq.scales.view(torch.int32))


@pytest.mark.parametrize("amode,bmode", [("tile", "block"), ("tile", "tensor"), ("tensor", "block")])
@pytest.mark.parametrize("M,N,K", [(520, 384, 384), (257, 768, 256), (8, 256, 128)])
@pytest.mark.parametrize("bf16_out", [True, False])
def test_fp8out_promoted_wide_tile(fgs, amode, bmode, M, N, K, bf16_out):
    """The promoted modes forced onto the 256 x 256 tile, whose accumulators
    are 16x16 output tiles (a row's 64 columns of a wave spread over four
    lanes): the epilogue's codes and scales equal the oracle's 1x128
    quantization of the BF16 C, with and without the BF16 output, and both
    tiles give the same codes (where their BF16 outputs agree bit for bit)."""
    A, ah = _e4m3_operand(fgs, synth.activations(M, K, seed=M + 11), amode)
    B, bh = _e4m3_operand(fgs, synth.weights(N, K, seed=N + 13), bmode)
    qq, c = fgs.gemm_block_scaled_fp8out(A, B, tile="wide")
    torch.cuda.synchronize()
    cref, sref = oracle.gemm_ref(ah, bh)
    ok, nbad = gemm_within_bf16_bound(c.float().cpu().numpy().astype(np.float64), cref, sref)
    assert ok, f"{nbad} BF16 outputs outside one ulp"
    _check_codes(qq, _bits(c))
    if not bf16_out:
        qq2, c2 = fgs.gemm_block_scaled_fp8out(A, B, bf16_out=False, tile="wide")
        torch.cuda.synchronize()
        assert c2 is None
        assert torch.equal(qq2.q, qq.q) and torch.equal(qq2.scales.view(torch.int32), qq.scales.view(torch.int32))
    # the plain BF16 GEMM on the same tile gives the same C
    c_plain = fgs.gemm_block_scaled(A, B, torch.bfloat16, tile="wide")
    torch.cuda.synchronize()
    assert torch.equal(c_plain.view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("policy", ["narrow", "wide"])
def test_fp8out_per_tensor_both_tiles_and_nan_row(fgs, policy):
    """Per-tensor operands on either workgroup tile (the wide tile pairs the
    waves of its two 1x128 tiles); a NaN code in one A row makes that
    output row NaN: scale NaN and every code 0x7F."""
    M, N, K = 520, 768, 384
    a = synth.activations(M, K, seed=3)
    q, s = oracle.quant_e4m3(a, "tensor")
    q = q.copy()
    q[77, 5] = 0x7F
    A = fgs.Operand(torch.from_numpy(q).cuda(), torch.from_numpy(s.reshape(1)).cuda(), 0)
    B, _ = _e4m3_operand(fgs, synth.weights(N, K, seed=4), "tensor")
    qq, c = fgs.gemm_block_scaled_fp8out(A, B, tile=policy)
    torch.cuda.synchronize()
    cb = _bits(c)
    _check_codes(qq, cb)
    assert np.all(qq.q.cpu().numpy()[77] == 0x7F) and np.all(np.isnan(qq.scales.cpu().numpy()[:, 77]))


def test_fp8out_grouped(fgs):
    """MoE gate/up forward with its output quantized for the next GEMM:
    ragged and empty experts; only the rows the experts cover are checked
    (and written)."""
    counts = np.array([0, 1, 130, 0, 257, 128, 3])
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T, N, K, G = int(offs[-1]), 256, 384, len(counts)
    A, ah = _e4m3_operand(fgs, synth.activations(T, K, seed=5), "tile")
    qs, ss, bhs = [], [], []
    for g in range(G):
        q, s = oracle.quant_e4m3(synth.weights(N, K, seed=40 + g), "block")
        qs.append(q)
        ss.append(s)
        bhs.append(oracle.dequant_e4m3(q, s, "block"))
    B = fgs.Operand(torch.from_numpy(np.concatenate(qs)).cuda(),
                    torch.from_numpy(np.concatenate([s[None] for s in ss])).cuda(), 2)
    qq, c = fgs.grouped_gemm_block_scaled_fp8out(A, B, torch.from_numpy(offs).cuda(), N)
    torch.cuda.synchronize()
    cref, sref = oracle.grouped_gemm_ref(ah, bhs, offs)
    ok, nbad = gemm_within_bf16_bound(c.float().cpu().numpy().astype(np.float64), cref, sref)
    assert ok, nbad
    _check_codes(qq, _bits(c))
