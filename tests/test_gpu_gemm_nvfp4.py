"""GPU parity of the NVFP4 GEMM (E2M1 codes with an E4M3 scale per 16
K-elements and an FP32 tensor scale on both operands) against the oracle's
FP64 product of the dequantized operands: |C - C_ref| <= 1e-5 * S + 1e-6
(FP32 out), within one BF16 ulp of the rounded reference (BF16 out).

"NVIDIA developed a method to train neural networks at 4-bit", section "How
it works".  Operands are quantized by the oracle (with the random Hadamard
transform and stochastic rounding where the wgrad orientation uses them)
and uploaded, so this isolates the GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import gemm_within_bf16_bound, gemm_within_fp32_bound, sample_rows

pytestmark = pytest.mark.gpu

RHT_SEED = synth.derived_seed(0, synth.TAG_RHT)
SR_SEED = synth.derived_seed(0, synth.TAG_SR)


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def nv_operand(fgs, bits, colwise=False, rht=False, stochastic=False, rows=None):
    q, s, ts = oracle.quant_nvfp4(bits, colwise=colwise, rht=rht, rht_seed=RHT_SEED,
                                  stochastic=stochastic, sr_seed=SR_SEED)
    K = q.shape[1] * 2
    deq = oracle.dequant_nvfp4(q if rows is None else q[rows], s if rows is None else s[rows], ts, K)
    op = fgs.Operand(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), fgs.SCALE_NV16_E4M3,
                     fgs.ELEM_E2M1, torch.tensor([ts], dtype=torch.float32, device="cuda"))
    return op, deq


def _check(fgs, A, B, ah, bh, out, rows=None, tile="auto"):
    c = fgs.gemm_block_scaled(A, B, out, tile=tile)
    torch.cuda.synchronize()
    c = c.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        c = c[rows]
    cref, sref = oracle.gemm_ref(ah, bh)
    if out == torch.float32:
        ok, worst = gemm_within_fp32_bound(c, cref, sref)
        assert ok, f"worst err/bound = {worst}"
    else:
        ok, nbad = gemm_within_bf16_bound(c, cref, sref)
        assert ok, f"{nbad} BF16 outputs outside one ulp"


@pytest.mark.parametrize("M,N,K", [(200, 130, 384), (1, 1, 128), (257, 129, 256), (256, 384, 1024), (520, 777, 384)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_nvfp4_gemm_ragged(fgs, M, N, K, out):
    A, ah = nv_operand(fgs, synth.activations(M, K, seed=M + 7))
    B, bh = nv_operand(fgs, synth.weights(N, K, seed=N + 9))
    _check(fgs, A, B, ah, bh, out)


@pytest.mark.parametrize("M,N,K", [(257, 129, 256), (520, 777, 384)])
def test_nvfp4_gemm_tile_policies_bit_identical(fgs, M, N, K):
    """The NVFP4 GEMM runs on either workgroup tile with the same bits."""
    A, ah = nv_operand(fgs, synth.activations(M, K, seed=M + 3))
    B, bh = nv_operand(fgs, synth.weights(N, K, seed=N + 5))
    res = {}
    for tile in ("narrow", "wide"):
        _check(fgs, A, B, ah, bh, torch.float32, tile=tile)
        res[tile] = fgs.gemm_block_scaled(A, B, torch.float32, tile=tile).cpu()
    assert torch.equal(res["narrow"].view(torch.uint8), res["wide"].view(torch.uint8))


def test_nvfp4_gemm_wgrad_rht_sr(fgs):
    """wgrad orientation at reduced size: dY^T (Student-t gradients, random
    Hadamard transform along the tokens, stochastic rounding) times X^T
    (transform, RNE); the transforms use one sign vector so they cancel in
    the product."""
    M, K, N = 1024, 640, 768
    dy = synth.gradients(M, N, seed=51)
    x = synth.activations(M, K, seed=52)
    A, ah = nv_operand(fgs, dy, colwise=True, rht=True, stochastic=True)
    B, bh = nv_operand(fgs, x, colwise=True, rht=True)
    _check(fgs, A, B, ah, bh, torch.float32)


def test_nvfp4_gemm_scale_extremes(fgs):
    """Blocks with zero, tiny and large E4M3 scales and a tensor scale far
    from 1 on each side."""
    M, N, K = 128, 256, 512
    a = oracle.bf16_bits_to_f32(synth.activations(M, K, seed=53)).copy() * np.float32(2.0 ** 40)
    b = oracle.bf16_bits_to_f32(synth.weights(N, K, seed=54)).copy() * np.float32(2.0 ** -60)
    a[:, 0:16] = 0.0
    a[::4, 16:32] *= np.float32(2.0 ** -12)
    b[::3, 32:48] *= np.float32(2.0 ** -9)
    A, ah = nv_operand(fgs, synth.f32_to_bf16_bits(a))
    B, bh = nv_operand(fgs, synth.f32_to_bf16_bits(b))
    _check(fgs, A, B, ah, bh, torch.float32)


def test_nvfp4_gemm_determinism(fgs):
    A, _ = nv_operand(fgs, synth.activations(512, 1024, seed=55))
    B, _ = nv_operand(fgs, synth.weights(384, 1024, seed=56))
    c1 = fgs.gemm_block_scaled(A, B)
    c2 = fgs.gemm_block_scaled(A, B)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


def test_nvfp4_gemm_wgrad_full_size_sampled(fgs):
    """12B-hybrid-like wgrad of the up projection at full size: A = dY^T
    [20480 x 8192] (gradients, random Hadamard transform along the 8192
    tokens, stochastic rounding), B = X^T [5120 x 8192] (transform, RNE);
    FP32 out.  The oracle quantizes the sampled rows of A under the whole
    tensor's scale (the other rows are uploaded as zero codes; the sampled
    output rows depend on the sampled A rows only) and all of B."""
    M, K, N = 8192, 5120, 20480
    dy = synth.gradients(M, N, seed=0)
    x = synth.activations(M, K, seed=0)
    rs = sample_rows(N)[::5]
    valsT = oracle.nvfp4_operand_values(dy, colwise=True, rht=True, rht_seed=RHT_SEED)
    ts = oracle.nvfp4_tensor_scale(valsT)
    qa = np.zeros((N, M // 2), dtype=np.uint8)
    sa = np.zeros((N, M // 16), dtype=np.uint8)
    for r in rs:
        q, s = oracle.quant_nvfp4_rows(valsT[r:r + 1], ts, True, SR_SEED, idx_base=int(r), idx_cs=N)
        qa[r], sa[r] = q[0], s[0]
    del valsT
    A = fgs.Operand(torch.from_numpy(qa).cuda(), torch.from_numpy(sa).cuda(), fgs.SCALE_NV16_E4M3,
                    fgs.ELEM_E2M1, torch.tensor([ts], dtype=torch.float32, device="cuda"))
    ah = oracle.dequant_nvfp4(qa[rs], sa[rs], ts, M)
    B, bh = nv_operand(fgs, x, colwise=True, rht=True)
    _check(fgs, A, B, ah, bh, torch.float32, rows=rs)
