"""GPU parity of per-tensor delayed scaling (E4M3 and E5M2, bit-exact codes,
scales and recorded amaxes against the oracle) and of the GEMM on E5M2
operands (|C - C_ref| <= 1e-5 * S + 1e-6 for FP32 out, one BF16 ulp for
BF16 out, C_ref the FP64 product of the dequantized operands).

"Can you explain the role of FP8 precision in DeepSeek-V3 training",
sections "Online quantization" (delayed scaling from historical maxima is
what online scaling replaces) and "Unified E4M3 format" (the hybrid recipe:
E4M3 forward, E5M2 backward).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import gemm_within_bf16_bound, gemm_within_fp32_bound, sample_rows

pytestmark = pytest.mark.gpu

F32 = np.float32
ELEMS = ["e4m3", "e5m2"]


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def _gpu_delayed(fgs, x_bits, elem, hist, slot, rowwise=True, colwise=True):
    x = synth.to_torch_bf16(x_bits).cuda()
    h = torch.from_numpy(np.asarray(hist, F32).copy()).cuda()
    qq = fgs.quantize_delayed(x, h, slot, elem, rowwise=rowwise, colwise=colwise)
    torch.cuda.synchronize()
    q = qq.q.cpu().numpy() if rowwise else None
    qT = qq.qT.cpu().numpy() if colwise else None
    return q, qT, qq.scales.cpu().numpy()[0], h.cpu().numpy()


def _check(fgs, x_bits, elem, hist, slot, rowwise=True, colwise=True):
    q, qT, s, h_after = _gpu_delayed(fgs, x_bits, elem, hist, slot, rowwise, colwise)
    oq, os_, oam = oracle.quant_delayed(x_bits, elem, hist)
    assert np.float32(s).tobytes() == np.float32(os_).tobytes(), (s, os_)
    if rowwise:
        assert np.array_equal(q, oq)
    if colwise:
        assert np.array_equal(qT, oq.T)
    want_h = np.asarray(hist, F32).copy()
    want_h[slot] = oam
    # equal entries, NaN where NaN (a NaN's payload carries no meaning)
    assert np.array_equal(h_after, want_h, equal_nan=True)
    assert np.array_equal(np.signbit(h_after), np.signbit(want_h))
    return oam


@pytest.mark.parametrize("elem", ELEMS)
def test_delayed_quant_wide_row_stride(fgs, elem):
    """A row stride of 2^24 + 8 elements, so 128 rows of it pass 2^31: the
    kernel then takes 64-bit offsets and one tile per workgroup (below that,
    32-bit offsets and several tiles per workgroup).  Row-wise codes, scale
    and the recorded amax against the oracle."""
    rows, cols, ldx = 2, 384, (1 << 24) + 8
    xb = synth.gradients(rows, cols, seed=77) if elem == "e5m2" else synth.activations(rows, cols, seed=77)
    big = torch.empty((rows, ldx), dtype=torch.bfloat16, device="cuda")
    big[:, :cols] = synth.to_torch_bf16(xb).cuda()
    x = big[:, :cols]
    amax = F32(np.abs(oracle.bf16_bits_to_f32(xb)).max())
    hist = [amax / F32(2.0), F32(0.0)]
    h = torch.from_numpy(np.asarray(hist, F32).copy()).cuda()
    qq = fgs.quantize_delayed(x, h, 1, elem, rowwise=True, colwise=False)
    torch.cuda.synchronize()
    oq, os_, oam = oracle.quant_delayed(xb, elem, hist)
    assert np.array_equal(qq.q.cpu().numpy(), oq)
    assert np.float32(qq.scales.cpu().numpy()[0]).tobytes() == np.float32(os_).tobytes()
    assert h.cpu().numpy()[1] == oam
    del big


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("rows,cols,colwise", [(256, 384, True), (128, 200, True), (300, 256, False), (1, 8, False)])
def test_delayed_quant_ragged_with_saturation(fgs, elem, rows, cols, colwise):
    """The history's max is a quarter of this tensor's amax, so the largest
    values saturate; the other two entries are left alone."""
    x = synth.gradients(rows, cols, seed=rows + cols) if elem == "e5m2" else synth.activations(rows, cols, seed=rows)
    amax = F32(np.abs(oracle.bf16_bits_to_f32(x)).max())
    _check(fgs, x, elem, [amax / F32(4.0), F32(0.5) * amax, F32(0.0)], 2, colwise=colwise)


@pytest.mark.parametrize("elem", ELEMS)
def test_delayed_quant_special_values(fgs, elem):
    x = synth.activations(128, 256, seed=61)
    xf = oracle.bf16_bits_to_f32(x).copy()
    xf[3, 17] = np.nan
    xf[70, 200] = -np.inf
    xf[5:9] = 0.0
    xf[5:9:2, ::3] = -0.0
    xb = synth.f32_to_bf16_bits(xf)
    _check(fgs, xb, elem, [2.0, 0.0], 0)                       # NaN amax recorded, Inf saturates
    _check(fgs, xb, elem, [np.nan, 3.0], 1)                    # NaN scale: every code 0x7F
    _check(fgs, xb, elem, [np.inf], 0)
    _check(fgs, xb, elem, [0.0, 0.0, 0.0], 1)                  # empty history: scale 1
    tiny = synth.f32_to_bf16_bits(oracle.bf16_bits_to_f32(synth.activations(128, 128, seed=62)) * F32(2.0 ** -120))
    _check(fgs, tiny, elem, [F32(2.0 ** -118)], 0)             # subnormal-range quotients and scale


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("log2_scale", [-61, -60, 60, 61])
def test_delayed_quant_scale_range_edges(fgs, elem, log2_scale):
    """Scales on either side of the kernel's fast-path range [2^-60, 2^60]
    (outside it every quotient takes the IEEE division): the history's max is
    fmax * 2^log2_scale, so s is that power of two exactly, and x spans the
    code range around it (with saturating outliers), zeros and -0 included."""
    fmax = F32(57344.0) if elem == "e5m2" else F32(448.0)
    xf = oracle.bf16_bits_to_f32(synth.activations(256, 256, seed=63 + log2_scale)).astype(np.float64)
    xf[9, :] *= 1e5                 # saturates in either format
    xf *= np.ldexp(1.0, log2_scale)
    xf[7, :] = 0.0
    xf[7, ::2] = -0.0
    xb = synth.f32_to_bf16_bits(xf.astype(F32))
    _check(fgs, xb, elem, [F32(np.ldexp(fmax, log2_scale)), F32(0.0)], 1)


@pytest.mark.parametrize("elem", ELEMS)
def test_delayed_rolling_window(fgs, elem):
    """Five steps on one device history of three entries (slot = step % 3):
    every step's codes, scale and history match the oracle run on the
    oracle's own history."""
    H = 3
    h_gpu = torch.zeros(H, dtype=torch.float32, device="cuda")
    h_ref = np.zeros(H, F32)
    for k in range(5):
        x = synth.gradients(256, 256, seed=70 + k)
        xb = synth.f32_to_bf16_bits(oracle.bf16_bits_to_f32(x) * F32(2.0 ** (2 * k - 4)))
        qq = fgs.quantize_delayed(synth.to_torch_bf16(xb).cuda(), h_gpu, k % H, elem, rowwise=True, colwise=True)
        torch.cuda.synchronize()
        oq, os_, oam = oracle.quant_delayed(xb, elem, h_ref)
        assert float(qq.scales.cpu()[0]) == float(os_) or (math.isnan(os_) and math.isnan(float(qq.scales.cpu()[0])))
        assert np.array_equal(qq.q.cpu().numpy(), oq) and np.array_equal(qq.qT.cpu().numpy(), oq.T)
        h_ref[k % H] = oam
        assert np.array_equal(h_gpu.cpu().numpy(), h_ref), k


def test_delayed_empty_tensor_records_zero(fgs):
    h = torch.tensor([5.0, 7.0], dtype=torch.float32, device="cuda")
    qq = fgs.quantize_delayed(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), h, 1, "e5m2",
                              rowwise=True, colwise=False)
    torch.cuda.synchronize()
    assert float(qq.scales.cpu()[0]) == float(F32(7.0) / F32(57344.0))
    assert h.cpu().tolist() == [5.0, 0.0]


# ------------------------------------------------------------- GEMM --------
def _tensor_operand(fgs, bits, elem, hist, colwise=False, rows=None):
    q, s, _ = oracle.quant_delayed(bits, elem, hist, colwise=colwise)
    code = fgs.ELEM_E5M2 if elem == "e5m2" else fgs.ELEM_E4M3
    op = fgs.Operand(torch.from_numpy(q).cuda(), torch.tensor([s], dtype=torch.float32, device="cuda"),
                     fgs.SCALE_TENSOR, code)
    return op, oracle.dequant_tensor(q if rows is None else q[rows], s, elem)


def _gemm_check(fgs, A, B, ah, bh, out, rows=None):
    c = fgs.gemm_block_scaled(A, B, out)
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


@pytest.mark.parametrize("ea,eb", [("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")])
@pytest.mark.parametrize("M,N,K", [(200, 130, 384), (257, 129, 256), (520, 777, 384)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_e5m2_gemm_ragged(fgs, ea, eb, M, N, K, out):
    a = synth.gradients(M, K, seed=M) if ea == "e5m2" else synth.activations(M, K, seed=M)
    b = synth.gradients(N, K, seed=N + 1) if eb == "e5m2" else synth.weights(N, K, seed=N + 1)
    ha = [F32(np.abs(oracle.bf16_bits_to_f32(a)).max()) * F32(0.75)]     # some saturation
    hb = [F32(np.abs(oracle.bf16_bits_to_f32(b)).max())]
    A, ah = _tensor_operand(fgs, a, ea, ha)
    B, bh = _tensor_operand(fgs, b, eb, hb)
    _gemm_check(fgs, A, B, ah, bh, out)


@pytest.mark.parametrize("ea,eb", [("e5m2", "e4m3"), ("e5m2", "e5m2")])
def test_e5m2_gemm_tile_policies_bit_identical(fgs, ea, eb):
    M, N, K = 520, 777, 384
    a = synth.gradients(M, K, seed=5)
    b = synth.weights(N, K, seed=6) if eb == "e4m3" else synth.gradients(N, K, seed=6)
    A, _ = _tensor_operand(fgs, a, ea, [1e-2])
    B, _ = _tensor_operand(fgs, b, eb, [0.1])
    res = {}
    for tile in ("narrow", "wide"):
        res[tile] = fgs.gemm_block_scaled(A, B, torch.float32, tile=tile).cpu()
    assert torch.equal(res["narrow"].view(torch.int32), res["wide"].view(torch.int32))


@pytest.mark.parametrize("orient", ["dgrad", "wgrad"])
def test_hybrid_llama8b_qkv_sampled(fgs, orient):
    """Llama-3-8B QKV projection at full size (M = 8192 tokens, K = 4096,
    N = 6144) in the hybrid recipe: dY in E5M2, W and X in E4M3, per-tensor
    delayed scales from a history; sampled output rows."""
    M, K, N = 8192, 4096, 6144
    dy = synth.gradients(M, N, seed=0)
    hist_dy = [F32(0.02)]
    if orient == "dgrad":
        w = synth.weights(N, K, seed=0)
        rs = sample_rows(M)
        A, ah = _tensor_operand(fgs, dy, "e5m2", hist_dy, rows=rs)
        B, bh = _tensor_operand(fgs, w, "e4m3", [F32(0.1)], colwise=True)
    else:
        x = synth.activations(M, K, seed=0)
        rs = sample_rows(N)
        A, ah = _tensor_operand(fgs, dy, "e5m2", hist_dy, colwise=True, rows=rs)
        B, bh = _tensor_operand(fgs, x, "e4m3", [F32(200.0)], colwise=True)
    _gemm_check(fgs, A, B, ah, bh, torch.bfloat16 if orient == "dgrad" else torch.float32, rows=rs)
