"""GPU parity of the quantizers on tensors past 2^31 and 2^32 elements, where
element offsets and the stochastic-rounding index need all 64 bits.

"NVIDIA developed a method to train neural networks at 4-bit", section
"How it works" (NVFP4, stochastic rounding: the random word of an element
hashes its linear index, whose upper 32 bits are nonzero past 2^32
elements); "Can you explain the role of FP8 precision in DeepSeek-V3
training", section "Fine-grained quantization" (1x128 tiles, both
orientations); "Accelerating FP8 training performance with the NVIDIA NeMo
framework" (MXFP8, one E8M0 scale per 32 values); and the block-scaled GEMM
("Mixed precision framework") on an operand past 2^31 bytes.  The inputs are drawn on the GPU in chunks (seeded, bounded
to (-1, 1)), so the tensor amax of the NVFP4 case is fixed by one planted
value and sampled rows and columns are checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import gemm_within_fp32_bound

pytestmark = pytest.mark.gpu

SR_SEED = synth.derived_seed(0, synth.TAG_SR)


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def _uniform_bf16(rows, cols, seed, chunk_rows=2048):
    """BF16 [rows x cols] on the GPU, uniform in (-1, 1), drawn chunk by chunk."""
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(r0 + chunk_rows, rows)
        x[r0:r1] = (torch.rand((r1 - r0, cols), generator=g, device="cuda") * 1.96 - 0.98).to(torch.bfloat16)
    return x


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_nvfp4_sr_past_2_32_elements(fgs):
    """65664 x 65536 = 2^32 + 2^23 elements, row-wise with stochastic
    rounding: rows from 65536 on hash an index with upper word 1.  The
    planted 2.0 makes the tensor amax 2.0 (every other value lies in
    (-1, 1)), so each sampled row is quantized by the oracle under that
    tensor's scale."""
    rows, cols = 65664, 65536
    assert rows * cols > 2 ** 32
    x = _uniform_bf16(rows, cols, seed=5)
    x[3, 17] = 2.0
    r = fgs.quantize_nvfp4(x, rowwise=True, colwise=False, stochastic=True, sr_seed=SR_SEED)
    torch.cuda.synchronize()
    t0 = oracle.nvfp4_tensor_scale(np.array([[2.0]], dtype=np.float32))
    ts = r.tensor_scale.cpu().numpy()
    assert np.float32(ts[0]).view(np.uint32) == np.float32(t0).view(np.uint32)
    for row in (0, 3, 65535, 65536, 65537, 65600, 65663):
        bits = _bits(x[row:row + 1])
        vals = oracle.nvfp4_operand_values(bits)
        q, s = oracle.quant_nvfp4_rows(vals, t0, True, SR_SEED, idx_base=row * cols)
        assert np.array_equal(r.q[row].cpu().numpy(), q[0]), f"row {row}"
        assert np.array_equal(r.scales[row].cpu().numpy(), s[0]), f"row {row}"
    del r, x
    torch.cuda.empty_cache()


def test_e4m3_tile_dual_output_past_2_31_elements(fgs):
    """65664 x 32768 = 2^31 + 2^22 elements, 1x128 tiles in both
    orientations: the row-wise offsets of the last rows and the column-wise
    offsets of the last columns pass 2^31."""
    rows, cols = 65664, 32768
    assert rows * cols > 2 ** 31
    x = _uniform_bf16(rows, cols, seed=6)
    r = fgs.quantize_blockwise(x, "tile", rowwise=True, colwise=True)
    torch.cuda.synchronize()
    rs = np.array([0, 127, 65535, 65536, 65600, 65663])
    q, s = oracle.quant_e4m3(_bits(x[torch.from_numpy(rs).cuda()]), "tile")
    assert np.array_equal(r.q[torch.from_numpy(rs).cuda()].cpu().numpy(), q)
    assert np.array_equal(r.scales[:, torch.from_numpy(rs).cuda()].cpu().numpy().T, s)
    cs = np.array([0, 8191, 16384, 32767])
    qt, st = oracle.quant_e4m3(np.ascontiguousarray(_bits(x[:, torch.from_numpy(cs).cuda()])), "tile", colwise=True)
    assert np.array_equal(r.qT[torch.from_numpy(cs).cuda()].cpu().numpy(), qt)
    assert np.array_equal(r.scalesT[:, torch.from_numpy(cs).cuda()].cpu().numpy().T, st)
    del r, x
    torch.cuda.empty_cache()


def test_mx_dual_output_past_2_31_elements(fgs):
    """65664 x 32768 MXFP8, row-wise and column-wise: the same 64-bit
    offsets (the scale bytes of the last rows and columns, too)."""
    rows, cols = 65664, 32768
    x = _uniform_bf16(rows, cols, seed=7)
    r = fgs.quantize_mx(x, rowwise=True, colwise=True)
    torch.cuda.synchronize()
    rs = np.array([0, 65535, 65536, 65663])
    idx = torch.from_numpy(rs).cuda()
    q, s = oracle.quant_mx(_bits(x[idx]))
    assert np.array_equal(r.q[idx].cpu().numpy(), q)
    assert np.array_equal(r.scales[idx].cpu().numpy(), s)
    cs = np.array([0, 16383, 32767])
    cidx = torch.from_numpy(cs).cuda()
    qt, st = oracle.quant_mx(np.ascontiguousarray(_bits(x[:, cidx])), colwise=True)
    assert np.array_equal(r.qT[cidx].cpu().numpy(), qt)
    assert np.array_equal(r.scalesT[cidx].cpu().numpy(), st)
    del r, x
    torch.cuda.empty_cache()


def _e4m3_codes(rows, cols, seed):
    """Random finite E4M3 codes (every byte but 0x7F and 0xFF) on the GPU."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    r = torch.randint(0, 254, (rows, cols), generator=g, device="cuda", dtype=torch.int16)
    return (r + (r >= 127).to(torch.int16)).to(torch.uint8)


def test_gemm_operand_past_2_31_bytes(fgs):
    """A 65664 x 32768 operand (2^31 + 2^22 code bytes) with 1x128 scales
    against a 256 x 32768 operand with 128x128 scales, FP32 out: rows past
    65536 are checked against the oracle's product of the dequantized
    operands.  Codes and power-of-two-spread scales are drawn on the GPU."""
    M, N, K = 65664, 256, 32768
    qa = _e4m3_codes(M, K, seed=8)
    qb = _e4m3_codes(N, K, seed=9)
    g = torch.Generator(device="cuda")
    g.manual_seed(10)
    sa = torch.exp2(torch.randint(-6, 7, (K // 128, M), generator=g, device="cuda").float()) * 0.75
    sb = torch.exp2(torch.randint(-6, 7, (N // 128, K // 128), generator=g, device="cuda").float()) * 1.25
    A = fgs.Operand(qa, sa, 1)
    B = fgs.Operand(qb, sb, 2)
    c = fgs.gemm_block_scaled(A, B, torch.float32)
    torch.cuda.synchronize()
    rs = np.array([0, 65535, 65536, 65600, 65663])
    idx = torch.from_numpy(rs).cuda()
    a_hat = oracle.dequant_e4m3(qa[idx].cpu().numpy(), np.ascontiguousarray(sa[:, idx].cpu().numpy().T), "tile")
    b_hat = oracle.dequant_e4m3(qb.cpu().numpy(), sb.cpu().numpy(), "block")
    cref, sref = oracle.gemm_ref(a_hat, b_hat)
    ok, worst = gemm_within_fp32_bound(c[idx].cpu().numpy().astype(np.float64), cref, sref)
    assert ok, worst
    del c, qa, qb
    torch.cuda.empty_cache()
