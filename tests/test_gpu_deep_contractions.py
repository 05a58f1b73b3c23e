"""GPU parity at the longest contractions the bench times, at their full
launch shapes: the single FP32 accumulators of the per-tensor, MX and NVFP4
modes run over all of K here (up to 53248 deep), and the blockwise mode
promotes up to 224 partial sums per output.

"Can you explain the role of FP8 precision in DeepSeek-V3 training",
section "Increasing accumulation precision" (limited accumulation precision
is the reason partial sums are promoted to FP32); "Accelerating FP8 training
performance with the NVIDIA NeMo framework" (per-tensor and MXFP8 recipes);
"NVIDIA developed a method to train neural networks at 4-bit", "How it
works" (NVFP4).

Each operand is a full-size device buffer in the layout the bench passes,
launched with the bench's (automatic) tile choice.  Only sampled rows carry
oracle-quantized data: rows {0, 127, one hashed} of every 128-row tile of A,
and of six 128-row blocks of B (the first three, the middle one and the last
two, so the workgroup tiles at both edges are covered).  Every other row
holds the zero quantization of its mode (code 0 with scale 1, MX exponent
byte 127, NVFP4 scale byte 0), which is the oracle's quantization of the
same matrix with those rows zero; a kernel that reads a wrong row or a wrong
K block therefore gets a wrong (zero or misplaced) sum.  The sampled outputs
C[rows_A][:, rows_B] are checked element by element against the oracle's
FP64 product: |C - C_ref| <= 1e-5 * S + 1e-6 (FP32 out), one BF16 ulp of the
rounded reference (BF16 out).
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import gemm_within_bf16_bound, gemm_within_fp32_bound, sample_rows

pytestmark = pytest.mark.gpu

SR_SEED = synth.derived_seed(0, synth.TAG_SR)


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def b_sample_rows(rows, seed=1):
    """Rows {0, 127, one hashed} of six 128-row blocks: 0, 1, 2, the middle
    one and the last two (clipped to the blocks that exist)."""
    nb = (rows + 127) // 128
    blocks = sorted({b for b in (0, 1, 2, nb // 2, nb - 2, nb - 1) if 0 <= b < nb})
    g = np.random.default_rng(seed)
    out = []
    for b in blocks:
        r0, r1 = 128 * b, min(128 * b + 128, rows)
        out += [r0, r1 - 1, int(g.integers(r0, r1))]
    return np.unique(np.array(out))


def draw(kind, n, K, seed):
    if kind == "act":
        return synth.activations(n, K, seed=seed)
    if kind == "act_plain":
        return synth.activations(n, K, seed=seed, outliers=False)
    if kind == "grad":
        return synth.gradients(n, K, seed=seed)
    return synth.weights(n, K, seed=seed)


def e4m3_operand(fgs, R, K, rows, bits, mode):
    """Full-size E4M3 operand [R x K] whose rows `rows` hold `bits` quantized
    by the oracle in `mode`; every other row is zero.  Returns the Operand
    and the dequantized sampled rows (FP64)."""
    dev = "cuda"
    codes = torch.zeros((R, K), dtype=torch.uint8, device=dev)
    rows_t = torch.from_numpy(rows).to(dev)
    if mode == "tile":
        q, s = oracle.quant_e4m3(bits, "tile")
        scales = torch.ones((K // 128, R), dtype=torch.float32, device=dev)
        scales[:, rows_t] = torch.from_numpy(np.ascontiguousarray(s.T)).to(dev)
        deq = oracle.dequant_e4m3(q, s, "tile")
        codes[rows_t] = torch.from_numpy(q).to(dev)
    elif mode == "tensor":
        q, s = oracle.quant_e4m3(bits, "tensor")
        scales = torch.from_numpy(np.asarray(s, dtype=np.float32).reshape(1)).to(dev)
        deq = oracle.dequant_e4m3(q, s, "tensor")
        codes[rows_t] = torch.from_numpy(q).to(dev)
    else:
        # 128x128 blocks: quantize the blocks that hold sampled rows as a
        # compact matrix (their other rows zero), then place them
        blocks = np.unique(rows // 128)
        compact = np.zeros((128 * len(blocks), K), dtype=np.uint16)
        pos = {b: i for i, b in enumerate(blocks)}
        crow = np.array([128 * pos[r // 128] + r % 128 for r in rows])
        compact[crow] = bits
        q, s = oracle.quant_e4m3(compact, "block")
        scales = torch.ones(((R + 127) // 128, K // 128), dtype=torch.float32, device=dev)
        for b in blocks:
            i = pos[b]
            n = min(128, R - 128 * b)
            codes[128 * b:128 * b + n] = torch.from_numpy(q[128 * i:128 * i + n]).to(dev)
            scales[b] = torch.from_numpy(s[i]).to(dev)
        deq = oracle.dequant_e4m3(q, s, "block")[crow]
    return fgs.Operand(codes, scales, {"tile": 1, "tensor": 0, "block": 2}[mode]), deq


def mx_operand(fgs, R, K, rows, bits):
    dev = "cuda"
    q, s = oracle.quant_mx(bits)
    rows_t = torch.from_numpy(rows).to(dev)
    codes = torch.zeros((R, K), dtype=torch.uint8, device=dev)
    scales = torch.full((R, K // 32), 127, dtype=torch.uint8, device=dev)   # 2^0: a zero block
    codes[rows_t] = torch.from_numpy(q).to(dev)
    scales[rows_t] = torch.from_numpy(s).to(dev)
    return fgs.Operand(codes, scales, fgs.SCALE_MX32_E8M0), oracle.dequant_mx(q, s)


def nv_operand(fgs, R, K, rows, bits, stochastic):
    dev = "cuda"
    q, s, ts = oracle.quant_nvfp4(bits, stochastic=stochastic, sr_seed=SR_SEED)
    rows_t = torch.from_numpy(rows).to(dev)
    codes = torch.zeros((R, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.zeros((R, K // 16), dtype=torch.uint8, device=dev)     # E4M3 0: a zero block
    codes[rows_t] = torch.from_numpy(q).to(dev)
    scales[rows_t] = torch.from_numpy(s).to(dev)
    op = fgs.Operand(codes, scales, fgs.SCALE_NV16_E4M3, fgs.ELEM_E2M1,
                     torch.tensor([ts], dtype=torch.float32, device=dev))
    return op, oracle.dequant_nvfp4(q, s, ts, K)


def run_and_check(fgs, A, B, ah, bh, ra, rb, out):
    c = fgs.gemm_block_scaled(A, B, out)
    got = c[torch.from_numpy(ra).cuda()][:, torch.from_numpy(rb).cuda()]
    torch.cuda.synchronize()
    got = got.float().cpu().numpy().astype(np.float64)
    del c
    cref, sref = oracle.gemm_ref(ah, bh)
    if out == torch.float32:
        ok, worst = gemm_within_fp32_bound(got, cref, sref)
        assert ok, f"worst err/bound = {worst}"
    else:
        ok, nbad = gemm_within_bf16_bound(got, cref, sref)
        assert ok, f"{nbad} BF16 outputs outside one ulp"
    # the sampled outputs are not trivially zero
    assert np.count_nonzero(cref) > 0.9 * cref.size


# Llama-3-8B: down fwd (contraction 14336) and gate/up dgrad (contraction
# 28672: dY [8192 x 28672] against W^T [4096 x 28672]), both recipes
E4M3_CASES = [("down_fwd", 8192, 4096, 14336, "act", "weight"),
              ("gate_up_dgrad", 8192, 4096, 28672, "grad", "weight")]
RECIPES = [("blockwise", "tile", "block"), ("per_tensor", "tensor", "tensor")]


@pytest.mark.parametrize("case", E4M3_CASES, ids=[c[0] for c in E4M3_CASES])
@pytest.mark.parametrize("recipe", RECIPES, ids=[r[0] for r in RECIPES])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_llama8b_deep_contraction(fgs, case, recipe, out):
    name, M, N, K, akind, bkind = case
    _, amode, bmode = recipe
    ra, rb = sample_rows(M), b_sample_rows(N)
    A, ah = e4m3_operand(fgs, M, K, ra, draw(akind, len(ra), K, seed=K + 1), amode)
    B, bh = e4m3_operand(fgs, N, K, rb, draw(bkind, len(rb), K, seed=K + 2), bmode)
    run_and_check(fgs, A, B, ah, bh, ra, rb, out)


# Llama-3.1-405B MXFP8 (one GPU's share): down fwd (contraction 53248) and
# gate/up fwd (N = 106496)
MX_CASES = [("down_fwd", 4096, 16384, 53248), ("gate_up_fwd", 4096, 106496, 16384)]


@pytest.mark.parametrize("case", MX_CASES, ids=[c[0] for c in MX_CASES])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_mx405b_deep_contraction(fgs, case, out):
    name, M, N, K = case
    ra, rb = sample_rows(M), b_sample_rows(N)
    A, ah = mx_operand(fgs, M, K, ra, draw("act_plain", len(ra), K, seed=K + 3))
    B, bh = mx_operand(fgs, N, K, rb, draw("weight", len(rb), K, seed=K + 4))
    run_and_check(fgs, A, B, ah, bh, ra, rb, out)


# 12B-hybrid NVFP4: down fwd (X [8192 x 20480] against W_down [5120 x
# 20480]) and up dgrad (dY [8192 x 20480], stochastically rounded, against
# W_up^T [5120 x 20480])
NV_CASES = [("down_fwd", 8192, 5120, 20480, "act", False), ("up_dgrad", 8192, 5120, 20480, "grad", True)]


@pytest.mark.parametrize("case", NV_CASES, ids=[c[0] for c in NV_CASES])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_nvfp4_12b_deep_contraction(fgs, case, out):
    name, M, N, K, akind, sr = case
    ra, rb = sample_rows(M), b_sample_rows(N)
    A, ah = nv_operand(fgs, M, K, ra, draw(akind, len(ra), K, seed=K + 5), sr)
    B, bh = nv_operand(fgs, N, K, rb, draw("weight", len(rb), K, seed=K + 6), False)
    run_and_check(fgs, A, B, ah, bh, ra, rb, out)
