"""GPU parity of the block-scaled FP8 GEMM and its grouped (MoE) variant
against the oracle's FP64 product of the dequantized operands:
|C - C_ref| <= 1e-5 * sum_k |a_k b_k| + 1e-6 (FP32 out), within one BF16 ulp
of the rounded reference (BF16 out).

"Can you explain the role of FP8 precision in DeepSeek-V3 training",
sections "Mixed precision framework", "Fine-grained quantization",
"Increasing accumulation precision".  Operands are quantized by the oracle
and uploaded, so this isolates the GEMM from the quantization kernels.
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import gemm_within_bf16_bound, gemm_within_fp32_bound, sample_rows

pytestmark = pytest.mark.gpu

MODE_CODE = {"tensor": 0, "tile": 1, "block": 2}


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def oracle_operand(fgs, bits, mode, colwise=False, rows_for_ref=None):
    """Quantize with the oracle; return (GPU Operand, dequantized FP64 rows)."""
    q, s = oracle.quant_e4m3(bits, mode, colwise=colwise)
    if mode == "tile":
        s_abi = np.ascontiguousarray(s.T)
    elif mode == "block":
        s_abi = s
    else:
        s_abi = s.reshape(1)
    if rows_for_ref is None:
        deq = oracle.dequant_e4m3(q, s, mode)
    else:
        qr = q[rows_for_ref]
        if mode == "tile":
            deq = oracle.dequant_e4m3(qr, s[rows_for_ref], mode)
        elif mode == "tensor":
            deq = oracle.dequant_e4m3(qr, s, mode)
        else:
            full = oracle.dequant_e4m3(q, s, mode)
            deq = full[rows_for_ref]
    op = fgs.Operand(torch.from_numpy(q).cuda(), torch.from_numpy(np.ascontiguousarray(s_abi)).cuda(),
                     MODE_CODE[mode])
    return op, deq


def _run_and_check(fgs, A, B, a_hat, b_hat, out_dtype, rows=None, tile="auto"):
    c = fgs.gemm_block_scaled(A, B, out_dtype, tile=tile)
    torch.cuda.synchronize()
    c = c.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        c = c[rows]
    cref, sref = oracle.gemm_ref(a_hat, b_hat)
    if out_dtype == torch.float32:
        ok, worst = gemm_within_fp32_bound(c, cref, sref)
        assert ok, f"worst err/bound = {worst}"
    else:
        ok, nbad = gemm_within_bf16_bound(c, cref, sref)
        assert ok, f"{nbad} BF16 outputs outside one ulp"


def test_tiny_blockwise_fp32(fgs):
    """128x256 A ~ N(0,1), 256x256 B ~ N(0,0.02), seed 0; A in 1x128 tiles,
    B in 128x128 blocks; C = A B^T in FP32."""
    a_bits = synth.activations(128, 256, seed=0)
    b_bits = synth.weights(256, 256, seed=0)
    A, ah = oracle_operand(fgs, a_bits, "tile")
    B, bh = oracle_operand(fgs, b_bits, "block")
    _run_and_check(fgs, A, B, ah, bh, torch.float32)


MODES = [("tile", "block"), ("tile", "tile"), ("tensor", "tensor"), ("tile", "tensor"),
         ("tensor", "block"), ("tensor", "tile")]


@pytest.mark.parametrize("amode,bmode", MODES)
@pytest.mark.parametrize("M,N,K", [(200, 130, 384), (1, 1, 128), (257, 129, 256), (128, 384, 1024), (520, 777, 384)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_modes_ragged(fgs, amode, bmode, M, N, K, out):
    a_bits = synth.activations(M, K, seed=M + K)
    b_bits = synth.weights(N, K, seed=N + K)
    A, ah = oracle_operand(fgs, a_bits, amode)
    B, bh = oracle_operand(fgs, b_bits, bmode)
    _run_and_check(fgs, A, B, ah, bh, out)


@pytest.mark.parametrize("M,N,K", [(257, 129, 256), (520, 777, 384), (1000, 600, 512)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_tile_policies_bit_identical(fgs, M, N, K, out):
    """Per-tensor x per-tensor runs on either workgroup tile (256 x 128 or
    256 x 256); both meet the bound and give the same bits."""
    A, ah = oracle_operand(fgs, synth.activations(M, K, seed=M), "tensor")
    B, bh = oracle_operand(fgs, synth.weights(N, K, seed=N), "tensor")
    res = {}
    for tile in ("narrow", "wide"):
        _run_and_check(fgs, A, B, ah, bh, out, tile=tile)
        res[tile] = fgs.gemm_block_scaled(A, B, out, tile=tile).cpu()
    assert torch.equal(res["narrow"].view(torch.uint8), res["wide"].view(torch.uint8))


def test_gemm_row_stride_and_ldc(fgs):
    """Operand row stride larger than K and an output with ldc > N."""
    M, N, K = 192, 160, 256
    a_bits = synth.activations(M, K, seed=1)
    b_bits = synth.weights(N, K, seed=2)
    A, ah = oracle_operand(fgs, a_bits, "tile")
    B, bh = oracle_operand(fgs, b_bits, "block")
    wide = torch.zeros((M, K + 128), dtype=torch.uint8, device="cuda")
    wide[:, :K] = A.data
    A2 = fgs.Operand(wide, A.scales, A.scale_mode)
    assert A2.c_struct().ld == K + 128
    out = torch.full((M, N + 40), 7.0, dtype=torch.float32, device="cuda")
    fgs.gemm_block_scaled(A2, B, torch.float32, out=out[:, :N], K=K)
    torch.cuda.synchronize()
    c = out.cpu().numpy().astype(np.float64)
    cref, sref = oracle.gemm_ref(ah, bh)
    ok, worst = gemm_within_fp32_bound(c[:, :N], cref, sref)
    assert ok, worst
    assert np.all(c[:, N:] == 7.0)


@pytest.mark.parametrize("tile", ["narrow", "wide"])
def test_gemm_row_stride_at_the_limit(fgs, tile):
    """A row stride of 2^24 - 16 bytes, the largest the 32-bit lane offsets
    (row within the tile x stride) admit: a 256-row A spans 4 GiB, and its
    last row's offset lands just under 2^32."""
    M, N, K = 256, 256, 256
    ld = (1 << 24) - 16
    a_bits = synth.activations(M, K, seed=11)
    b_bits = synth.weights(N, K, seed=12)
    A, ah = oracle_operand(fgs, a_bits, "tile")
    B, bh = oracle_operand(fgs, b_bits, "block")
    wide = torch.zeros((M, ld), dtype=torch.uint8, device="cuda")
    wide[:, :K] = A.data
    A2 = fgs.Operand(wide, A.scales, A.scale_mode)
    assert A2.c_struct().ld == ld
    c = fgs.gemm_block_scaled(A2, B, torch.float32, K=K, tile=tile)
    torch.cuda.synchronize()
    del wide
    cref, sref = oracle.gemm_ref(ah, bh)
    ok, worst = gemm_within_fp32_bound(c.cpu().numpy().astype(np.float64), cref, sref)
    assert ok, worst


def test_gemm_adversarial_promotion(fgs):
    """Each 128-K block of A has its own scale spanning 2^-20 .. 2^20, so an
    accumulator without per-block FP32 promotion of the scale would fail."""
    M, N, K = 128, 128, 1024
    a = oracle.bf16_bits_to_f32(synth.activations(M, K, seed=7, outliers=False)).copy()
    for kb in range(K // 128):
        a[:, kb * 128:(kb + 1) * 128] *= np.float32(2.0 ** (5 * kb - 20))
    a_bits = synth.f32_to_bf16_bits(a)
    b_bits = synth.weights(N, K, seed=8)
    A, ah = oracle_operand(fgs, a_bits, "tile")
    B, bh = oracle_operand(fgs, b_bits, "block")
    _run_and_check(fgs, A, B, ah, bh, torch.float32)


def test_gemm_determinism(fgs):
    a_bits = synth.activations(512, 1024, seed=3)
    b_bits = synth.weights(768, 1024, seed=4)
    A, _ = oracle_operand(fgs, a_bits, "tile")
    B, _ = oracle_operand(fgs, b_bits, "block")
    c1 = fgs.gemm_block_scaled(A, B)
    c2 = fgs.gemm_block_scaled(A, B)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


# ------------------------------------------------------------------ grouped --
def _grouped_case(fgs, counts, N, K, out=torch.float32, seed=0, dgrad=False):
    """Grouped GEMM of row-wise 1x128 A against per-group 128x128 B.  With
    dgrad=True, A is a gradient and each group's B is the transpose of a
    forward weight W_g [K x N] (a layer N -> K), quantized column-wise: the
    GEMM contracts over the forward layer's output dimension K."""
    counts = np.asarray(counts)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(offs[-1])
    G = len(counts)
    a_bits = synth.gradients(total, K, seed=seed) if dgrad else synth.activations(total, K, seed=seed)
    A, ah = oracle_operand(fgs, a_bits, "tile")
    qs, ss, bhs = [], [], []
    for g in range(G):
        if dgrad:
            wb = synth.weights(K, N, seed=seed + 100 + g)          # forward weight [K out x N in]
            q, s = oracle.quant_e4m3(wb, "block", colwise=True)    # W_g^T codes [N x K]
        else:
            wb = synth.weights(N, K, seed=seed + 100 + g)
            q, s = oracle.quant_e4m3(wb, "block")
        qs.append(q)
        ss.append(s)
        bhs.append(oracle.dequant_e4m3(q, s, "block"))
    B = fgs.Operand(torch.from_numpy(np.concatenate(qs)).cuda(),
                    torch.from_numpy(np.concatenate([s[None] for s in ss])).cuda(), 2)
    off_t = torch.from_numpy(offs).cuda()
    c = torch.full((total, N), 3.0, dtype=out, device="cuda")
    fgs.grouped_gemm_block_scaled(A, B, off_t, N, out_dtype=out, out=c)
    torch.cuda.synchronize()
    c = c.float().cpu().numpy().astype(np.float64)
    cref, sref = oracle.grouped_gemm_ref(ah, bhs, offs)
    if out == torch.float32:
        ok, worst = gemm_within_fp32_bound(c, cref, sref)
        assert ok, worst
    else:
        ok, nbad = gemm_within_bf16_bound(c, cref, sref)
        assert ok, nbad


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_grouped_ragged_and_empty(fgs, out):
    _grouped_case(fgs, [0, 1, 130, 0, 257, 128, 3], N=256, K=384, out=out)


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_grouped_dgrad_orientation(fgs, out):
    """MoE expert dgrad: dX_g = dY_g W_g with W_g^T taken from the column-wise
    (transposed) 128x128 quantization of each expert's forward weight."""
    _grouped_case(fgs, [0, 1, 130, 0, 257, 128, 3], N=384, K=256, out=out, seed=3, dgrad=True)


def test_grouped_single_group_equals_dense(fgs):
    _grouped_case(fgs, [300], N=200, K=256)


def test_grouped_many_groups(fgs):
    """300 groups (more than one 256-wide scan chunk), Zipf-like counts."""
    counts = synth.expert_counts(tokens=4000, experts=300, seed=1)
    _grouped_case(fgs, counts, N=128, K=128, seed=5)


def test_grouped_long_groups_every_output(fgs):
    """Groups of 256 rows or more (the 256 x 256 tile's launch) over 2048
    columns: 4 + 3 + 6 + 4 m-tiles x 8 n-tiles = 136 tiles, so the device
    schedule deals two full blocks of 64 workgroups (each XCD taking 8
    consecutive tiles, blocks alternating between the two ends of the tile
    order) and a partial one; every output is checked."""
    _grouped_case(fgs, [1000, 700, 1300, 1000], N=2048, K=256, out=torch.bfloat16, seed=9)


# ------------------------------------------------------- full-size layer --
@pytest.mark.parametrize("orient", ["fwd", "dgrad", "wgrad"])
def test_llama8b_qkv_layer_sampled(fgs, orient):
    """Llama-3-8B QKV projection (K, N) = (4096, 6144), M = 8192 tokens,
    1x128 x 128x128 blockwise; sampled rows against the oracle."""
    M, K, N = 8192, 4096, 6144
    if orient == "fwd":
        a_bits = synth.activations(M, K, seed=0)
        b_bits = synth.weights(N, K, seed=0)
        a_mode, b_mode, a_col, b_col = "tile", "block", False, False
    elif orient == "dgrad":
        a_bits = synth.gradients(M, N, seed=0)          # dY [M x N], contraction over N
        b_bits = synth.weights(N, K, seed=0)            # W^T codes [K x N]
        a_mode, b_mode, a_col, b_col = "tile", "block", False, True
    else:
        a_bits = synth.gradients(M, N, seed=0)          # dY^T [N x M], contraction over M
        b_bits = synth.activations(M, K, seed=0)        # X^T  [K x M]
        a_mode, b_mode, a_col, b_col = "tile", "tile", True, True
    rows_total = a_bits.shape[1] if a_col else a_bits.shape[0]
    rs = sample_rows(rows_total)
    A, ah = oracle_operand(fgs, a_bits, a_mode, colwise=a_col, rows_for_ref=rs)
    B, bh = oracle_operand(fgs, b_bits, b_mode, colwise=b_col)
    out = torch.float32 if orient == "wgrad" else torch.bfloat16
    _run_and_check(fgs, A, B, ah, bh, out, rows=rs)


# ------------------------------------------------- full-size MoE (sampled) --
@pytest.mark.parametrize("N,K", [(4096, 7168), (7168, 2048)], ids=["gate_up", "down"])
def test_grouped_deepseek_moe_sampled(fgs, N, K):
    """DeepSeek-V3 MoE grouped GEMM at full size: 256 experts, 32768 routed
    rows (4096 tokens x top-8) with seeded Zipf(1.1) counts, one expert made
    empty; gate/up (K, N) = (7168, 4096) and down (2048, 7168).  Only the
    sampled experts (the largest, one just over 128 rows, one under 16) carry
    oracle-quantized weights and only the sampled rows oracle-quantized
    activations; every other code is zero (scale 1), so a row that reads the
    wrong expert or the wrong rows gives a wrong (zero) result."""
    G = 256
    counts = synth.expert_counts(32768, G, 1.1, seed=0).copy()
    empty = G - 1
    counts[0] += counts[empty]
    counts[empty] = 0
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    total = int(offs[-1])
    mid = int(np.flatnonzero((counts > 128) & (counts < 256))[0])
    small = int(np.flatnonzero((counts > 0) & (counts < 16))[0])
    experts = [0, mid, small]
    rows = []
    for g in experts:
        r0, r1 = int(offs[g]), int(offs[g + 1])
        for d in (0, 1, 127, 128, 255, 256, (r1 - r0) // 2, r1 - r0 - 2, r1 - r0 - 1):
            if 0 <= d < r1 - r0:
                rows.append(r0 + d)
    rows = np.unique(np.array(rows))

    # activations: oracle-quantized sampled rows, zero codes elsewhere
    a_bits = synth.activations(len(rows), K, seed=21)
    qa, sa = oracle.quant_e4m3(a_bits, "tile")
    ah = oracle.dequant_e4m3(qa, sa, "tile")
    qa_full = torch.zeros((total, K), dtype=torch.uint8)
    qa_full[torch.from_numpy(rows)] = torch.from_numpy(qa)
    sa_full = torch.ones((K // 128, total), dtype=torch.float32)
    sa_full[:, torch.from_numpy(rows)] = torch.from_numpy(np.ascontiguousarray(sa.T))
    A = fgs.Operand(qa_full.cuda(), sa_full.cuda(), 1)

    # weights: oracle-quantized for the sampled experts, zero codes elsewhere
    qb = torch.zeros((G * N, K), dtype=torch.uint8, device="cuda")
    sb = torch.ones((G * (N // 128), K // 128), dtype=torch.float32, device="cuda")
    bh = {}
    for g in experts:
        q, s = oracle.quant_e4m3(synth.weights(N, K, seed=300 + g), "block")
        qb[g * N:(g + 1) * N] = torch.from_numpy(q).cuda()
        sb[g * (N // 128):(g + 1) * (N // 128)] = torch.from_numpy(s).cuda()
        bh[g] = oracle.dequant_e4m3(q, s, "block")
    B = fgs.Operand(qb, sb, 2)

    c = torch.full((total, N), 3.0, dtype=torch.bfloat16, device="cuda")
    fgs.grouped_gemm_block_scaled(A, B, torch.from_numpy(offs).cuda(), N, out_dtype=torch.bfloat16, out=c)
    torch.cuda.synchronize()
    got = c[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    group_of = np.searchsorted(offs, rows, side="right") - 1
    for g in experts:
        sel = group_of == g
        cref, sref = oracle.gemm_ref(ah[sel], bh[g])
        ok, nbad = gemm_within_bf16_bound(got[sel], cref, sref)
        assert ok, f"expert {g}: {nbad} BF16 outputs outside one ulp"
    # an unsampled row of a zero-weight expert is exactly zero
    other = int(offs[1])
    assert float(c[other].float().abs().max()) == 0.0


@pytest.mark.parametrize("amode,bmode", [("tile", "block"), ("tile", "tensor"), ("tensor", "block")])
@pytest.mark.parametrize("M,N,K", [(257, 129, 256), (520, 777, 384), (1000, 600, 512)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gemm_promoted_wide_tile(fgs, amode, bmode, M, N, K, out):
    """The promoted modes on the 256 x 256 tile (16x16 output tiles: four
    chained 16x16x32 FP16 MFMAs per scale block, promoted one tile at a time;
    A 1x128 scales staged in LDS), forced on ragged shapes the automatic choice
    would give the 256 x 128 tile: the same bound."""
    A, ah = oracle_operand(fgs, synth.activations(M, K, seed=M + 3 * K), amode)
    B, bh = oracle_operand(fgs, synth.weights(N, K, seed=N + 3 * K), bmode)
    _run_and_check(fgs, A, B, ah, bh, out, tile="wide")


def test_gemm_promoted_wide_tile_adversarial_promotion(fgs):
    """Per-128-K-block A scales spanning 2^-20 .. 2^20 on the 256 x 256
    promoted tile."""
    M, N, K = 128, 256, 1024
    a = oracle.bf16_bits_to_f32(synth.activations(M, K, seed=7, outliers=False)).copy()
    for kb in range(K // 128):
        a[:, kb * 128:(kb + 1) * 128] *= np.float32(2.0 ** (5 * kb - 20))
    A, ah = oracle_operand(fgs, synth.f32_to_bf16_bits(a), "tile")
    B, bh = oracle_operand(fgs, synth.weights(N, K, seed=8), "block")
    _run_and_check(fgs, A, B, ah, bh, torch.float32, tile="wide")
