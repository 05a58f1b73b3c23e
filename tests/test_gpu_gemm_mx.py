"""GPU parity of the MXFP8 GEMM (E4M3 codes with one E8M0 scale per 32
K-elements on both operands) against the oracle's FP64 product of the
dequantized operands: |C - C_ref| <= 1e-5 * sum_k |a_k b_k| + 1e-6 (FP32
out), within one BF16 ulp of the rounded reference (BF16 out).

"Accelerating FP8 training performance with the NVIDIA NeMo framework":
MXFP8 with blocks of 32 values.  Operands are quantized by the oracle and
uploaded, so this isolates the GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import gemm_within_bf16_bound, gemm_within_fp32_bound, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def mx_operand(fgs, bits, colwise=False, rows=None):
    q, s = oracle.quant_mx(bits, colwise=colwise)
    deq = oracle.dequant_mx(q if rows is None else q[rows], s if rows is None else s[rows])
    op = fgs.Operand(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), fgs.SCALE_MX32_E8M0)
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


@pytest.mark.parametrize("M,N,K", [(200, 130, 384), (1, 1, 128), (257, 129, 256), (256, 384, 1024)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_mx_gemm_ragged(fgs, M, N, K, out):
    A, ah = mx_operand(fgs, synth.activations(M, K, seed=M + 3, outliers=False))
    B, bh = mx_operand(fgs, synth.weights(N, K, seed=N + 5))
    _check(fgs, A, B, ah, bh, out)


@pytest.mark.parametrize("M,N,K", [(200, 130, 384), (300, 520, 1024), (256, 264, 4096), (130, 600, 16896)])
@pytest.mark.parametrize("tile", ["narrow", "wide"])
def test_mx_gemm_workspace_same_bits(fgs, M, N, K, tile):
    """With a workspace the rows' reference exponents come from a pass of
    their own; without one every tile scans its rows' scale bytes (4 bytes
    at a time for K = 384, 16 at a time from K = 512 on, in batches of 8
    from K = 4096).  Both give the same references, so the same bits, here
    with a NaN scale byte planted in one A row and one B row; the result is
    checked against the oracle too."""
    a_bits = synth.activations(M, K, seed=M + 40, outliers=False)
    b_bits = synth.weights(N, K, seed=N + 41)
    qa, sa = oracle.quant_mx(a_bits)
    qb, sb = oracle.quant_mx(b_bits)
    sa[M // 3, K // 64] = 0xFF
    sb[N - 2, 1] = 0xFF
    A = fgs.Operand(torch.from_numpy(qa).cuda(), torch.from_numpy(sa).cuda(), fgs.SCALE_MX32_E8M0)
    B = fgs.Operand(torch.from_numpy(qb).cuda(), torch.from_numpy(sb).cuda(), fgs.SCALE_MX32_E8M0)
    c_ws = fgs.gemm_block_scaled(A, B, torch.float32, tile=tile)
    c_scan = fgs.gemm_block_scaled(A, B, torch.float32, tile=tile, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(c_ws.view(torch.int32), c_scan.view(torch.int32))
    c = c_ws.cpu().numpy().astype(np.float64)
    assert np.isnan(c[M // 3]).all() and np.isnan(c[:, N - 2]).all()
    keep_r = np.setdiff1d(np.arange(M), [M // 3])
    keep_c = np.setdiff1d(np.arange(N), [N - 2])
    ah = oracle.dequant_mx(qa[keep_r], sa[keep_r])
    bh = oracle.dequant_mx(qb[keep_c], sb[keep_c])
    cref, sref = oracle.gemm_ref(ah, bh)
    ok, worst = gemm_within_fp32_bound(c[np.ix_(keep_r, keep_c)], cref, sref)
    assert ok, f"worst err/bound = {worst}"


def test_mx_gemm_exponent_spread(fgs):
    """Every 32-block of both operands scaled by its own power of two in
    2^-40 .. 2^40, so the E8M0 exponents inside one 128-K block and across
    the rows of a tile differ widely: exercises the per-row (A) and per-tile
    (B) reference exponents and the promotion factor."""
    M, N, K = 256, 256, 512
    rng = np.random.default_rng(21)
    a = oracle.bf16_bits_to_f32(synth.activations(M, K, seed=22, outliers=False)).copy()
    b = oracle.bf16_bits_to_f32(synth.weights(N, K, seed=23)).copy()
    a *= np.repeat(np.ldexp(1.0, rng.integers(-40, 41, (M, K // 32))), 32, axis=1).astype(np.float32)
    b *= np.repeat(np.ldexp(1.0, rng.integers(-40, 41, (N, K // 32))), 32, axis=1).astype(np.float32)
    A, ah = mx_operand(fgs, synth.f32_to_bf16_bits(a))
    B, bh = mx_operand(fgs, synth.f32_to_bf16_bits(b))
    _check(fgs, A, B, ah, bh, torch.float32)


def _spread_operands(fgs, da, db, E=200, seed=41):
    """A [64 x 256] and B [96 x 256] MX operands whose only pair of nonzero
    blocks that meet is block 1.  Block 0 carries both references (scale
    byte E): A's has codes, B's is all zeros, so it adds nothing.  Block 1's
    scale byte lies da (A) and db (B) below E; its codes are positive (no
    cancellation) and include the smallest subnormal E4M3 codes, so the
    products reach down to 2^-18 2^(da+db) of the reference unit
    2^(2E - 254).  Blocks 2-7 are zero."""
    rng = np.random.default_rng(seed)
    M, N, K = 64, 96, 256
    small = np.concatenate([np.arange(1, 16), rng.integers(1, 0x7F, 17)]).astype(np.uint8)

    def operand(rows, d, ref_codes):
        q = np.zeros((rows, K), dtype=np.uint8)
        s = np.full((rows, K // 32), 127, dtype=np.uint8)
        s[:, 0] = E
        if ref_codes:
            q[:, 0:32] = rng.integers(0x08, 0x7F, (rows, 32))
        s[:, 1] = E + d
        q[:, 32:64] = rng.permuted(np.tile(small, (rows, 1)), axis=1)
        return q, s

    qa, sa = operand(M, da, True)     # A block 0: the reference, meets B's zeros
    qb, sb = operand(N, db, False)    # B block 0: the reference scale, zero codes
    A = fgs.Operand(torch.from_numpy(qa).cuda(), torch.from_numpy(sa).cuda(), fgs.SCALE_MX32_E8M0)
    B = fgs.Operand(torch.from_numpy(qb).cuda(), torch.from_numpy(sb).cuda(), fgs.SCALE_MX32_E8M0)
    return A, B, oracle.dequant_mx(qa, sa), oracle.dequant_mx(qb, sb)


@pytest.mark.parametrize("da,db", [(-54, -54), (-100, -8), (0, -108)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_mx_gemm_exponent_limit(fgs, da, db, out):
    """At the exactness limit of the MX decode: block pairs whose exponents
    lie da + db = -108 below the references (A: the row over all of K; B:
    the tile's rows over all of K) decode to BF16 numbers and multiply to
    normal FP32 numbers (the smallest, 2^-9 * 2^-9 * 2^-108 = 2^-126, is
    reached), so the outputs, made of those products only, meet the
    standard bound."""
    A, B, ah, bh = _spread_operands(fgs, da, db)
    _check(fgs, A, B, ah, bh, out)


@pytest.mark.parametrize("da,db", [(-60, -60), (-130, 0), (-200, -40)])
def test_mx_gemm_beyond_exponent_limit(fgs, da, db):
    """Past the limit (da + db < -108, or a block more than 127 below its
    reference, where the converter's power-of-two scale saturates at
    2^-127): each such product of two codes is below 448^2 2^-108 < 2^-90
    reference units, and what the kernel adds for it (rounded, flushed or
    saturated) stays below 2^-90 units too, so every output is finite and
    within the standard bound plus 32 2^-90 units per meeting block pair."""
    A, B, ah, bh = _spread_operands(fgs, da, db)
    c = fgs.gemm_block_scaled(A, B, torch.float32)
    torch.cuda.synchronize()
    c = c.cpu().numpy().astype(np.float64)
    cref, sref = oracle.gemm_ref(ah, bh)
    unit = 2.0 ** (2 * 200 - 254)
    assert np.all(np.isfinite(c))
    assert np.all(np.abs(c - cref) <= 1e-5 * sref + 1e-6 + 32 * 2.0 ** -90 * unit)


def test_mx_gemm_zero_and_tiny_blocks(fgs):
    """All-zero 32-blocks (scale byte 127) next to blocks of tiny values."""
    M, N, K = 128, 128, 256
    a = oracle.bf16_bits_to_f32(synth.activations(M, K, seed=24, outliers=False)).copy()
    b = oracle.bf16_bits_to_f32(synth.weights(N, K, seed=25)).copy()
    a[:, 0:32] = 0.0
    a[::3, 32:64] *= np.float32(2.0 ** -30)
    b[::2, 64:96] = 0.0
    b[1::5, 96:128] *= np.float32(2.0 ** -25)
    A, ah = mx_operand(fgs, synth.f32_to_bf16_bits(a))
    B, bh = mx_operand(fgs, synth.f32_to_bf16_bits(b))
    _check(fgs, A, B, ah, bh, torch.float32)


@pytest.mark.parametrize("policy", ["narrow", "wide"])
def test_mx_gemm_nan_blocks(fgs, policy):
    """A NaN in one 32-block of an A row and of a B row gives that block the
    NaN scale byte 0xFF: exactly that row and that column of C are NaN (as in
    the dequantized product), every other output meets the bound."""
    M, N, K = 300, 260, 512
    a = oracle.bf16_bits_to_f32(synth.activations(M, K, seed=28, outliers=False)).copy()
    b = oracle.bf16_bits_to_f32(synth.weights(N, K, seed=29)).copy()
    a[7, 70] = np.nan
    b[131, 300] = np.nan
    A, ah = mx_operand(fgs, synth.f32_to_bf16_bits(a))
    B, bh = mx_operand(fgs, synth.f32_to_bf16_bits(b))
    c = fgs.gemm_block_scaled(A, B, torch.float32, tile=policy)
    torch.cuda.synchronize()
    c = c.cpu().numpy().astype(np.float64)
    cref, sref = oracle.gemm_ref(ah, bh)
    assert np.array_equal(np.isnan(c), np.isnan(cref))
    assert np.isnan(c[7]).all() and np.isnan(c[:, 131]).all()
    ok = ~np.isnan(cref)
    good, worst = gemm_within_fp32_bound(c[ok], cref[ok], sref[ok])
    assert good, worst


@pytest.mark.parametrize("policy", ["narrow", "wide"])
def test_mx_gemm_tile_policies(fgs, policy):
    """The MX GEMM on either workgroup tile, ragged shapes, both outputs."""
    M, N, K = 520, 777, 384
    A, ah = mx_operand(fgs, synth.activations(M, K, seed=30, outliers=False))
    B, bh = mx_operand(fgs, synth.weights(N, K, seed=31))
    _check(fgs, A, B, ah, bh, torch.float32, tile=policy)
    _check(fgs, A, B, ah, bh, torch.bfloat16, tile=policy)


def test_mx_gemm_determinism(fgs):
    A, _ = mx_operand(fgs, synth.activations(512, 1024, seed=26, outliers=False))
    B, _ = mx_operand(fgs, synth.weights(384, 1024, seed=27))
    c1 = fgs.gemm_block_scaled(A, B)
    c2 = fgs.gemm_block_scaled(A, B)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("orient", ["fwd", "wgrad"])
def test_mx_llama405b_qkv_sampled(fgs, orient):
    """Llama-3.1-405B QKV projection, one GPU's share: M = 4096 tokens,
    (K, N) = (16384, 18432); fwd in BF16 out, wgrad (contraction over the
    4096 tokens, both operands MX-quantized along M) in FP32; sampled rows."""
    M, K, N = 4096, 16384, 18432
    if orient == "fwd":
        a_bits = synth.activations(M, K, seed=0, outliers=False)
        b_bits = synth.weights(N, K, seed=0)
        a_col = b_col = False
        out = torch.bfloat16
    else:
        a_bits = synth.normal_gradients(M, N, seed=0)       # dY [M x N] -> dY^T [N x M]
        b_bits = synth.activations(M, K, seed=0, outliers=False)   # X -> X^T [K x M]
        a_col = b_col = True
        out = torch.float32
    rows_total = a_bits.shape[1] if a_col else a_bits.shape[0]
    rs = sample_rows(rows_total)
    A, ah = mx_operand(fgs, a_bits, colwise=a_col, rows=rs)
    B, bh = mx_operand(fgs, b_bits, colwise=b_col)
    _check(fgs, A, B, ah, bh, out, rows=rs)
