"""GPU parity of the MoE weight-gradient path: the per-expert transposed
1x128 quantizer (bit-exact against the oracle) and the grouped wgrad GEMM
(|C - C_ref| <= 1e-5 * S + 1e-6 for FP32 out, one BF16 ulp for BF16 out,
C_ref the oracle's FP64 product of the dequantized operands).

"Can you explain the role of FP8 precision in DeepSeek-V3 training",
sections "Mixed precision framework" (expert GEMMs in FP8),
"Fine-grained quantization" (1x128 tiles along the contraction, here each
expert's tokens) and "Increasing accumulation precision" (FP32 promotion per
128-token tile).  Every call goes through the C ABI (the quantizer test calls
it directly with sentinel-filled buffers, so stray or missing writes show).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import _lib, synth

from _helpers import gemm_within_bf16_bound, gemm_within_fp32_bound, sample_rows

pytestmark = pytest.mark.gpu

SENT_CODE = 0xA5
SENT_SCALE = -7.0


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def _blocks_of(offs):
    """(group, first 128-token block, blocks) of every non-empty group."""
    out = []
    for g in range(len(offs) - 1):
        m = int(offs[g + 1] - offs[g])
        if m > 0:
            out.append((g, int(offs[g]) // 128 + g, (m + 127) // 128))
    return out


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _quant_abi(x_bits, offs, rowwise, row_index=None):
    """fgs_quantize_grouped_colwise on sentinel-filled outputs."""
    lib = _lib.load()
    src_rows, C = x_bits.shape
    T = src_rows if row_index is None else len(row_index)
    G = len(offs) - 1
    nb = lib.fgs_grouped_colwise_blocks(T, G)
    assert nb == T // 128 + G
    x = synth.to_torch_bf16(x_bits).cuda()
    off_t = torch.from_numpy(offs).cuda()
    qT = torch.full((C, 128 * nb), SENT_CODE, dtype=torch.uint8, device="cuda")
    sT = torch.full((nb, C), SENT_SCALE, dtype=torch.float32, device="cuda")
    q = s = None
    if rowwise:
        q = torch.full((T, C), SENT_CODE, dtype=torch.uint8, device="cuda")
        s = torch.full((C // 128, T), SENT_SCALE, dtype=torch.float32, device="cuda")
    idx = None if row_index is None else torch.from_numpy(np.asarray(row_index, np.int32)).cuda()
    st = lib.fgs_quantize_grouped_colwise(_ptr(x), T, C, C, _ptr(idx), src_rows, _ptr(off_t), G, _ptr(q), _ptr(s),
                                          _ptr(qT), 128 * nb, _ptr(sT),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(st)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    return cpu(q), cpu(s), cpu(qT), cpu(sT)


def _check_grouped_quant(x_bits, offs, rowwise, row_index=None):
    q, s, qT, sT = _quant_abi(x_bits, offs, rowwise, row_index)
    ref = oracle.quant_e4m3_grouped_colwise(x_bits, offs, row_index=row_index)
    nb = sT.shape[0]
    owned = np.zeros(nb, dtype=bool)
    for g, kb, n in _blocks_of(offs):
        qo, so = ref[g]
        m = qo.shape[1]
        assert np.array_equal(qT[:, 128 * kb:128 * kb + m], qo), f"group {g} codes"
        assert np.array_equal(sT[kb:kb + n].T.view(np.uint32), so.view(np.uint32)), f"group {g} scales"
        # padding of the last tile: code 0, or 0x7F where the tile's scale is NaN
        pad = qT[:, 128 * kb + m:128 * (kb + n)]
        want = np.where(np.isnan(so[:, -1])[:, None], 0x7F, 0).astype(np.uint8)
        assert np.array_equal(pad, np.broadcast_to(want, pad.shape)), f"group {g} padding"
        owned[kb:kb + n] = True
    for b in np.flatnonzero(~owned):
        assert np.all(qT[:, 128 * b:128 * (b + 1)] == SENT_CODE), f"block {b} written"
        assert np.all(sT[b] == SENT_SCALE), f"scales of block {b} written"
    if rowwise:
        rows_bits = x_bits if row_index is None else oracle.gather_rows(x_bits, row_index)
        qr, sr = oracle.quant_e4m3(rows_bits, "tile")
        covered = np.zeros(rows_bits.shape[0], dtype=bool)
        for g in range(len(offs) - 1):
            covered[offs[g]:offs[g + 1]] = True
        assert np.array_equal(q[covered], qr[covered])
        assert np.array_equal(s[:, covered].T.view(np.uint32), sr[covered].view(np.uint32))
        assert np.all(q[~covered] == SENT_CODE) and np.all(s[:, ~covered] == SENT_SCALE)


COUNTS = [0, 1, 130, 0, 257, 128, 3, 200]


@pytest.mark.parametrize("C,rowwise", [(384, True), (200, False)])
def test_grouped_colwise_quant_ragged(C, rowwise):
    offs = _offsets(COUNTS)
    _check_grouped_quant(synth.gradients(int(offs[-1]), C, seed=C), offs, rowwise)


def test_grouped_colwise_quant_special_and_uncovered():
    """A NaN in an expert's partial tile, an Inf in a full one, an all-zero expert (with
    negative zeros), and rows 0..9 and the last 5 rows in no group."""
    counts = [0, 1, 130, 0, 257, 128, 3, 200]
    offs = _offsets(counts) + 10
    offs[0] = 10
    T = int(offs[-1]) + 5
    x = synth.activations(T, 256, seed=4)
    xf = oracle.bf16_bits_to_f32(x).copy()
    xf[offs[2] + 129, 7] = np.nan             # the partial last tile: NaN padding
    xf[offs[4] + 200, 130] = np.inf
    xf[offs[5]:offs[6]] = 0.0
    xf[offs[5]:offs[6]:2, ::3] = -0.0
    _check_grouped_quant(synth.f32_to_bf16_bits(xf), offs.astype(np.int32), rowwise=True)


def test_grouped_colwise_quant_gathered_dispatch():
    """The MoE dispatch gather fused into the read: 300 tokens routed top-3
    to 8 experts (rows sorted by expert), two routed rows with an index
    outside the tokens (zero rows)."""
    tokens, topk, G = 300, 3, 8
    rng = np.random.default_rng(8)
    expert = rng.integers(0, G, (tokens, topk)).ravel()
    expert[expert == 5] = 4                                 # one expert without tokens
    order = np.argsort(expert, kind="stable")
    row_index = (order // topk).astype(np.int32)
    row_index[[7, 500]] = [-1, tokens]
    offs = _offsets(np.bincount(expert, minlength=G))
    _check_grouped_quant(synth.activations(tokens, 384, seed=13), offs, rowwise=True, row_index=row_index)


def test_grouped_colwise_quant_many_groups():
    """300 groups (more than one pass of the workgroup's group search)."""
    counts = synth.expert_counts(tokens=3000, experts=300, seed=2)
    _check_grouped_quant(synth.gradients(int(counts.sum()), 128, seed=9), _offsets(counts), rowwise=False)


# ------------------------------------------------------------- GEMM --------
def _wgrad_case(fgs, counts, M, N, out, seed=0):
    offs = _offsets(counts)
    T = int(offs[-1])
    G = len(counts)
    dy = synth.gradients(T, M, seed=seed)
    x = synth.activations(T, N, seed=seed + 1)
    off_t = torch.from_numpy(offs).cuda()
    qa = fgs.quantize_grouped_colwise(synth.to_torch_bf16(dy).cuda(), off_t)
    qb = fgs.quantize_grouped_colwise(synth.to_torch_bf16(x).cuda(), off_t)
    c = torch.full((G, M, N), 3.0, dtype=out, device="cuda")
    fgs.grouped_wgrad_block_scaled(qa.colwise(), qb.colwise(), off_t, T, out_dtype=out, out=c)
    torch.cuda.synchronize()
    got = c.float().cpu().numpy().astype(np.float64)
    ra = oracle.quant_e4m3_grouped_colwise(dy, offs)
    rb = oracle.quant_e4m3_grouped_colwise(x, offs)
    ah = [oracle.dequant_e4m3(q, s, "tile") for q, s in ra]
    bh = [oracle.dequant_e4m3(q, s, "tile") for q, s in rb]
    cref, sref = oracle.grouped_wgrad_ref(ah, bh)
    for g in range(G):
        if counts[g] == 0:
            assert not got[g].any(), f"empty expert {g} not zero"
    if out == torch.float32:
        ok, worst = gemm_within_fp32_bound(got, cref, sref)
        assert ok, f"worst err/bound = {worst}"
    else:
        ok, nbad = gemm_within_bf16_bound(got, cref, sref)
        assert ok, f"{nbad} BF16 outputs outside one ulp"


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_grouped_wgrad_ragged_and_empty(fgs, out):
    """Ragged experts (1, 3, 130, 200, 257 tokens; two empty), M = 328 (a
    partial 128-row tile), N = 200 (a partial 128-column tile)."""
    _wgrad_case(fgs, COUNTS, M=328, N=200, out=out)


def test_grouped_wgrad_many_groups(fgs):
    counts = synth.expert_counts(tokens=3000, experts=300, seed=3)
    _wgrad_case(fgs, counts, M=128, N=256, out=torch.float32, seed=7)


def test_grouped_wgrad_single_group_is_dense_wgrad(fgs):
    """One expert over 128-aligned tokens: the same tiles, scales and
    accumulation order as the dense wgrad GEMM, so the same bits."""
    T, M, N = 512, 384, 256
    dy = synth.to_torch_bf16(synth.gradients(T, M, seed=11)).cuda()
    x = synth.to_torch_bf16(synth.activations(T, N, seed=12)).cuda()
    off_t = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    qa, qb = fgs.quantize_grouped_colwise(dy, off_t), fgs.quantize_grouped_colwise(x, off_t)
    cg = fgs.grouped_wgrad_block_scaled(qa.colwise(), qb.colwise(), off_t, T)
    da = fgs.quantize_blockwise(dy, "tile", rowwise=False, colwise=True)
    db = fgs.quantize_blockwise(x, "tile", rowwise=False, colwise=True)
    cd = fgs.gemm_block_scaled(da.colwise(), db.colwise(), torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(cg[0].view(torch.int32), cd.view(torch.int32))


# ------------------------------------------------- full-size MoE (sampled) --
@pytest.mark.parametrize("M,N,out", [(4096, 7168, torch.bfloat16), (7168, 2048, torch.float32)],
                         ids=["gate_up", "down"])
def test_grouped_wgrad_deepseek_moe_sampled(fgs, M, N, out):
    """DeepSeek-V3 MoE weight gradients at full size: 256 experts over 32768
    routed rows with seeded Zipf(1.1) counts (one expert made empty);
    gate/up dW_g [4096 x 7168] = dY_g^T X_g (BF16 out) and down dW_g
    [7168 x 2048] (FP32 out).  The GPU quantizes the whole dY and X; the
    oracle quantizes the sampled columns (1x128 tiles run along the tokens,
    so columns are independent) of the sampled experts, and the sampled
    outputs of those experts are checked, plus the empty expert in full."""
    G = 256
    counts = synth.expert_counts(32768, G, 1.1, seed=0).copy()
    empty = 100
    counts[0] += counts[empty]
    counts[empty] = 0
    offs = _offsets(counts)
    T = int(offs[-1])
    mid = int(np.flatnonzero((counts > 128) & (counts < 256))[0])
    small = int(np.flatnonzero((counts > 0) & (counts < 16))[0])
    dy = synth.gradients(T, M, seed=31)
    x = synth.activations(T, N, seed=32)
    off_t = torch.from_numpy(offs).cuda()
    qa = fgs.quantize_grouped_colwise(synth.to_torch_bf16(dy).cuda(), off_t)
    qb = fgs.quantize_grouped_colwise(synth.to_torch_bf16(x).cuda(), off_t)
    c = torch.full((G, M, N), 3.0, dtype=out, device="cuda")
    fgs.grouped_wgrad_block_scaled(qa.colwise(), qb.colwise(), off_t, T, out_dtype=out, out=c)
    torch.cuda.synchronize()
    assert float(c[empty].float().abs().max()) == 0.0
    rs, cs = sample_rows(M, seed=1), sample_rows(N, seed=2)
    rs_t, cs_t = torch.from_numpy(rs).cuda(), torch.from_numpy(cs).cuda()
    for g in (0, mid, small):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        kb = r0 // 128 + g
        qo_a, so_a = oracle.quant_e4m3_grouped_colwise(dy[:, rs], [r0, r1])[0]
        qo_b, so_b = oracle.quant_e4m3_grouped_colwise(x[:, cs], [r0, r1])[0]
        m = r1 - r0
        assert np.array_equal(qa.qT[rs_t, 128 * kb:128 * kb + m].cpu().numpy(), qo_a), f"expert {g} dY codes"
        assert np.array_equal(qb.qT[cs_t, 128 * kb:128 * kb + m].cpu().numpy(), qo_b), f"expert {g} X codes"
        ah = oracle.dequant_e4m3(qo_a, so_a, "tile")
        bh = oracle.dequant_e4m3(qo_b, so_b, "tile")
        cref, sref = oracle.gemm_ref(ah, bh)
        got = c[g][rs_t][:, cs_t].float().cpu().numpy().astype(np.float64)
        if out == torch.float32:
            ok, worst = gemm_within_fp32_bound(got, cref, sref)
            assert ok, f"expert {g}: worst err/bound = {worst}"
        else:
            ok, nbad = gemm_within_bf16_bound(got, cref, sref)
            assert ok, f"expert {g}: {nbad} BF16 outputs outside one ulp"


# ------------------------------------------- offsets out of order or range --
def test_invalid_offsets_stay_in_bounds(fgs):
    """Offsets that decrease or leave [0, T]: groups with such bounds are
    empty (no codes; dW = 0), overlapping valid groups give unspecified
    values, and no write lands outside the buffers (guard bytes around each
    output stay as filled)."""
    lib = _lib.load()
    T, C, M = 719, 256, 256
    offs = np.array([0, 500, 100, 719, 600, 719, 800], dtype=np.int32)   # groups 1, 3 decrease; 5 leaves [0, T]
    G = len(offs) - 1
    nb = T // 128 + G
    x = synth.to_torch_bf16(synth.activations(T, C, seed=81)).cuda()
    off_t = torch.from_numpy(offs).cuda()
    guard = 4096
    qbuf = torch.full((C * 128 * nb + 2 * guard,), SENT_CODE, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((nb * C + 2 * guard,), SENT_SCALE, dtype=torch.float32, device="cuda")
    qT = qbuf[guard:guard + C * 128 * nb]
    sT = sbuf[guard:guard + nb * C]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    _lib.check(lib.fgs_quantize_grouped_colwise(_ptr(x), T, C, C, None, 0, _ptr(off_t), G, None, None,
                                                _ptr(qT), 128 * nb, _ptr(sT), stream))
    torch.cuda.synchronize()
    q = qbuf.cpu().numpy()
    s = sbuf.cpu().numpy()
    assert np.all(q[:guard] == SENT_CODE) and np.all(q[-guard:] == SENT_CODE)
    assert np.all(s[:guard] == SENT_SCALE) and np.all(s[-guard:] == SENT_SCALE)
    # group 4 ([600, 719)) alone owns block 600 // 128 + 4 = 8: exact codes there
    qo, so = oracle.quant_e4m3_grouped_colwise(synth.activations(T, C, seed=81), [600, 719])[0]
    qmat = q[guard:guard + C * 128 * nb].reshape(C, 128 * nb)
    assert np.array_equal(qmat[:, 128 * 8:128 * 8 + 119], qo)

    # the wgrad GEMM over the same offsets: empty groups exactly zero, no stray writes
    qa = fgs.quantize_grouped_colwise(synth.to_torch_bf16(synth.gradients(T, M, seed=82)).cuda(), off_t)
    qb = fgs.Operand(qT.view(C, 128 * nb), sT.view(nb, C), fgs.SCALE_TILE_1x128)
    cbuf = torch.full((G * M * C + 2 * guard,), 3.0, dtype=torch.float32, device="cuda")
    c = cbuf[guard:guard + G * M * C].view(G, M, C)
    fgs.grouped_wgrad_block_scaled(qa.colwise(), qb, off_t, T, torch.float32, out=c)
    torch.cuda.synchronize()
    cb = cbuf.cpu().numpy()
    assert np.all(cb[:guard] == 3.0) and np.all(cb[-guard:] == 3.0)
    cc = cb[guard:guard + G * M * C].reshape(G, M, C)
    for g in (1, 3, 5):
        assert not cc[g].any(), g
    assert np.all(np.isfinite(cc))


# --------------------------------------------- SwiGLU fused into the quant --
def _bf16_adjacent(a_bits, b_bits):
    """Equal or neighbouring BF16 numbers (ordered bit patterns)."""
    def key(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(a_bits) - key(b_bits)) <= 1


def _check_swiglu(fgs, gu_bits, offs, rowwise, sample_cols=None):
    inter = gu_bits.shape[1] // 2
    off_t = torch.from_numpy(offs).cuda()
    qq, h = fgs.swiglu_quantize_grouped(synth.to_torch_bf16(gu_bits).cuda(), off_t, rowwise=rowwise,
                                        colwise=True, return_h=True)
    torch.cuda.synchronize()
    T = gu_bits.shape[0]
    covered = np.zeros(T, dtype=bool)
    for g in range(len(offs) - 1):
        covered[offs[g]:offs[g + 1]] = True
    hb = h.cpu().view(torch.int16).numpy().view(np.uint16)
    # the activation: within one BF16 step of the exactly rounded SwiGLU
    ref = oracle.swiglu_bf16(gu_bits, inter)
    adj = _bf16_adjacent(hb[covered], ref[covered])
    assert adj.all(), f"{int((~adj).sum())} activations off by more than one BF16 step"
    # the codes: exactly the oracle's quantization of that activation
    cols = np.arange(inter) if sample_cols is None else sample_cols
    hsel = np.ascontiguousarray(hb[:, cols])
    res = oracle.quant_e4m3_grouped_colwise(hsel, offs)
    qT = qq.qT[torch.from_numpy(cols).cuda()].cpu().numpy()
    sT = qq.scalesT[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    for g, kb, n in _blocks_of(offs):
        qo, so = res[g]
        assert np.array_equal(qT[:, 128 * kb:128 * kb + qo.shape[1]], qo), g
        assert np.array_equal(sT[kb:kb + n].T.view(np.uint32), so.view(np.uint32)), g
    if rowwise:
        qr, sr = oracle.quant_e4m3(hb, "tile")
        assert np.array_equal(qq.q.cpu().numpy()[covered], qr[covered])
        assert np.array_equal(qq.scales.cpu().numpy()[:, covered].T.view(np.uint32), sr[covered].view(np.uint32))


@pytest.mark.parametrize("inter,rowwise", [(256, True), (200, False)])
def test_swiglu_quantize_ragged(fgs, inter, rowwise):
    """Gate/up outputs with x50 outlier channels (|g| up to ~200, both tails
    of the logistic), ragged and empty experts."""
    offs = _offsets(COUNTS)
    _check_swiglu(fgs, synth.activations(int(offs[-1]), 2 * inter, seed=inter), offs, rowwise)


def test_swiglu_quantize_deepseek_moe_sampled(fgs):
    """DeepSeek-V3 down-projection input at full size: 32768 routed rows of
    the gate/up output [x 4096], 256 Zipf experts; every activation checked,
    the codes on sampled columns."""
    counts = synth.expert_counts(32768, 256, 1.1, seed=0)
    offs = _offsets(counts)
    gu = synth.activations(int(offs[-1]), 2 * 2048, seed=91)
    _check_swiglu(fgs, gu, offs, rowwise=True, sample_cols=sample_rows(2048, seed=3))
