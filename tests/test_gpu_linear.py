"""The autograd Linear layer over the library's kernels: its forward,
dgrad and wgrad products match the oracle on the oracle's quantization of
the same BF16 operands (per recipe), and a toy teacher-student regression
trains under every recipe to a loss close to the FP32 one.

"Accelerating FP8 training performance with the NVIDIA NeMo framework"
compares per-tensor and block-wise scaling in training; "Can you explain
the role of FP8 precision in DeepSeek-V3 training" ("Fine-grained
quantization", "Online quantization", "Unified E4M3 format") gives the
block-wise recipe and names the delayed / hybrid one it replaces.
"""
import numpy as np
import pytest
import torch

import oracle
from fine_grained_scaled_amd import synth

from _helpers import gemm_within_bf16_bound, gemm_within_fp32_bound

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module")
def fgs():
    import fine_grained_scaled_amd as m
    return m


def _bits(t):
    return t.detach().to(torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)


def _deq(bits, recipe, role, colwise, hist):
    if recipe == "delayed":
        q, s, _ = oracle.quant_delayed(bits, "e5m2" if role == "dy" else "e4m3", hist, colwise=colwise)
        return oracle.dequant_tensor(q, s, "e5m2" if role == "dy" else "e4m3")
    mode = "tensor" if recipe == "per_tensor" else ("block" if role == "w" else "tile")
    q, s = oracle.quant_e4m3(bits, mode, colwise=colwise)
    return oracle.dequant_e4m3(q, s, mode)


def _amax(bits):
    return F32(np.abs(oracle.bf16_bits_to_f32(bits)).max())


@pytest.mark.parametrize("recipe", ["blockwise", "per_tensor", "delayed"])
def test_linear_products_match_oracle(fgs, recipe):
    """Two steps (the second reads the delayed histories the first wrote):
    Y (BF16), dX (BF16) and dW (FP32) of the second step against the oracle."""
    T, K, N = 256, 384, 256
    layer = fgs.Linear(K, N, recipe=recipe, device="cuda")
    hist = {"x": np.zeros(16, F32), "w": np.zeros(16, F32), "dy": np.zeros(16, F32)}
    for step in range(2):
        x = synth.to_torch_bf16(synth.activations(T, K, seed=10 + step)).cuda().requires_grad_(True)
        dy = synth.to_torch_bf16(synth.gradients(T, N, seed=20 + step)).cuda()
        y = layer(x)
        y.backward(dy)
        torch.cuda.synchronize()
        xb, wb, dyb = _bits(x), _bits(layer.weight), _bits(dy)
        if step == 1:
            yr, ys = oracle.gemm_ref(_deq(xb, recipe, "x", False, hist["x"]), _deq(wb, recipe, "w", False, hist["w"]))
            ok, nbad = gemm_within_bf16_bound(y.detach().float().cpu().numpy(), yr, ys)
            assert ok, f"Y: {nbad} outside one BF16 ulp"
            dxr, dxs = oracle.gemm_ref(_deq(dyb, recipe, "dy", False, hist["dy"]),
                                       _deq(wb, recipe, "w", True, hist["w"]))
            ok, nbad = gemm_within_bf16_bound(x.grad.float().cpu().numpy(), dxr, dxs)
            assert ok, f"dX: {nbad} outside one BF16 ulp"
            dwr, dws = oracle.gemm_ref(_deq(dyb, recipe, "dy", True, hist["dy"]),
                                       _deq(xb, recipe, "x", True, hist["x"]))
            ok, worst = gemm_within_fp32_bound(layer.weight.grad.cpu().numpy().astype(np.float64), dwr, dws)
            assert ok, f"dW: worst err/bound {worst}"
            assert layer.weight.grad.dtype == torch.float32
        for k, b in (("x", xb), ("w", wb), ("dy", dyb)):
            hist[k][step] = _amax(b)
        layer.weight.grad = None


def test_linear_rejects_unaligned_shapes(fgs):
    layer = fgs.Linear(256, 256, device="cuda")
    with pytest.raises(ValueError):
        layer(torch.zeros((100, 256), dtype=torch.bfloat16, device="cuda"))


class _BF16Linear(torch.autograd.Function):
    """The BF16 baseline layer: y = x W^T with BF16 operands and products
    (hipBLASLt through torch), FP32 weight gradient.  Every product takes
    contiguous operands (no transposed views)."""

    @staticmethod
    def forward(ctx, x, w):
        xb, wb = x.to(torch.bfloat16).contiguous(), w.to(torch.bfloat16).contiguous()
        ctx.save_for_backward(xb, wb)
        return xb @ wb.t().contiguous()

    @staticmethod
    def backward(ctx, dy):
        xb, wb = ctx.saved_tensors
        dyb = dy.to(torch.bfloat16).contiguous()
        return dyb @ wb, (dyb.t().contiguous() @ xb).float()


class _BF16Layer(torch.nn.Module):
    def __init__(self, d_in, d_out):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.randn(d_out, d_in, device="cuda") * d_in ** -0.5)

    def forward(self, x):
        return _BF16Linear.apply(x, self.weight)


def _train(fgs, recipe, steps=120, T=1024, D=256, H=512, seed=0, fp8_mma=False, outlier=0.0, frac=0.01):
    """Student MLP D -> H -> D (GELU) regressing a fixed random teacher on
    Gaussian inputs; Adam, MSE.  recipe "fp32" / "bf16": torch layers in that
    precision; else the library's Linear.  outlier > 0: in every batch a
    random `frac` of the tokens is scaled by `outlier` (outlier tokens), and
    the loss is taken over the other tokens only."""
    torch.manual_seed(seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    t1 = torch.randn(H, D, device="cuda", generator=g) * D ** -0.5
    t2 = torch.randn(D, H, device="cuda", generator=g) * H ** -0.5
    if recipe == "fp32":
        l1 = torch.nn.Linear(D, H, bias=False, device="cuda")
        l2 = torch.nn.Linear(H, D, bias=False, device="cuda")
        torch.nn.init.normal_(l1.weight, std=D ** -0.5)
        torch.nn.init.normal_(l2.weight, std=H ** -0.5)
    elif recipe == "bf16":
        l1, l2 = _BF16Layer(D, H), _BF16Layer(H, D)
    else:
        l1 = fgs.Linear(D, H, recipe=recipe, device="cuda", fp8_mma=fp8_mma)
        l2 = fgs.Linear(H, D, recipe=recipe, device="cuda", fp8_mma=fp8_mma)
    opt = torch.optim.Adam(list(l1.parameters()) + list(l2.parameters()), lr=2e-3)
    mask = torch.ones(T, 1, device="cuda")
    n_out = int(round(frac * T))
    losses = []
    for s in range(steps):
        x = torch.randn(T, D, device="cuda", generator=g)
        if outlier:
            idx = torch.randperm(T, device="cuda", generator=g)[:n_out]
            x[idx] *= outlier
            mask.fill_(1.0)
            mask[idx] = 0.0
        with torch.no_grad():
            target = torch.nn.functional.gelu(x @ t1.t().contiguous()) @ t2.t().contiguous()
        h = torch.nn.functional.gelu(l1(x).float())
        out = l2(h).float()
        loss = torch.sum(((out - target) * mask) ** 2) / (mask.sum() * D)
        opt.zero_grad()
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    return np.array(losses)


def _tail(a):
    return float(a[-10:].mean())


def test_toy_training_tracks_bf16(fgs):
    """On plain Gaussian data every recipe learns (the loss falls by 4x in
    120 steps) and ends within 3% of the BF16 run's final loss (mean of the
    last 10 steps; measured: within 0.4%); so does the blockwise recipe with
    its products on the FP8 matrix instructions.  The FP32 run is printed
    for reference."""
    ref = _train(fgs, "bf16")
    fp32 = _train(fgs, "fp32")
    print(f"bf16: first {ref[0]:.4f} last-10 {_tail(ref):.4f}; fp32 last-10 {_tail(fp32):.4f}")
    assert _tail(ref) < ref[0] / 4
    for recipe, mma in (("blockwise", False), ("per_tensor", False), ("delayed", False), ("blockwise", True)):
        got = _train(fgs, recipe, fp8_mma=mma)
        name = recipe + (" on FP8 instructions" if mma else "")
        print(f"{name}: first {got[0]:.4f} last-10 {_tail(got):.4f}")
        assert np.all(np.isfinite(got)), name
        assert _tail(got) < got[0] / 4, (name, got[0], _tail(got))
        assert abs(_tail(got) - _tail(ref)) < 0.03 * _tail(ref), (name, _tail(got), _tail(ref))


def test_toy_training_outlier_tokens_blockwise_vs_per_tensor(fgs):
    """The pages' comparison of the recipes ("Accelerating FP8 training
    performance with the NVIDIA NeMo framework": block-wise scaling tracks
    BF16 closely, per-tensor scaling less so; "Can you explain the role of
    FP8 precision in DeepSeek-V3 training", "Fine-grained quantization": the
    small groups keep outliers from spoiling the other values' scale), at
    toy scale: with 1% of the tokens scaled by 3e4, one per-tensor scale
    pushes the other tokens' activations towards E4M3's subnormals while each
    token's 1x128 tiles keep their own scale.  Blockwise ends within 2% of
    BF16 (measured 0.3%); per-tensor current and delayed scaling end at least
    8% above blockwise (measured 18% and 19%)."""
    ref = _train(fgs, "bf16", outlier=3e4)
    blk = _train(fgs, "blockwise", outlier=3e4)
    print(f"outlier tokens x3e4: bf16 last-10 {_tail(ref):.4f}, blockwise {_tail(blk):.4f}")
    assert abs(_tail(blk) - _tail(ref)) < 0.02 * _tail(ref)
    for recipe in ("per_tensor", "delayed"):
        got = _train(fgs, recipe, outlier=3e4)
        print(f"outlier tokens x3e4: {recipe} last-10 {_tail(got):.4f}")
        assert np.all(np.isfinite(got)), recipe
        assert _tail(got) > 1.08 * _tail(blk), (recipe, _tail(got), _tail(blk))


def test_linear_fp8_mma_products_within_derived_bound(fgs):
    """The layer with fp8_mma=True: Y, dX and dW against the oracle's
    blockwise products within the FP8-instruction bound 2^-9 * S + 1e-6
    (plus one BF16 ulp for the BF16 outputs)."""
    from _helpers import _bf16_ulp
    T, K, N = 256, 384, 256
    layer = fgs.Linear(K, N, recipe="blockwise", device="cuda", fp8_mma=True)
    x = synth.to_torch_bf16(synth.activations(T, K, seed=30)).cuda().requires_grad_(True)
    dy = synth.to_torch_bf16(synth.gradients(T, N, seed=31)).cuda()
    y = layer(x)
    y.backward(dy)
    torch.cuda.synchronize()
    xb, wb, dyb = _bits(x), _bits(layer.weight), _bits(dy)
    none = np.zeros(16, F32)
    cases = [(y.detach(), _deq(xb, "blockwise", "x", False, none), _deq(wb, "blockwise", "w", False, none), True),
             (x.grad, _deq(dyb, "blockwise", "dy", False, none), _deq(wb, "blockwise", "w", True, none), True),
             (layer.weight.grad, _deq(dyb, "blockwise", "dy", True, none), _deq(xb, "blockwise", "x", True, none), False)]
    for got, a, b, bf16 in cases:
        cref, sref = oracle.gemm_ref(a, b)
        err = np.abs(got.float().cpu().numpy().astype(np.float64) - cref)
        bound = 2.0 ** -9 * sref + 1e-6 + (_bf16_ulp(cref) if bf16 else 0.0)
        assert np.all(err <= bound)
