"""The allocation-free entry point fgs_quantize_blockwise_noalloc (for
callers that cannot allocate device memory), called through the C ABI,
gives bit for bit what fgs_quantize_blockwise gives with a caller-owned
workspace: codes and scales of both outputs, in every mode, on two calls in
a row.  The first call quantizes a large tensor with a large amax (its amax
pass fills many scratch slots); the second a smaller one with a small amax,
whose amax pass runs far fewer workgroups: a cast pass that read a slot the
second call did not write would take the first tensor's amax and give a
different scale.  ("Can you explain the role of FP8 precision in
DeepSeek-V3 training", "Fine-grained quantization", "Online quantization";
"Accelerating FP8 training performance with the NVIDIA NeMo framework",
per-tensor current scaling.)"""
import ctypes

import pytest
import torch

from fine_grained_scaled_amd import _lib, synth

pytestmark = pytest.mark.gpu

MODES = {"tensor": _lib.SCALE_TENSOR, "tile": _lib.SCALE_TILE_1x128, "block": _lib.SCALE_BLOCK_128x128}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _outputs(rows, cols, mode):
    dev = "cuda"
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    if mode == "tile":
        s = torch.empty(((cols + 127) // 128, rows), dtype=torch.float32, device=dev)
        sT = torch.empty(((rows + 127) // 128, cols), dtype=torch.float32, device=dev)
    elif mode == "block":
        s = torch.empty(((rows + 127) // 128, (cols + 127) // 128), dtype=torch.float32, device=dev)
        sT = torch.empty(((cols + 127) // 128, (rows + 127) // 128), dtype=torch.float32, device=dev)
    else:
        s = torch.empty(1, dtype=torch.float32, device=dev)
        sT = torch.empty(1, dtype=torch.float32, device=dev)
    return q, s, qT, sT


def _noalloc(x, mode):
    rows, cols = x.shape
    q, s, qT, sT = _outputs(rows, cols, mode)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    _lib.check(_lib.load().fgs_quantize_blockwise_noalloc(
        _ptr(x), rows, cols, x.stride(0), MODES[mode], _ptr(q), _ptr(s), _ptr(qT), _ptr(sT), stream))
    return q, s, qT, sT


def _with_workspace(x, mode):
    rows, cols = x.shape
    q, s, qT, sT = _outputs(rows, cols, mode)
    lib = _lib.load()
    ws = torch.empty(lib.fgs_workspace_bytes(rows, cols), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    _lib.check(lib.fgs_quantize_blockwise(_ptr(x), rows, cols, x.stride(0), MODES[mode], _ptr(q), _ptr(s),
                                          _ptr(qT), _ptr(sT), _ptr(ws), ws.numel(), stream))
    return q, s, qT, sT


@pytest.mark.parametrize("mode", ["tensor", "tile", "block"])
def test_noalloc_equals_workspace_entry_point_on_two_calls(mode):
    for rows, cols, gain, seed in ((8192, 4096, 64.0, 11), (384, 256, 1.0, 12)):
        x = synth.to_torch_bf16(synth.activations(rows, cols, seed=seed)).cuda()
        if gain != 1.0:
            x *= gain                          # exact: a power of two
        got = _noalloc(x, mode)
        ref = _with_workspace(x, mode)
        torch.cuda.synchronize()
        for name, g, r in zip(("q", "scales", "qT", "scalesT"), got, ref):
            if g.dtype == torch.float32:
                g, r = g.view(torch.int32), r.view(torch.int32)
            assert torch.equal(g, r), f"{mode} {rows}x{cols}: {name} differs"
        if mode == "tensor":
            # the scale is this tensor's own: fl32(amax / 448)
            amax = x.float().abs().max().cpu()
            assert float(got[1][0].cpu()) == float(amax / 448.0)      # IEEE FP32 division on the host


def test_noalloc_validation_before_any_hip_call():
    """Argument errors are returned before the scratch is resolved."""
    lib = _lib.load()
    FAKE, NULL = ctypes.c_void_p(0x10000), ctypes.c_void_p(0)
    f = lib.fgs_quantize_blockwise_noalloc
    assert f(FAKE, 128, 128, 128, 7, FAKE, FAKE, NULL, NULL, NULL) == _lib.FGS_ERR_INVALID_ARG
    assert f(FAKE, 128, 100, 104, 0, FAKE, FAKE, NULL, NULL, NULL) == _lib.FGS_ERR_UNSUPPORTED
    assert f(FAKE, 0, 128, 128, 0, FAKE, FAKE, NULL, NULL, NULL) == _lib.FGS_OK
