"""Python binding of libfgs: argument marshalling only.

Every step of the path runs in the HIP kernels behind the C ABI; this module
checks tensor placement and dtypes, allocates outputs with torch, and passes
raw device pointers plus torch's current HIP stream.  There is no CPU
fallback: without the built library or a GPU every call raises.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import (ELEM_E2M1, ELEM_E4M3, ELEM_E5M2, OUT_BF16, OUT_FP32, ROUND_RNE, ROUND_STOCHASTIC,
                   SCALE_BLOCK_128x128, SCALE_MX32_E8M0, SCALE_NV16_E4M3, SCALE_TENSOR,
                   SCALE_TILE_1x128, FgsOperand, check)

MODES = {"tensor": SCALE_TENSOR, "tile": SCALE_TILE_1x128, "block": SCALE_BLOCK_128x128}


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("fine_grained_scaled_amd operates on GPU tensors only")


def _bf16_matrix(x: torch.Tensor):
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("x must be a 2-D bfloat16 tensor")
    _need_gpu(x)
    if x.stride(1) != 1:
        raise ValueError("x must have unit stride along columns")
    return x.shape[0], x.shape[1], x.stride(0)


def _workspace(device) -> torch.Tensor:
    n = _lib.load().fgs_workspace_bytes(0, 0)
    return torch.empty(n, dtype=torch.uint8, device=device)


@dataclass
class Operand:
    """A quantized GEMM operand of `rows` x `K`, K-contiguous."""
    data: torch.Tensor
    scales: torch.Tensor
    scale_mode: int
    elem: int = ELEM_E4M3
    tensor_scale: Optional[torch.Tensor] = None
    ld: Optional[int] = None

    def c_struct(self) -> FgsOperand:
        ld = self.ld
        if ld is None:
            ld = self.data.stride(-2) * (2 if self.elem == ELEM_E2M1 else 1)
        return FgsOperand(self.data.data_ptr(), ld, self.elem, self.scale_mode,
                          self.scales.data_ptr(),
                          self.tensor_scale.data_ptr() if self.tensor_scale is not None else 0)


@dataclass
class Quantized:
    q: Optional[torch.Tensor]
    scales: Optional[torch.Tensor]
    qT: Optional[torch.Tensor]
    scalesT: Optional[torch.Tensor]
    scale_mode: int
    elem: int = ELEM_E4M3
    tensor_scale: Optional[torch.Tensor] = None   # NVFP4: [2] (row-wise, column-wise)

    def rowwise(self) -> Operand:
        ts = self.tensor_scale[0:1] if self.tensor_scale is not None else None
        return Operand(self.q, self.scales, self.scale_mode, self.elem, ts)

    def colwise(self) -> Operand:
        ts = self.tensor_scale[1:2] if self.tensor_scale is not None else None
        scales = self.scalesT
        if scales is None and self.scale_mode == SCALE_TENSOR:
            scales = self.scales
        return Operand(self.qT, scales, self.scale_mode, self.elem, ts)


def quantize_blockwise(x: torch.Tensor, mode: str = "tile", rowwise: bool = True,
                       colwise: bool = False, workspace: Optional[torch.Tensor] = None) -> Quantized:
    """Online FP32-scaled E4M3 quantization (1x128 tiles, 128x128 blocks or
    one per-tensor scale); row-wise and/or transposed (column-wise) outputs.
    workspace: optional uint8 device scratch for the per-tensor amax pass
    (default: fgs_workspace_bytes() bytes)."""
    rows, cols, ldx = _bf16_matrix(x)
    m = MODES[mode]
    dev = x.device
    q = s = qT = sT = None
    if rowwise:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        if m == SCALE_TILE_1x128:
            s = torch.empty(((cols + 127) // 128, rows), dtype=torch.float32, device=dev)
        elif m == SCALE_BLOCK_128x128:
            s = torch.empty(((rows + 127) // 128, (cols + 127) // 128), dtype=torch.float32, device=dev)
        else:
            s = torch.empty(1, dtype=torch.float32, device=dev)
    if colwise:
        qT = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
        if m == SCALE_TILE_1x128:
            sT = torch.empty(((rows + 127) // 128, cols), dtype=torch.float32, device=dev)
        elif m == SCALE_BLOCK_128x128:
            sT = torch.empty(((cols + 127) // 128, (rows + 127) // 128), dtype=torch.float32, device=dev)
        else:
            sT = torch.empty(1, dtype=torch.float32, device=dev)
    ws = None
    if m == SCALE_TENSOR:
        ws = _workspace(dev) if workspace is None else workspace
        _need_gpu(ws)
    check(_lib.load().fgs_quantize_blockwise(
        _ptr(x), rows, cols, ldx, m, _ptr(q), _ptr(s), _ptr(qT), _ptr(sT),
        _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0, _stream()))
    return Quantized(q, s, qT, sT, m)


def quantize_delayed(x: torch.Tensor, amax_history: torch.Tensor, slot: int, elem: str = "e4m3",
                     rowwise: bool = True, colwise: bool = False) -> Quantized:
    """Per-tensor delayed scaling: the scale comes from the max of
    amax_history (float32 [H] on the GPU, zeros before the first step),
    this tensor's amax is then stored in amax_history[slot]; codes saturate.
    elem "e4m3" (448) or "e5m2" (57344, the hybrid recipe's gradients)."""
    rows, cols, ldx = _bf16_matrix(x)
    _need_gpu(amax_history)
    if amax_history.dtype != torch.float32 or amax_history.dim() != 1 or not amax_history.is_contiguous():
        raise TypeError("amax_history must be a contiguous 1-D float32 tensor")
    codes = {"e4m3": ELEM_E4M3, "e5m2": ELEM_E5M2}
    if elem not in codes:
        raise ValueError("elem must be 'e4m3' or 'e5m2'")
    dev = x.device
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev) if rowwise else None
    qT = torch.empty((cols, rows), dtype=torch.uint8, device=dev) if colwise else None
    s = torch.empty(1, dtype=torch.float32, device=dev)
    check(_lib.load().fgs_quantize_delayed(_ptr(x), rows, cols, ldx, codes[elem], _ptr(amax_history),
                                           amax_history.numel(), slot, _ptr(q), _ptr(qT), _ptr(s), _stream()))
    return Quantized(q, s, qT, None, SCALE_TENSOR, codes[elem])


def quantize_mx(x: torch.Tensor, rowwise: bool = True, colwise: bool = False) -> Quantized:
    """MXFP8: E4M3 codes with an E8M0 power-of-two scale per 32 elements."""
    rows, cols, ldx = _bf16_matrix(x)
    dev = x.device
    q = s = qT = sT = None
    if rowwise:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        s = torch.empty((rows, (cols + 31) // 32), dtype=torch.uint8, device=dev)
    if colwise:
        qT = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
        sT = torch.empty((cols, (rows + 31) // 32), dtype=torch.uint8, device=dev)
    check(_lib.load().fgs_quantize_mx(_ptr(x), rows, cols, ldx, _ptr(q), _ptr(s), _ptr(qT), _ptr(sT), _stream()))
    return Quantized(q, s, qT, sT, SCALE_MX32_E8M0)


def quantize_nvfp4(x: torch.Tensor, rowwise: bool = True, colwise: bool = False,
                   rht_mask: int = 0, rht_seed: int = 0, stochastic: bool = False,
                   sr_seed: int = 0, workspace: Optional[torch.Tensor] = None) -> Quantized:
    """NVFP4: packed E2M1 codes, E4M3 scale per 16 elements, FP32 tensor
    scale; optional random Hadamard transform and stochastic rounding.
    workspace: optional uint8 device scratch for the tensor-amax pass
    (default: fgs_workspace_bytes() bytes)."""
    rows, cols, ldx = _bf16_matrix(x)
    dev = x.device
    q = s = qT = sT = None
    if rowwise:
        q = torch.empty((rows, (cols + 1) // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((rows, (cols + 15) // 16), dtype=torch.uint8, device=dev)
    if colwise:
        qT = torch.empty((cols, (rows + 1) // 2), dtype=torch.uint8, device=dev)
        sT = torch.empty((cols, (rows + 15) // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(2, dtype=torch.float32, device=dev)
    ws = _workspace(dev) if workspace is None else workspace
    _need_gpu(ws)
    check(_lib.load().fgs_quantize_nvfp4(
        _ptr(x), rows, cols, ldx, rht_mask, rht_seed & (2**64 - 1),
        ROUND_STOCHASTIC if stochastic else ROUND_RNE, sr_seed & (2**64 - 1),
        _ptr(q), _ptr(s), _ptr(qT), _ptr(sT), _ptr(ts), _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return Quantized(q, s, qT, sT, SCALE_NV16_E4M3, ELEM_E2M1, ts)


def _check_operand(op: Operand, rows: int, K: int, name: str, groups: int = 1):
    """Shape checks of an operand's device buffers against what the kernels
    read for `rows` x `K` (per group), so a mis-sized tensor raises here
    instead of being read out of bounds."""
    if op.data.dtype != torch.uint8 or op.data.dim() != 2:
        raise TypeError(f"{name}.data must be a 2-D uint8 tensor")
    per_byte = 2 if op.elem == ELEM_E2M1 else 1
    if op.data.shape[0] < rows * groups or op.data.shape[1] * per_byte < K or op.data.stride(1) != 1:
        raise ValueError(f"{name}.data has shape {tuple(op.data.shape)}; needs {rows * groups} x {K} codes, unit column stride")
    m = op.scale_mode
    if m == SCALE_TENSOR:
        need, dt = 1, torch.float32
    elif m == SCALE_TILE_1x128:
        need, dt = (K // 128) * rows, torch.float32
    elif m == SCALE_BLOCK_128x128:
        need, dt = groups * ((rows + 127) // 128) * (K // 128), torch.float32
    elif m == SCALE_MX32_E8M0:
        need, dt = rows * (K // 32), torch.uint8
    elif m == SCALE_NV16_E4M3:
        need, dt = rows * (K // 16), torch.uint8
        if op.tensor_scale is None or op.tensor_scale.numel() < 1 or op.tensor_scale.dtype != torch.float32:
            raise ValueError(f"{name}.tensor_scale must be a float32 tensor with one element")
    else:
        raise ValueError(f"{name}: unknown scale mode {m}")
    if op.scales.dtype != dt or op.scales.numel() < need or not op.scales.is_contiguous():
        raise ValueError(f"{name}.scales must be a contiguous {dt} tensor of at least {need} elements "
                         f"(got {op.scales.dtype}, {op.scales.numel()})")


TILES = {"auto": _lib.TILE_AUTO, "narrow": _lib.TILE_NARROW, "wide": _lib.TILE_WIDE}


def _tile_code(tile: str) -> int:
    if tile not in TILES:
        raise ValueError(f"tile must be one of {sorted(TILES)}")
    return TILES[tile]


def _out_code(out_dtype):
    if out_dtype == torch.float32:
        return OUT_FP32
    if out_dtype == torch.bfloat16:
        return OUT_BF16
    raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")


def gemm_block_scaled(A: Operand, B: Operand, out_dtype=torch.float32,
                      out: Optional[torch.Tensor] = None, K: Optional[int] = None,
                      fp8_mma: bool = False, tile: str = "auto", workspace: bool = True) -> torch.Tensor:
    """C[M x N] = sum_k A^[m, k] * B^[n, k] over scaled low-precision operands.
    fp8_mma=True runs the FP8 matrix instructions with promotion per 128-K
    block (FP8 operands only; a looser error bound than the exact default).
    tile: "auto" (chosen per problem), "narrow" (256 x 128 outputs per
    workgroup) or "wide" (256 x 256).  workspace: for MXFP8 on the exact
    path, hand the library fgs_gemm_workspace_bytes of torch-allocated
    scratch (same bits, faster); False makes every tile scan its rows' scale
    bytes.  The defaults call fgs_gemm_block_scaled /
    fgs_gemm_block_scaled_fp8mma; a forced tile or a workspace
    fgs_gemm_block_scaled_ex."""
    _need_gpu(A.data, B.data, A.scales, B.scales)
    M, N = A.data.shape[0], B.data.shape[0]
    if K is None:
        K = A.data.shape[1] * (2 if A.elem == ELEM_E2M1 else 1)
    code = _out_code(out_dtype)
    tcode = _tile_code(tile)
    _check_operand(A, M, K, "A")
    _check_operand(B, N, K, "B")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.data.device)
    if out.dtype != out_dtype or out.dim() != 2 or out.shape[0] < M or out.shape[1] < N or out.stride(1) != 1:
        raise ValueError("out must be a [M x N] tensor of out_dtype with unit column stride")
    a, b = A.c_struct(), B.c_struct()
    lib = _lib.load()
    # MXFP8 on the exact path: a workspace for the rows' reference exponents
    # (formed once per launch instead of by every tile)
    ws_bytes = 0 if fp8_mma else lib.fgs_gemm_workspace_bytes(A.scale_mode, M, N) if workspace else 0
    if tcode == _lib.TILE_AUTO and ws_bytes == 0:
        fn = lib.fgs_gemm_block_scaled_fp8mma if fp8_mma else lib.fgs_gemm_block_scaled
        check(fn(ctypes.byref(a), ctypes.byref(b), M, N, K, _ptr(out), out.stride(0), code, _stream()))
    else:
        ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=A.data.device) if ws_bytes else None
        opt = _lib.FgsGemmOptions(tcode, 1 if fp8_mma else 0, None, None,
                                  ws.data_ptr() if ws is not None else None, ws_bytes)
        check(lib.fgs_gemm_block_scaled_ex(ctypes.byref(a), ctypes.byref(b), M, N, K, _ptr(out), out.stride(0),
                                           code, ctypes.byref(opt), _stream()))
    return out


def gemm_kernel_name(A: Operand, B: Operand, out_dtype=torch.float32, K: Optional[int] = None,
                     fp8_mma: bool = False, tile: str = "auto") -> str:
    """Name of the kernel instantiation gemm_block_scaled(A, B, out_dtype,
    fp8_mma=..., tile=...) launches, as profilers print it (nothing is
    launched)."""
    M, N = A.data.shape[0], B.data.shape[0]
    if K is None:
        K = A.data.shape[1] * (2 if A.elem == ELEM_E2M1 else 1)
    a, b = A.c_struct(), B.c_struct()
    opt = _lib.FgsGemmOptions(_tile_code(tile), 1 if fp8_mma else 0, None, None)
    buf = ctypes.create_string_buffer(256)
    check(_lib.load().fgs_gemm_kernel_name(ctypes.byref(a), ctypes.byref(b), M, N, K, _out_code(out_dtype),
                                           ctypes.byref(opt), buf, len(buf)))
    return buf.value.decode()


def gemm_block_scaled_fp8out(A: Operand, B: Operand, bf16_out: bool = True, K: Optional[int] = None,
                             tile: str = "auto"):
    """gemm_block_scaled with BF16 output whose epilogue also quantizes it in
    1x128 tiles along N (the next layer's A operand).  Returns (Quantized
    with q [M x N] and scales [N/128][M], the BF16 C or None).  tile as for
    gemm_block_scaled (a forced tile calls fgs_gemm_block_scaled_ex)."""
    _need_gpu(A.data, B.data, A.scales, B.scales)
    M, N = A.data.shape[0], B.data.shape[0]
    if K is None:
        K = A.data.shape[1] * (2 if A.elem == ELEM_E2M1 else 1)
    tcode = _tile_code(tile)
    _check_operand(A, M, K, "A")
    _check_operand(B, N, K, "B")
    dev = A.data.device
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if bf16_out else None
    q = torch.empty((M, N), dtype=torch.uint8, device=dev)
    s = torch.empty(((N + 127) // 128, M), dtype=torch.float32, device=dev)
    a, b = A.c_struct(), B.c_struct()
    lib = _lib.load()
    if tcode == _lib.TILE_AUTO:
        check(lib.fgs_gemm_block_scaled_fp8out(ctypes.byref(a), ctypes.byref(b), M, N, K, _ptr(c),
                                               N, _ptr(q), _ptr(s), _stream()))
    else:
        opt = _lib.FgsGemmOptions(tcode, 0, q.data_ptr(), s.data_ptr())
        check(lib.fgs_gemm_block_scaled_ex(ctypes.byref(a), ctypes.byref(b), M, N, K, _ptr(c), N, OUT_BF16,
                                           ctypes.byref(opt), _stream()))
    return Quantized(q, s, None, None, SCALE_TILE_1x128), c


def grouped_gemm_block_scaled_fp8out(A: Operand, B: Operand, group_offsets: torch.Tensor, N: int,
                                     bf16_out: bool = True, K: Optional[int] = None):
    """grouped_gemm_block_scaled with BF16 output and the 1x128 E4M3 codes of
    that output from the same epilogue (rows of no group are not written)."""
    _need_gpu(A.data, B.data, group_offsets)
    if group_offsets.dtype != torch.int32:
        raise TypeError("group_offsets must be int32")
    total_M = A.data.shape[0]
    G = group_offsets.numel() - 1
    if K is None:
        K = A.data.shape[1]
    _check_operand(A, total_M, K, "A")
    if B.scale_mode != SCALE_BLOCK_128x128 or B.data.shape[0] < G * N:
        raise ValueError("B must hold G x N rows of codes with 128x128 block scales")
    _check_operand(B, N, K, "B", groups=G)
    dev = A.data.device
    c = torch.empty((total_M, N), dtype=torch.bfloat16, device=dev) if bf16_out else None
    q = torch.empty((total_M, N), dtype=torch.uint8, device=dev)
    s = torch.empty(((N + 127) // 128, total_M), dtype=torch.float32, device=dev)
    a, b = A.c_struct(), B.c_struct()
    check(_lib.load().fgs_grouped_gemm_block_scaled_fp8out(ctypes.byref(a), ctypes.byref(b), _ptr(group_offsets),
                                                           G, total_M, N, K, _ptr(c), N, _ptr(q), _ptr(s),
                                                           _stream()))
    return Quantized(q, s, None, None, SCALE_TILE_1x128), c


def grouped_gemm_block_scaled(A: Operand, B: Operand, group_offsets: torch.Tensor, N: int,
                              out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                              K: Optional[int] = None, fp8_mma: bool = False) -> torch.Tensor:
    """MoE expert GEMMs: rows offsets[g]..offsets[g+1] of A times B_g^T.
    B.data is [G*N x K] (groups contiguous); group_offsets is int32 [G+1] on the GPU.
    fp8_mma=True runs fgs_grouped_gemm_block_scaled_fp8mma (FP8 instructions)."""
    _need_gpu(A.data, B.data, group_offsets)
    if group_offsets.dtype != torch.int32:
        raise TypeError("group_offsets must be int32")
    total_M = A.data.shape[0]
    G = group_offsets.numel() - 1
    if K is None:
        K = A.data.shape[1]
    code = _out_code(out_dtype)
    _check_operand(A, total_M, K, "A")
    if B.scale_mode != SCALE_BLOCK_128x128 or B.data.shape[0] < G * N:
        raise ValueError("B must hold G x N rows of codes with 128x128 block scales")
    _check_operand(B, N, K, "B", groups=G)
    if out is None:
        out = torch.empty((total_M, N), dtype=out_dtype, device=A.data.device)
    if out.dtype != out_dtype or out.dim() != 2 or out.shape[0] < total_M or out.shape[1] < N or out.stride(1) != 1:
        raise ValueError("out must be a [total_M x N] tensor of out_dtype with unit column stride")
    a, b = A.c_struct(), B.c_struct()
    lib = _lib.load()
    fn = lib.fgs_grouped_gemm_block_scaled_fp8mma if fp8_mma else lib.fgs_grouped_gemm_block_scaled
    check(fn(ctypes.byref(a), ctypes.byref(b), _ptr(group_offsets), G, total_M, N, K, _ptr(out), out.stride(0),
             code, _stream()))
    return out


def grouped_colwise_blocks(rows: int, G: int) -> int:
    """128-token blocks of the per-group column-wise layout: rows // 128 + G."""
    return int(_lib.load().fgs_grouped_colwise_blocks(rows, G))


def quantize_grouped_colwise(x: torch.Tensor, group_offsets: torch.Tensor,
                             rowwise: bool = False, row_index: Optional[torch.Tensor] = None,
                             colwise: bool = True) -> Quantized:
    """MoE weight-gradient operand: per-group transposed 1x128 E4M3
    quantization of x [T x C] (rows offsets[g]..offsets[g+1]-1 are group g).
    qT is [C x 128 * blocks]: group g takes the 128-column blocks from
    offsets[g] // 128 + g on, zero-padded to whole blocks; scalesT is
    [blocks x C].  rowwise=True adds the ordinary 1x128 row-wise output of
    the grouped rows from the same read.  row_index (int32 [T] on the GPU)
    gathers: row t is x[row_index[t]] (the MoE dispatch permutation), an
    index outside x's rows reading as zeros."""
    src_rows, cols, ldx = _bf16_matrix(x)
    _need_gpu(group_offsets, row_index)
    rows = src_rows
    if row_index is not None:
        if row_index.dtype != torch.int32 or row_index.dim() != 1 or not row_index.is_contiguous():
            raise TypeError("row_index must be a contiguous 1-D int32 tensor")
        rows = row_index.numel()
    if group_offsets.dtype != torch.int32 or group_offsets.dim() != 1 or not group_offsets.is_contiguous():
        raise TypeError("group_offsets must be a contiguous 1-D int32 tensor")
    G = group_offsets.numel() - 1
    if G < 0:
        raise ValueError("group_offsets needs G + 1 >= 1 entries")
    nb = grouped_colwise_blocks(rows, G)
    dev = x.device
    qT = sT = q = s = None
    if colwise:
        qT = torch.empty((cols, 128 * nb), dtype=torch.uint8, device=dev)
        sT = torch.empty((nb, cols), dtype=torch.float32, device=dev)
    if rowwise:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        s = torch.empty(((cols + 127) // 128, rows), dtype=torch.float32, device=dev)
    check(_lib.load().fgs_quantize_grouped_colwise(
        _ptr(x), rows, cols, ldx, _ptr(row_index), src_rows, _ptr(group_offsets), G, _ptr(q), _ptr(s),
        _ptr(qT), 128 * nb, _ptr(sT), _stream()))
    return Quantized(q, s, qT, sT, SCALE_TILE_1x128)


def swiglu_quantize_grouped(gate_up: torch.Tensor, group_offsets: torch.Tensor, rowwise: bool = True,
                            colwise: bool = True, return_h: bool = False):
    """SwiGLU of a gate/up GEMM output [T x 2*I] (gate | up halves) fused
    into the grouped 1x128 quantizer: the row-wise codes feed the down
    projection's forward, the per-expert transposed codes its wgrad.
    Returns the Quantized outputs, and the BF16 activation [T x I] too when
    return_h (rows of no group are left unwritten)."""
    rows, cols2, ld = _bf16_matrix(gate_up)
    _need_gpu(group_offsets)
    if group_offsets.dtype != torch.int32 or group_offsets.dim() != 1 or not group_offsets.is_contiguous():
        raise TypeError("group_offsets must be a contiguous 1-D int32 tensor")
    if cols2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    inter = cols2 // 2
    G = group_offsets.numel() - 1
    nb = grouped_colwise_blocks(rows, G)
    dev = gate_up.device
    q = s = qT = sT = h = None
    if rowwise:
        q = torch.empty((rows, inter), dtype=torch.uint8, device=dev)
        s = torch.empty(((inter + 127) // 128, rows), dtype=torch.float32, device=dev)
    if colwise:
        qT = torch.empty((inter, 128 * nb), dtype=torch.uint8, device=dev)
        sT = torch.empty((nb, inter), dtype=torch.float32, device=dev)
    if return_h:
        h = torch.empty((rows, inter), dtype=torch.bfloat16, device=dev)
    check(_lib.load().fgs_swiglu_quantize_grouped(
        _ptr(gate_up), rows, inter, ld, _ptr(group_offsets), G, _ptr(h), _ptr(q), _ptr(s),
        _ptr(qT), 128 * nb, _ptr(sT), _stream()))
    qq = Quantized(q, s, qT, sT, SCALE_TILE_1x128)
    return (qq, h) if return_h else qq


def grouped_wgrad_block_scaled(A: Operand, B: Operand, group_offsets: torch.Tensor, total_T: int,
                               out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                               fp8_mma: bool = False) -> torch.Tensor:
    """MoE weight gradients: C_g [M x N] = sum over group g's tokens of
    A^[m, t] B^[n, t], for operands from quantize_grouped_colwise (A of dY,
    B of X) over total_T tokens.  Returns [G x M x N]; empty groups get 0.
    fp8_mma=True runs fgs_grouped_wgrad_block_scaled_fp8mma (FP8 instructions)."""
    _need_gpu(A.data, B.data, group_offsets)
    if group_offsets.dtype != torch.int32 or group_offsets.dim() != 1:
        raise TypeError("group_offsets must be a 1-D int32 tensor")
    G = group_offsets.numel() - 1
    M, N = A.data.shape[0], B.data.shape[0]
    code = _out_code(out_dtype)
    if out is None:
        out = torch.empty((max(G, 0), M, N), dtype=out_dtype, device=A.data.device)
    if G <= 0:
        return out
    Kcap = 128 * grouped_colwise_blocks(total_T, G)
    if A.scale_mode != SCALE_TILE_1x128 or B.scale_mode != SCALE_TILE_1x128:
        raise ValueError("grouped wgrad takes 1x128-tile operands")
    _check_operand(A, M, Kcap, "A")
    _check_operand(B, N, Kcap, "B")
    if (out.dtype != out_dtype or out.dim() != 3 or out.shape[0] < G or out.shape[1] < M or out.shape[2] < N
            or out.stride(2) != 1 or out.stride(0) != M * out.stride(1)):
        raise ValueError("out must be a [G x M x N] tensor of out_dtype, rows contiguous, "
                         "matrices M * ldc elements apart")
    a, b = A.c_struct(), B.c_struct()
    lib = _lib.load()
    fn = lib.fgs_grouped_wgrad_block_scaled_fp8mma if fp8_mma else lib.fgs_grouped_wgrad_block_scaled
    check(fn(ctypes.byref(a), ctypes.byref(b), _ptr(group_offsets), G, total_T, M, N, _ptr(out), out.stride(1),
             code, _stream()))
    return out
