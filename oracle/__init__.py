"""CPU oracle for fine-grained scaled low-precision quantization and GEMM.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU library ``fine_grained_scaled_amd``: the element codecs,
quantizers, Hadamard transform and hash live in ``fgs_oracle.c`` (plain C,
IEEE binary32 where the method fixes FP32, exact elsewhere); the GEMM
reference is the plain definition in FP64 with numpy.

Sources are cited by page title and section:
  [DSV3]  "Can you explain the role of FP8 precision in DeepSeek-V3 training"
          (codingmall.com): "Fine-grained quantization" (1x128 activation
          tiles, 128x128 weight blocks, each scaled independently), "Online
          quantization" (scales from the current tile/block), "Increasing
          accumulation precision" (partial sums promoted to FP32 registers at
          intervals), "Unified E4M3 format".
  [NEMO]  "Accelerating FP8 training performance with the NVIDIA NeMo
          framework" (hyper.ai): per-tensor vs block-wise recipes, MXFP8 with
          blocks of 32 values.
  [NVFP4] "NVIDIA developed a method to train neural networks at 4-bit"
          (news.hamidun.com), "How it works": NVFP4, random 16x16 Hadamard
          transforms of gradient inputs, stochastic rounding.

Layouts returned here are the natural row-major ones of the quantized
matrix: codes [rows x cols], scales [row-blocks x col-blocks].  A
"column-wise" (transposed) quantization is the row-wise quantization of the
transposed BF16 matrix, i.e. blocks run along the source rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fgs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-Wall", "-fPIC", "-shared",
             "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile fgs_oracle.c into liboracle.so (gcc, no fused multiply-add)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    U64 = ctypes.c_uint64
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e5m2_decode.restype = ctypes.c_double
    lib.orc_e5m2_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e5m2_encode.restype = ctypes.c_uint8
    lib.orc_e5m2_encode.argtypes = [ctypes.c_float]
    lib.orc_e5m2_encode_array.argtypes = [P, I64, P]
    lib.orc_quant_delayed.argtypes = [P, I64, ctypes.c_int, P, I64, P, P, P]
    lib.orc_f64_to_bf16.restype = ctypes.c_uint16
    lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.orc_f64_to_bf16_array.argtypes = [P, I64, P]
    lib.orc_e2m1_decode.restype = ctypes.c_double
    lib.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e8m0_decode.restype = ctypes.c_double
    lib.orc_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.orc_fmix32.restype = ctypes.c_uint32
    lib.orc_fmix32.argtypes = [ctypes.c_uint32]
    lib.orc_sr_word.restype = ctypes.c_uint32
    lib.orc_sr_word.argtypes = [U64, U64]
    lib.orc_rht_signs.argtypes = [U64, P]
    lib.orc_rht16.argtypes = [P, P, P]
    lib.orc_rht_rows.argtypes = [P, I64, I64, U64, P]
    lib.orc_quant_e4m3_blocks.argtypes = [P, I64, I64, I64, I64, P, P]
    lib.orc_quant_mx.argtypes = [P, I64, I64, P, P]
    lib.orc_quant_nvfp4.argtypes = [P, I64, I64, ctypes.c_int, U64, I64, I64, P, P, P]
    lib.orc_nvfp4_tensor_scale.restype = ctypes.c_float
    lib.orc_nvfp4_tensor_scale.argtypes = [P, I64]
    lib.orc_quant_nvfp4_blocks.argtypes = [P, I64, I64, ctypes.c_float, ctypes.c_int, U64, I64, I64, I64, P, P]
    lib.orc_e4m3_encode_array.argtypes = [P, I64, P]
    lib.orc_e2m1_encode_array.argtypes = [P, I64, ctypes.c_int, P, P]
    lib.orc_sr_word_array.argtypes = [U64, P, I64, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_bf16_bits(x) -> np.ndarray:
    """Accept a uint16 array of BF16 bit patterns (or a torch bfloat16 CPU tensor)."""
    if hasattr(x, "dtype") and str(getattr(x, "dtype", "")) == "torch.bfloat16":
        import torch  # plumbing only: reinterpret the bits
        x = x.contiguous().view(torch.int16).numpy().view(np.uint16)
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("expected BF16 bit patterns as uint16")
    if x.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    return x


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact: BF16 is the upper half)."""
    return (np.ascontiguousarray(x).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# element codecs
# --------------------------------------------------------------------------
def e4m3_decode_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e2m1_decode_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_e2m1_decode(c) for c in range(16)], dtype=np.float64)


def e8m0_decode_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_e8m0_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    out = np.empty(y.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def e5m2_decode_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_e5m2_decode(c) for c in range(256)], dtype=np.float64)


def e5m2_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    out = np.empty(y.shape, dtype=np.uint8)
    _load().orc_e5m2_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def e2m1_encode(y, r=None) -> np.ndarray:
    """E2M1 codes (4-bit, one per uint8); RNE when r is None, else SR with words r."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    out = np.empty(y.shape, dtype=np.uint8)
    if r is None:
        _load().orc_e2m1_encode_array(_ptr(y), y.size, 0, None, _ptr(out))
    else:
        r = np.ascontiguousarray(np.broadcast_to(np.asarray(r, dtype=np.uint32), y.shape))
        _load().orc_e2m1_encode_array(_ptr(y), y.size, 1, _ptr(r), _ptr(out))
    return out


def fmix32(h: int) -> int:
    return int(_load().orc_fmix32(h & 0xFFFFFFFF))


def sr_words(seed: int, idx) -> np.ndarray:
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.uint64))
    out = np.empty(idx.shape, dtype=np.uint32)
    _load().orc_sr_word_array(seed & (2**64 - 1), _ptr(idx), idx.size, _ptr(out))
    return out


def rht_signs(seed: int) -> np.ndarray:
    d = np.empty(16, dtype=np.float32)
    _load().orc_rht_signs(seed & (2**64 - 1), _ptr(d))
    return d


def rht_rows(x_f32: np.ndarray, seed: int) -> np.ndarray:
    """Random Hadamard transform of every 16-chunk of every row (FP32)."""
    x = np.ascontiguousarray(x_f32, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % 16:
        raise ValueError("rows must be a whole number of 16-chunks")
    y = np.empty_like(x)
    _load().orc_rht_rows(_ptr(x), x.shape[0], x.shape[1], seed & (2**64 - 1), _ptr(y))
    return y


# --------------------------------------------------------------------------
# quantizers
# --------------------------------------------------------------------------
_BLOCK = {"tile": (1, 128), "block": (128, 128)}


def quant_e4m3(x, mode: str, colwise: bool = False):
    """FP32-scaled E4M3 quantization ([DSV3] "Fine-grained quantization",
    "Online quantization"; [NEMO] per-tensor recipe).

    mode: "tile" (1x128 along the quantized rows), "block" (128x128) or
    "tensor".  colwise=True quantizes the transpose (blocks along source rows).
    Returns (codes uint8 [R x C], scales float32 [R/br x C/bc]) of the
    quantized matrix (the transpose when colwise).
    """
    xb = _as_bf16_bits(x)
    if colwise:
        xb = np.ascontiguousarray(xb.T)
    rows, cols = xb.shape
    if mode == "tensor":
        br, bc = max(rows, 1), max(cols, 1)
    else:
        br, bc = _BLOCK[mode]
    q = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty(((rows + br - 1) // br, (cols + bc - 1) // bc), dtype=np.float32)
    _load().orc_quant_e4m3_blocks(_ptr(xb), rows, cols, br, bc, _ptr(q), _ptr(scales))
    return q, scales


def quant_delayed(x, elem: str, history, colwise: bool = False):
    """Per-tensor delayed scaling (the recipe that online scaling replaces,
    [DSV3] "Online quantization"; E5M2 for the hybrid recipe, [DSV3]
    "Unified E4M3 format"): the scale comes from the NaN-propagating max of
    the amax history, every element saturates to the format's range.
    elem: "e4m3" or "e5m2".  Returns (codes uint8 [R x C] of x, or of its
    transpose when colwise, scale float32, amax float32 of x: the entry to
    record for later steps)."""
    xb = _as_bf16_bits(x)
    if colwise:
        xb = np.ascontiguousarray(xb.T)
    h = np.ascontiguousarray(np.asarray(history, dtype=np.float32).reshape(-1))
    q = np.empty(xb.shape, dtype=np.uint8)
    sc = np.empty(1, dtype=np.float32)
    am = np.empty(1, dtype=np.float32)
    _load().orc_quant_delayed(_ptr(xb), xb.size, int(elem == "e5m2"), _ptr(h), h.size,
                              _ptr(q), _ptr(sc), _ptr(am))
    return q, sc[0], am[0]


def dequant_tensor(q: np.ndarray, scale, elem: str) -> np.ndarray:
    """codes with one FP32 scale -> FP64 (E4M3 or E5M2 elements)."""
    tab = e5m2_decode_table() if elem == "e5m2" else e4m3_decode_table()
    return tab[q] * np.float64(scale)


def quant_mx(x, colwise: bool = False):
    """MXFP8: E4M3 codes + E8M0 scale per 32 elements ([NEMO] MXFP8)."""
    xb = _as_bf16_bits(x)
    if colwise:
        xb = np.ascontiguousarray(xb.T)
    rows, cols = xb.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty((rows, (cols + 31) // 32), dtype=np.uint8)
    _load().orc_quant_mx(_ptr(xb), rows, cols, _ptr(q), _ptr(scales))
    return q, scales


def quant_nvfp4(x, colwise: bool = False, rht: bool = False, rht_seed: int = 0,
                stochastic: bool = False, sr_seed: int = 0):
    """NVFP4 ([NVFP4] "How it works"): packed E2M1 codes, E4M3 scale per 16,
    FP32 tensor scale; optional random Hadamard transform along the quantized
    dimension and stochastic rounding.  Returns (packed uint8 [R x C/2],
    scales uint8 [R x C/16], tensor_scale float32)."""
    xb = _as_bf16_bits(x)
    src_rows, src_cols = xb.shape
    xf = bf16_bits_to_f32(xb)
    if colwise:
        xf = np.ascontiguousarray(xf.T)
        idx_rs, idx_cs = 1, src_cols          # element (c, r) of x.T is source (r, c)
    else:
        idx_rs, idx_cs = src_cols, 1
    if rht:
        xf = rht_rows(xf, rht_seed)
    rows, cols = xf.shape
    q = np.empty((rows, (cols + 1) // 2), dtype=np.uint8)
    scales = np.empty((rows, (cols + 15) // 16), dtype=np.uint8)
    ts = np.empty(1, dtype=np.float32)
    _load().orc_quant_nvfp4(_ptr(np.ascontiguousarray(xf)), rows, cols, int(stochastic),
                            sr_seed & (2**64 - 1), idx_rs, idx_cs, _ptr(q), _ptr(scales), _ptr(ts))
    return q, scales, ts[0]


def nvfp4_operand_values(x, colwise: bool = False, rht: bool = False, rht_seed: int = 0) -> np.ndarray:
    """The FP32 values NVFP4 quantizes: the BF16 matrix (transposed when
    colwise) widened, with the random Hadamard transform along the quantized
    dimension when rht."""
    xf = bf16_bits_to_f32(_as_bf16_bits(x))
    if colwise:
        xf = np.ascontiguousarray(xf.T)
    if rht:
        xf = rht_rows(xf, rht_seed)
    return np.ascontiguousarray(xf)


def nvfp4_tensor_scale(values_f32: np.ndarray) -> np.float32:
    """s_t of NVFP4 quantization over all of the given FP32 values."""
    v = np.ascontiguousarray(values_f32, dtype=np.float32)
    return np.float32(_load().orc_nvfp4_tensor_scale(_ptr(v), v.size))


def quant_nvfp4_rows(values_f32: np.ndarray, tensor_scale, stochastic: bool = False, sr_seed: int = 0,
                     idx_base: int = 0, idx_rs: int = 0, idx_cs: int = 1):
    """NVFP4 blocks of the given rows under a given tensor scale (the rows
    may be a sample of a larger matrix); the SR word of element (r, c) uses
    source index idx_base + r * idx_rs + c * idx_cs.  Returns (packed, scales)."""
    v = np.ascontiguousarray(values_f32, dtype=np.float32)
    rows, cols = v.shape
    q = np.empty((rows, (cols + 1) // 2), dtype=np.uint8)
    scales = np.empty((rows, (cols + 15) // 16), dtype=np.uint8)
    _load().orc_quant_nvfp4_blocks(_ptr(v), rows, cols, float(tensor_scale), int(stochastic),
                                   sr_seed & (2**64 - 1), idx_base, idx_rs, idx_cs, _ptr(q), _ptr(scales))
    return q, scales


def f64_to_bf16(v) -> np.ndarray:
    """BF16 bits of FP64 values, rounded once to nearest even."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_f64_to_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def swiglu_f64(gate_up, inter: int) -> np.ndarray:
    """The SwiGLU activation between the two expert GEMMs, exact up to FP64:
    h = silu(g) * u = g / (1 + exp(-g)) * u, with [g | u] the two halves of
    the gate/up GEMM's BF16 output [T x 2*inter]."""
    v = bf16_bits_to_f32(_as_bf16_bits(gate_up)).astype(np.float64)
    g, u = v[:, :inter], v[:, inter:2 * inter]
    with np.errstate(over="ignore", invalid="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def swiglu_bf16(gate_up, inter: int) -> np.ndarray:
    """BF16 bits of the SwiGLU activation (one rounding of swiglu_f64)."""
    return f64_to_bf16(swiglu_f64(gate_up, inter))


def gather_rows(x, row_index):
    """BF16 bits of the gathered matrix: row t = x[row_index[t]], zeros for
    an index outside [0, rows of x)."""
    xb = _as_bf16_bits(x)
    idx = np.asarray(row_index, dtype=np.int64)
    out = np.zeros((len(idx), xb.shape[1]), dtype=np.uint16)
    ok = (idx >= 0) & (idx < xb.shape[0])
    out[ok] = xb[idx[ok]]
    return out


def quant_e4m3_grouped_colwise(x, offsets, row_index=None):
    """Per-group transposed 1x128 quantization of the MoE weight-gradient
    operands ([DSV3] "Fine-grained quantization", "Online quantization",
    "Mixed precision framework": the expert GEMMs, wgrad included, take
    1x128 tiles along their contraction, which for wgrad is the tokens).

    Group g holds rows offsets[g] .. offsets[g+1]-1 of x [T x C] (the tokens
    routed to expert g).  Its wgrad operand is the transpose [C x M_g],
    quantized in 1x128 tiles along the tokens; tiles never mix tokens of two
    experts, so the last tile of a group is partial whenever M_g % 128 != 0
    and takes its scale from the tokens present (zero padding would leave
    the amax unchanged).  Returns one (codes uint8 [C x M_g], scales float32
    [C x ceil(M_g/128)]) per group; an empty group gives empty arrays.

    row_index: the MoE dispatch permutation.  When given, the groups index
    the gathered matrix whose row t is x[row_index[t]] (a row of zeros for
    an index outside x).
    """
    xb = gather_rows(x, row_index) if row_index is not None else _as_bf16_bits(x)
    cols = xb.shape[1]
    out = []
    for g in range(len(offsets) - 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 <= r0:
            out.append((np.zeros((cols, 0), np.uint8), np.zeros((cols, 0), np.float32)))
        else:
            out.append(quant_e4m3(xb[r0:r1], "tile", colwise=True))
    return out


# --------------------------------------------------------------------------
# dequantization (exact in FP64)
# --------------------------------------------------------------------------
def dequant_e4m3(q: np.ndarray, scales, mode: str) -> np.ndarray:
    """codes [R x C] with FP32 scales per (1x128 | 128x128 | tensor) block -> FP64."""
    vals = e4m3_decode_table()[q]
    rows, cols = q.shape
    s = np.asarray(scales, dtype=np.float64)
    if mode == "tensor":
        return vals * s.reshape(-1)[0]
    br, bc = _BLOCK[mode]
    full = np.repeat(np.repeat(s, br, axis=0), bc, axis=1)[:rows, :cols]
    return vals * full


def dequant_mx(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    vals = e4m3_decode_table()[q]
    full = np.repeat(e8m0_decode_table()[scales], 32, axis=1)[:, :q.shape[1]]
    return vals * full


def unpack_e2m1(packed: np.ndarray, cols: int) -> np.ndarray:
    lo = packed & 0x0F
    hi = packed >> 4
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out[:, :cols]


def dequant_nvfp4(packed: np.ndarray, scales: np.ndarray, tensor_scale: float, cols: int) -> np.ndarray:
    codes = unpack_e2m1(packed, cols)
    vals = e2m1_decode_table()[codes]
    sb = np.repeat(e4m3_decode_table()[scales], 16, axis=1)[:, :cols]
    return vals * sb * float(tensor_scale)


# --------------------------------------------------------------------------
# GEMM reference: C[m, n] = sum_k A[m, k] * B[n, k] in FP64, plus the bound
# term S[m, n] = sum_k |A[m, k] * B[n, k]|.  The promotion of partial sums to
# FP32 per 128-deep K block ([DSV3] "Increasing accumulation precision") is
# an accuracy device of the GPU path; the reference is exact-ish FP64, and
# the GPU result is accepted within |C - C_ref| <= 1e-5 * S + 1e-6.
# --------------------------------------------------------------------------
def gemm_ref(a_hat: np.ndarray, b_hat: np.ndarray):
    a = np.asarray(a_hat, dtype=np.float64)
    b = np.asarray(b_hat, dtype=np.float64)
    c = a @ b.T
    s = np.abs(a) @ np.abs(b).T
    return c, s


def grouped_wgrad_ref(a_hat_groups, b_hat_groups):
    """MoE weight gradients: per group g, C_g = A_g B_g^T with the
    contraction over the group's tokens (A_g = dequantized dY_g^T [M x M_g],
    B_g = dequantized X_g^T [N x M_g]); a group with no tokens gives C_g = 0.
    Returns (C [G x M x N], S [G x M x N]) in FP64."""
    G = len(a_hat_groups)
    m = a_hat_groups[0].shape[0] if G else 0
    n = b_hat_groups[0].shape[0] if G else 0
    c = np.zeros((G, m, n))
    s = np.zeros((G, m, n))
    for g in range(G):
        if a_hat_groups[g].shape[1] > 0:
            c[g], s[g] = gemm_ref(a_hat_groups[g], b_hat_groups[g])
    return c, s


def grouped_gemm_ref(a_hat: np.ndarray, b_hat_groups, offsets):
    """Per group g: rows offsets[g]..offsets[g+1] of A times B_g^T."""
    a = np.asarray(a_hat, dtype=np.float64)
    n = b_hat_groups[0].shape[0] if len(b_hat_groups) else 0
    c = np.zeros((a.shape[0], n))
    s = np.zeros((a.shape[0], n))
    for g, bg in enumerate(b_hat_groups):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            c[r0:r1], s[r0:r1] = gemm_ref(a[r0:r1], bg)
    return c, s
