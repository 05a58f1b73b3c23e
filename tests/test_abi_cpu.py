"""The C ABI library loads, exports every entry point declared in
include/fgs.h, and rejects invalid arguments with the documented status
codes before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from fine_grained_scaled_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "fgs.h")).read()
    return sorted(set(re.findall(r"\b(fgs_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from fine_grained_scaled_amd import _build
        _build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_workspace(lib):
    assert b"gfx950" in lib.fgs_version()
    assert lib.fgs_workspace_bytes(8192, 4096) >= 8
    assert lib.fgs_last_error() is not None


# Fake, 16-byte aligned, never-dereferenced addresses: every call below must
# be rejected by validation, which happens before any HIP call.
FAKE = ctypes.c_void_p(0x10000)
NULL = ctypes.c_void_p(0)


def _q(lib, *a):
    return lib.fgs_quantize_blockwise(*a)


def test_quantize_blockwise_validation(lib):
    S = ctypes.c_void_p(0)
    assert _q(lib, FAKE, 128, 128, 128, 7, FAKE, FAKE, NULL, NULL, NULL, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert b"mode" in lib.fgs_last_error()
    assert _q(lib, FAKE, -1, 128, 128, 1, FAKE, FAKE, NULL, NULL, NULL, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert _q(lib, NULL, 128, 128, 128, 1, FAKE, FAKE, NULL, NULL, NULL, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert _q(lib, FAKE, 128, 128, 64, 1, FAKE, FAKE, NULL, NULL, NULL, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert _q(lib, FAKE, 128, 100, 104, 1, FAKE, FAKE, NULL, NULL, NULL, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert _q(lib, FAKE, 128, 192, 192, 1, FAKE, FAKE, NULL, NULL, NULL, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert b"128" in lib.fgs_last_error()
    assert _q(lib, FAKE, 100, 128, 128, 1, NULL, NULL, FAKE, FAKE, NULL, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert _q(lib, FAKE, 128, 128, 128, 1, FAKE, NULL, NULL, NULL, NULL, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert _q(lib, FAKE, 128, 128, 128, 0, FAKE, FAKE, NULL, NULL, NULL, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert b"workspace" in lib.fgs_last_error()
    assert _q(lib, ctypes.c_void_p(0x10008), 128, 128, 128, 1, FAKE, FAKE, NULL, NULL, NULL, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    # empty inputs are a no-op success
    assert _q(lib, NULL, 0, 128, 128, 1, NULL, NULL, NULL, NULL, NULL, 0, S) == _lib.FGS_OK


def test_quantize_mx_nvfp4_validation(lib):
    S = NULL
    assert lib.fgs_quantize_mx(FAKE, 128, 48, 48, FAKE, FAKE, NULL, NULL, S) == _lib.FGS_ERR_UNSUPPORTED
    assert lib.fgs_quantize_mx(FAKE, 64, 128, 128, NULL, NULL, FAKE, FAKE, S) == _lib.FGS_ERR_UNSUPPORTED
    assert lib.fgs_quantize_mx(FAKE, 128, 128, 128, FAKE, NULL, NULL, NULL, S) == _lib.FGS_ERR_INVALID_ARG
    args = [FAKE, 128, 128, 128, 4, 0, 0, 0, FAKE, FAKE, NULL, NULL, FAKE, FAKE, 256, S]
    assert lib.fgs_quantize_nvfp4(*args) == _lib.FGS_ERR_INVALID_ARG          # rht_mask 4
    args[4] = 1
    args[6] = 2
    assert lib.fgs_quantize_nvfp4(*args) == _lib.FGS_ERR_INVALID_ARG          # round 2
    args[6] = 1
    args[12] = NULL
    assert lib.fgs_quantize_nvfp4(*args) == _lib.FGS_ERR_INVALID_ARG          # no tensor_scale
    args[12] = FAKE
    args[14] = 4
    assert lib.fgs_quantize_nvfp4(*args) == _lib.FGS_ERR_INVALID_ARG          # workspace too small


def _op(data=FAKE, ld=256, elem=0, mode=1, scales=FAKE, ts=NULL):
    return _lib.FgsOperand(data.value or 0, ld, elem, mode, scales.value or 0, ts.value or 0)


def test_gemm_validation(lib):
    S = NULL
    g = lib.fgs_gemm_block_scaled
    a, b = _op(mode=1), _op(mode=2)
    r = ctypes.byref
    assert g(r(a), r(b), 128, 128, 200, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED      # K % 128
    assert g(r(a), r(b), 128, 128, 0, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED        # K = 0
    assert g(r(a), r(b), -1, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), 128, 128, 256, FAKE, 64, 0, S) == _lib.FGS_ERR_INVALID_ARG       # ldc < N
    assert g(r(a), r(b), 128, 128, 256, FAKE, 128, 5, S) == _lib.FGS_ERR_INVALID_ARG      # out dtype
    assert g(r(a), r(b), 128, 128, 256, NULL, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG      # C NULL
    a2 = _op(ld=100)
    assert g(r(a2), r(b), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG     # ld < K
    a3 = _op(ld=264)
    assert g(r(a3), r(b), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED     # ld % 16
    a4 = _op(mode=2)
    assert g(r(a4), r(b), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED     # A block
    a5 = _op(mode=3)
    assert g(r(a5), r(b), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED     # mixed MX/FP32
    an, bn = _op(elem=1, mode=4), _op(elem=1, mode=4)
    assert g(r(an), r(bn), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG    # no tensor scale
    a6 = _op(scales=NULL)
    assert g(r(a6), r(b), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), 0, 128, 256, NULL, 128, 0, S) == _lib.FGS_OK                     # empty
    big = 1 << 30
    assert g(r(a), r(b), big + 1, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED  # M too large
    assert g(r(a), r(b), big, big, 256, FAKE, big, 0, S) == _lib.FGS_ERR_UNSUPPORTED      # 2^45 tiles
    assert b"tiles" in lib.fgs_last_error()


def test_gemm_ex_options_validation(lib):
    """The per-call options of fgs_gemm_block_scaled_ex: an unknown tile or
    fp8_mma value, a half-given E4M3 output, the E4M3 output with FP32 C,
    on the FP8 instructions or with N % 128 != 0 are rejected before any HIP
    call; NULL options and an all-zero struct validate like the plain entry
    point."""
    S = NULL
    a, b = _op(), _op(mode=2)
    g = lib.fgs_gemm_block_scaled_ex
    r = ctypes.byref
    O = _lib.FgsGemmOptions
    assert g(r(a), r(b), 128, 128, 200, FAKE, 128, 0, None, S) == _lib.FGS_ERR_UNSUPPORTED    # K % 128, NULL opts
    assert g(r(a), r(b), 128, 128, 200, FAKE, 128, 0, r(O()), S) == _lib.FGS_ERR_UNSUPPORTED  # same, zero opts
    assert g(r(a), r(b), 128, 128, 256, FAKE, 128, 0, r(O(3, 0, None, None)), S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), 128, 128, 256, FAKE, 128, 0, r(O(-1, 0, None, None)), S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), 128, 128, 256, FAKE, 128, 0, r(O(0, 2, None, None)), S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), 128, 128, 256, FAKE, 128, 1, r(O(0, 0, 0x10000, None)), S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), 128, 128, 256, FAKE, 128, 0, r(O(0, 0, 0x10000, 0x10000)), S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), 128, 128, 256, FAKE, 128, 1, r(O(2, 1, 0x10000, 0x10000)), S) == _lib.FGS_ERR_UNSUPPORTED
    assert g(r(a), r(b), 128, 136, 256, FAKE, 136, 1, r(O(1, 0, 0x10000, 0x10000)), S) == _lib.FGS_ERR_UNSUPPORTED
    # every valid tile with a K error still reaches the K check
    for tile in (_lib.TILE_AUTO, _lib.TILE_NARROW, _lib.TILE_WIDE):
        assert g(r(a), r(b), 128, 128, 200, FAKE, 128, 0, r(O(tile, 0, None, None)), S) == _lib.FGS_ERR_UNSUPPORTED
    # nothing to do: M = 0 succeeds with any valid option and launches nothing
    assert g(r(a), r(b), 0, 128, 256, FAKE, 128, 0, r(O(2, 1, None, None)), S) == _lib.FGS_OK
    # the workspace: 2 (M + N) bytes for MX32 A scales, none otherwise; one
    # given too small, without a pointer, or misaligned is refused
    wsb = lib.fgs_gemm_workspace_bytes
    assert wsb(3, 300, 200) == 1000 and wsb(1, 300, 200) == 0 and wsb(4, 300, 200) == 0 and wsb(3, -1, 5) == 0
    am, bm = _op(mode=3), _op(mode=3)
    need = wsb(3, 128, 128)
    assert g(r(am), r(bm), 128, 128, 256, FAKE, 128, 0, r(O(0, 0, None, None, 0x10000, need - 1)), S) == \
        _lib.FGS_ERR_INVALID_ARG
    assert b"workspace" in lib.fgs_last_error()
    assert g(r(am), r(bm), 128, 128, 256, FAKE, 128, 0, r(O(0, 0, None, None, None, need)), S) == \
        _lib.FGS_ERR_INVALID_ARG
    assert g(r(am), r(bm), 128, 128, 256, FAKE, 128, 0, r(O(0, 0, None, None, 0x10008, need)), S) == \
        _lib.FGS_ERR_INVALID_ARG
    # the argument checks come first: a valid workspace with a K error still reports K
    assert g(r(am), r(bm), 128, 128, 200, FAKE, 128, 0, r(O(0, 0, None, None, 0x10000, need)), S) == \
        _lib.FGS_ERR_UNSUPPORTED


def test_gemm_kernel_name(lib):
    """The instantiation query launches nothing (fake addresses are fine) and
    names what the GEMM call would run: the forced tiles, the 256 x 128 tile
    for 1x128 B scales, the FP8-instruction flag, BF16 out; "" for an empty
    problem; an argument error returns the GEMM's status and an empty name."""
    import ctypes as C
    O = _lib.FgsGemmOptions
    buf = C.create_string_buffer(256)

    def name(M, N, K, am, bm, out=0, tile=0, mma=0, elem=0):
        a, b = _op(ld=K, mode=am, elem=elem), _op(ld=K, mode=bm, elem=elem)
        st = lib.fgs_gemm_kernel_name(C.byref(a), C.byref(b), M, N, K, out, C.byref(O(tile, mma, None, None)), buf, 256)
        return st, buf.value.decode()

    st, n = name(512, 512, 256, 1, 2, tile=_lib.TILE_NARROW)
    assert st == _lib.FGS_OK and n == "gemm_block_scaled_kernel<Shape<4, 2, 2>, 1, 2, false, 0, 0, false>"
    assert name(512, 512, 256, 1, 2, tile=_lib.TILE_WIDE)[1].startswith("gemm_block_scaled_kernel<Shape<2, 4, 4>, 1, 2,")
    assert name(8192, 6144, 4096, 1, 1, tile=_lib.TILE_WIDE)[1].startswith("gemm_block_scaled_kernel<Shape<4, 2, 2>, 1, 1")
    assert name(512, 512, 256, 0, 0, out=1, tile=_lib.TILE_WIDE)[1].endswith(", 0, 0, true, 0, 0, false>")
    assert name(512, 512, 256, 1, 2, mma=1)[1].endswith(", 0, 0, true>")
    assert name(512, 512, 256, 3, 3, tile=_lib.TILE_NARROW)[1] == \
        "gemm_block_scaled_kernel<Shape<4, 2, 2>, 3, 3, false, 0, 0, false>"
    assert name(0, 512, 256, 1, 2) == (_lib.FGS_OK, "")
    assert name(512, 512, 200, 1, 2) == (_lib.FGS_ERR_UNSUPPORTED, "")
    assert lib.fgs_gemm_kernel_name(C.byref(_op()), C.byref(_op(mode=2)), 128, 128, 256, 0, None, buf, 1) == \
        _lib.FGS_ERR_INVALID_ARG


def test_grouped_validation(lib):
    S = NULL
    g = lib.fgs_grouped_gemm_block_scaled
    a, b = _op(mode=1), _op(mode=2)
    r = ctypes.byref
    assert g(r(a), r(b), FAKE, -1, 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), NULL, 4, 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG
    bt = _op(mode=0)
    assert g(r(a), r(bt), FAKE, 4, 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert g(r(a), r(b), FAKE, 0, 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_OK          # no groups


def test_quantize_delayed_validation(lib):
    S = NULL
    f = lib.fgs_quantize_delayed

    def call(elem=0, rows=256, cols=256, hist=FAKE, H=4, slot=1, q=FAKE, qT=FAKE, sc=FAKE):
        return f(FAKE, rows, cols, cols, elem, hist, H, slot, q, qT, sc, S)
    assert call(elem=1) == _lib.FGS_ERR_INVALID_ARG                 # E2M1 is not an FP8 format
    assert call(hist=NULL) == _lib.FGS_ERR_INVALID_ARG
    assert call(H=0, slot=0) == _lib.FGS_ERR_INVALID_ARG
    assert call(slot=4) == _lib.FGS_ERR_INVALID_ARG
    assert call(slot=-1) == _lib.FGS_ERR_INVALID_ARG
    assert call(sc=NULL) == _lib.FGS_ERR_INVALID_ARG
    assert call(rows=200) == _lib.FGS_ERR_UNSUPPORTED                # column-wise needs rows % 128
    assert call(rows=-1) == _lib.FGS_ERR_INVALID_ARG


def test_gemm_e5m2_operands_need_tensor_scales(lib):
    S = NULL
    g = lib.fgs_gemm_block_scaled
    r = ctypes.byref
    a5, b4 = _op(elem=2, mode=0), _op(elem=0, mode=0)
    assert g(r(a5), r(_op(elem=2, mode=1)), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert b"TENSOR" in lib.fgs_last_error()
    assert g(r(_op(elem=2, mode=2)), r(b4), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert g(r(a5), r(_op(elem=1, mode=4)), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert g(r(_op(elem=7, mode=0)), r(b4), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG


def test_grouped_colwise_validation(lib):
    S = NULL
    q = lib.fgs_quantize_grouped_colwise
    assert lib.fgs_grouped_colwise_blocks(300, 4) == 2 + 4
    assert lib.fgs_grouped_colwise_blocks(-1, 4) == 0
    ld = 128 * 6
    N0 = NULL

    def call(x=FAKE, rows=300, cols=256, ldx=256, idx=N0, src=0, offs=FAKE, G=4, qq=N0, s=N0, qT=FAKE,
             ldq=ld, sT=FAKE):
        return q(x, rows, cols, ldx, idx, src, offs, G, qq, s, qT, ldq, sT, S)
    assert call(G=-1) == _lib.FGS_ERR_INVALID_ARG
    assert call(offs=NULL) == _lib.FGS_ERR_INVALID_ARG
    assert call(sT=NULL) == _lib.FGS_ERR_INVALID_ARG                      # qT without scalesT
    assert call(ldq=ld - 16) == _lib.FGS_ERR_INVALID_ARG
    assert b"ldqT" in lib.fgs_last_error()
    assert call(ldq=ld + 8) == _lib.FGS_ERR_UNSUPPORTED
    assert call(cols=200, ldx=200, qq=FAKE, s=FAKE) == _lib.FGS_ERR_UNSUPPORTED   # row-wise cols % 128
    assert call(qq=FAKE, s=NULL) == _lib.FGS_ERR_INVALID_ARG                     # scales
    assert call(G=0, qT=NULL, ldq=0, sT=NULL) == _lib.FGS_OK                      # no groups
    assert call(rows=0) == _lib.FGS_OK                                            # no rows
    assert call(qT=NULL, sT=NULL) == _lib.FGS_OK                                  # no output
    # gather: x holds src_rows rows, the groups index rows of the gathered matrix
    assert call(idx=FAKE, src=-1) == _lib.FGS_ERR_INVALID_ARG
    assert call(idx=FAKE, src=100, ldx=100) == _lib.FGS_ERR_INVALID_ARG           # ldx < cols
    assert call(x=NULL, idx=FAKE, src=100) == _lib.FGS_ERR_INVALID_ARG
    # the token blocks (floor(rows / 128) + G) run along grid.y: at most 65535
    big_ld = 128 * 65536
    assert call(rows=128 * 65535, G=1, ldq=big_ld) == _lib.FGS_ERR_UNSUPPORTED
    assert b"token blocks" in lib.fgs_last_error()
    assert call(rows=128 * 65534, idx=FAKE, src=100, G=2, ldq=big_ld) == _lib.FGS_ERR_UNSUPPORTED


def test_swiglu_quantize_validation(lib):
    S = NULL
    f = lib.fgs_swiglu_quantize_grouped

    def call(rows=300, inter=256, ld=512, offs=FAKE, G=4, h=NULL, q=FAKE, s=FAKE, qT=FAKE, ldq=128 * 6, sT=FAKE):
        return f(FAKE, rows, inter, ld, offs, G, h, q, s, qT, ldq, sT, S)
    assert call(G=-1) == _lib.FGS_ERR_INVALID_ARG
    assert call(ld=300) == _lib.FGS_ERR_INVALID_ARG                    # ld < 2 * inter
    assert call(inter=252, ld=504) == _lib.FGS_ERR_UNSUPPORTED         # inter % 8
    assert call(inter=200, ld=400) == _lib.FGS_ERR_UNSUPPORTED         # row-wise needs inter % 128
    assert call(offs=NULL) == _lib.FGS_ERR_INVALID_ARG
    assert call(ldq=128 * 5) == _lib.FGS_ERR_INVALID_ARG
    assert call(q=NULL, s=NULL, qT=NULL, sT=NULL) == _lib.FGS_OK        # nothing to write
    assert call(G=0) == _lib.FGS_OK
    assert call(rows=128 * 65000, G=600, ldq=128 * 65600) == _lib.FGS_ERR_UNSUPPORTED   # token blocks


def test_grouped_wgrad_validation(lib):
    S = NULL
    g = lib.fgs_grouped_wgrad_block_scaled
    r = ctypes.byref
    ld = 128 * (2 + 4)
    a, b = _op(mode=1, ld=ld), _op(mode=1, ld=ld)
    assert g(r(a), r(b), FAKE, -1, 300, 128, 128, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), FAKE, 4, -5, 128, 128, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(b), NULL, 4, 300, 128, 128, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG
    short = _op(mode=1, ld=ld - 128)
    assert g(r(short), r(b), FAKE, 4, 300, 128, 128, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG       # ld < 128 * blocks
    blk = _op(mode=2, ld=ld)
    assert g(r(a), r(blk), FAKE, 4, 300, 128, 128, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert g(r(a), r(b), FAKE, 4, 300, 128, 128, FAKE, 64, 0, S) == _lib.FGS_ERR_INVALID_ARG          # ldc < N
    assert g(r(a), r(b), FAKE, 0, 300, 128, 128, NULL, 128, 0, S) == _lib.FGS_OK                      # no groups
    assert g(r(a), r(b), FAKE, 4, 300, 0, 128, NULL, 128, 0, S) == _lib.FGS_OK                        # M = 0
    big = 1 << 30
    wide = _op(mode=1, ld=128 * (2 + 100000))
    assert g(r(wide), r(wide), FAKE, 100000, 300, big, big, FAKE, big, 0, S) == _lib.FGS_ERR_UNSUPPORTED


def test_binding_rejects_mis_sized_operands():
    """The Python binding checks operand buffer sizes before any C call, so a
    mis-sized scale tensor raises instead of being read out of bounds."""
    import torch
    from fine_grained_scaled_amd import ops
    M, K = 256, 512
    codes = torch.zeros((M, K), dtype=torch.uint8)
    ok = [
        ops.Operand(codes, torch.zeros(1), _lib.SCALE_TENSOR),
        ops.Operand(codes, torch.zeros((K // 128, M)), _lib.SCALE_TILE_1x128),
        ops.Operand(codes, torch.zeros((M // 128, K // 128)), _lib.SCALE_BLOCK_128x128),
        ops.Operand(codes, torch.zeros((M, K // 32), dtype=torch.uint8), _lib.SCALE_MX32_E8M0),
    ]
    for op in ok:
        ops._check_operand(op, M, K, "A")
    bad = [
        ops.Operand(codes, torch.zeros((M // 128, K // 128)), _lib.SCALE_MX32_E8M0),      # FP32 block grid as MX
        ops.Operand(codes, torch.zeros((K // 128, M - 1)), _lib.SCALE_TILE_1x128),        # one row short
        ops.Operand(codes[:, :256], torch.zeros(1), _lib.SCALE_TENSOR),                   # K too short
        ops.Operand(codes, torch.zeros((M, K // 32), dtype=torch.uint8), 9),              # unknown mode
        ops.Operand(torch.zeros((M, K // 2), dtype=torch.uint8), torch.zeros((M, K // 16), dtype=torch.uint8),
                    _lib.SCALE_NV16_E4M3, _lib.ELEM_E2M1, None),                          # NVFP4 without tensor scale
    ]
    for op in bad:
        with pytest.raises((ValueError, TypeError)):
            ops._check_operand(op, M, K, "A")


def test_gemm_fp8mma_validation(lib):
    """The FP8 matrix-instruction GEMM validates like the default GEMM and
    rejects E2M1 operands (their E4M3 block scales have no FP8-instruction
    form) before any HIP call."""
    S = NULL
    g = lib.fgs_gemm_block_scaled_fp8mma
    r = ctypes.byref
    a, b = _op(mode=1), _op(mode=2)
    assert g(r(a), r(b), 128, 128, 200, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED      # K % 128
    assert g(r(a), r(b), 128, 128, 0, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED        # K = 0
    assert g(r(a), r(b), 128, 128, 256, FAKE, 64, 0, S) == _lib.FGS_ERR_INVALID_ARG       # ldc < N
    assert g(r(_op(mode=2)), r(b), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED   # A block
    an, bn = _op(elem=1, mode=4, ts=FAKE), _op(elem=1, mode=4, ts=FAKE)
    assert g(r(an), r(bn), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert b"E4M3 / E5M2" in lib.fgs_last_error()
    assert g(r(_op(elem=2, mode=1)), r(b), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert g(r(a), r(b), 0, 128, 256, NULL, 128, 0, S) == _lib.FGS_OK                     # empty


def test_gemm_rejects_row_strides_of_2_pow_24_bytes(lib):
    """Tile rows are addressed by 32-bit offsets from the tile's first row,
    so operand row strides must stay below 2^24 bytes."""
    S = NULL
    r = ctypes.byref
    a_big, b = _op(mode=1, ld=1 << 24), _op(mode=2)
    for g in (lib.fgs_gemm_block_scaled, lib.fgs_gemm_block_scaled_fp8mma):
        assert g(r(a_big), r(b), 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
        assert b"2^24" in lib.fgs_last_error()


def test_grouped_fp8mma_validation(lib):
    """The grouped FP8-instruction entry points validate like their exact
    counterparts (before any HIP call)."""
    S = NULL
    r = ctypes.byref
    a, b = _op(mode=1), _op(mode=2)
    g = lib.fgs_grouped_gemm_block_scaled_fp8mma
    assert g(r(a), r(b), FAKE, -1, 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert g(r(a), r(_op(mode=0)), FAKE, 4, 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert g(r(a), r(b), FAKE, 0, 128, 128, 256, FAKE, 128, 0, S) == _lib.FGS_OK
    w = lib.fgs_grouped_wgrad_block_scaled_fp8mma
    ld = 128 * (2 + 4)
    wa, wb = _op(mode=1, ld=ld), _op(mode=1, ld=ld)
    assert w(r(wa), r(wb), FAKE, -1, 300, 128, 128, FAKE, 128, 0, S) == _lib.FGS_ERR_INVALID_ARG
    assert w(r(wa), r(_op(mode=2, ld=ld)), FAKE, 4, 300, 128, 128, FAKE, 128, 0, S) == _lib.FGS_ERR_UNSUPPORTED
    assert w(r(wa), r(wb), FAKE, 0, 300, 128, 128, NULL, 128, 0, S) == _lib.FGS_OK
