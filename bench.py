#!/usr/bin/env python3
"""Throughput of the fine-grained scaled low-precision training path on one
MI355X.

The headline workload (`value`): one step is one pass of the path over the
Llama-3-8B linear layers (M = 8192 tokens; (K, N) = (4096, 6144) QKV,
(4096, 4096) O, (4096, 28672) gate+up, (14336, 4096) down) in both scaling
recipes the pages compare ("Accelerating FP8 training performance with the
NVIDIA NeMo framework": per-tensor current scaling vs block-wise scaling;
"Can you explain the role of FP8 precision in DeepSeek-V3 training",
"Fine-grained quantization": 1x128 activation/gradient tiles, 128x128
weight blocks).  For every layer and recipe the step runs
  quantize X  (row-wise for fwd, column-wise along M for wgrad; one read)
  quantize W  (row-wise for fwd, transposed for dgrad; one read)
  quantize dY (row-wise along N for dgrad, column-wise along M for wgrad)
  fwd   Y  = X  W^T   (BF16 out)
  dgrad dX = dY W     (BF16 out)
  wgrad dW = dY^T X   (FP32 out)
`value` is the step's GEMM FLOPs over its wall time (quantization
included) in TFLOP/s.  Inputs are seeded synthetic BF16 tensors resident in
HBM before timing starts: every layer has its own X, W and dY, and four
copies of that set (5.9 GiB) sit at distinct addresses, step s reading copy
s mod 4, so no step finds its inputs in the 256 MB last-level cache (MALL)
from the step before.  The line reports the median, p10 and p90 step time,
the rate of every GEMM kernel instantiation (named as profilers print it)
with the dominant one as the roofline, and the quantizers against the HBM
peak and against the read and copy rates of in-tree streaming kernels.

The other workloads of the path are measured in the same run and reported
under "workloads" (per-kernel throughput against the roofline): the tiny
blockwise GEMM, the Llama-3-8B layers in the hybrid delayed-scaling recipe
(per-tensor scales from an amax history, E5M2 gradients), the DeepSeek-V3
MoE grouped GEMMs (forward, dgrad and wgrad), MXFP8 at Llama-3.1-405B
shapes (one GPU's share) and NVFP4 at 12B-hybrid shapes; and the headline
step, the MXFP8 layers and the MoE step again with their GEMMs on the FP8 matrix
instructions (fgs_gemm_block_scaled_fp8mma: FP8 accumulation inside the
instruction with FP32 promotion per 128-K block, MX scales applied by the
instruction; a looser error bound than the exact headline GEMM).

Prints ONE JSON line on stdout; per-kernel breakdowns go to stderr.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-scaled FP8 GEMM TFLOP/s + quant GB/s (% of MI355X peak), 8B/405B shapes"
PEAK_FP16_MFMA = 2500.0     # TFLOP/s, MI355X dense FP16/BF16 matrix peak
PEAK_FP8_MFMA = 5000.0      # TFLOP/s, MI355X dense FP8 matrix peak (context)
PEAK_HBM = 8000.0           # GB/s, MI355X HBM3E

# HBM traffic of the GEMM kernel comes from two committed rocprofv3 counter
# runs (FETCH_SIZE, WRITE_SIZE) summarised here; it is reported only while
# the kernel's sources still hash to the digest recorded with the counters.
COUNTER_PROFILE = os.path.join("profiles", "counters_llama3_8b_linears.md")
# MFMA busy fraction and sustained clock of each GEMM instantiation, from one
# committed rocprofv3 counter run, under the same source-digest rule
MFMA_PROFILE = os.path.join("profiles", "mfma_utilisation_llama3_8b_linears.md")
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_BUSY_CU_CYCLES",
                 "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT")
N_XCD, N_SIMD = 8, 1024                 # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
MAX_SCLK_GHZ = 2.4
GEMM_SOURCES = [os.path.join("fine_grained_scaled_amd", "csrc", f)
                for f in ("gemm_block_scaled.hip", "fgs_device.h", "fgs_internal.h")]
CALIBRATION_BYTES = 1 << 30
HBM_LIB = os.path.join(ROOT, "fine_grained_scaled_amd", "libfgs_hbm.so")
INPUT_SETS = 4

LLAMA8B_M = 8192
LLAMA8B_LAYERS = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672), ("down", 14336, 4096)]
RECIPES = [("blockwise", "tile", "block"), ("per_tensor", "tensor", "tensor")]

MOE_TOKENS, MOE_EXPERTS, MOE_HIDDEN, MOE_INTER = 32768, 256, 7168, 2048
MOE_SOURCE_TOKENS = 4096          # 32768 routed rows = 4096 tokens x top-8
MX_M = 4096
MX_LAYERS = [("qkv", 16384, 18432), ("o", 16384, 16384), ("gate_up", 16384, 106496), ("down", 53248, 16384)]
NV_M = 8192
NV_LAYERS = [("up", 5120, 20480), ("down", 20480, 5120)]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# algorithmic byte counts (what the method itself must move)
# --------------------------------------------------------------------------
def e4m3_bytes(rows, cols, mode, outputs=2):
    """Read BF16 once, write `outputs` code tensors and their FP32 scales;
    per-tensor scaling reads the input a second time for the amax."""
    n = rows * cols
    b = 2 * n + outputs * n
    if mode == "tile":
        b += outputs * 4 * (n // 128)
    elif mode == "block":
        b += outputs * 4 * math.ceil(rows / 128) * math.ceil(cols / 128)
    else:
        b += 2 * n + 4 * outputs
    return b


def mx_bytes(rows, cols, outputs):
    n = rows * cols
    return 2 * n + outputs * (n + n // 32)


def nvfp4_bytes(rows, cols, outputs):
    """Tensor-amax pass (read) + quantize pass (read, codes at 4 bits, one
    E4M3 scale byte per 16)."""
    n = rows * cols
    return 2 * n + 2 * n + outputs * (n // 2 + n // 16)


# --------------------------------------------------------------------------
# timing of individual launches with HIP events on torch's current stream
# (the stream the library launches on)
# --------------------------------------------------------------------------
class Timer:
    """HIP events around each launch on torch's current stream (the stream
    the library launches on).  kname: a callable naming the kernel
    instantiation a GEMM launch runs (asked once per label)."""

    def __init__(self, torch, enabled=True):
        self.torch = torch
        self.enabled = enabled
        self.rec = []
        self.names = {}

    def run(self, kind, label, units, fn, kname=None):
        if not self.enabled:
            return fn()
        if kname is not None and label not in self.names:
            self.names[label] = kname()
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        r = fn()
        e1.record()
        self.rec.append((kind, label, units, e0, e1))
        return r

    def times(self):
        """[(kind, label, units, seconds, kernel name or None)]"""
        return [(k, lab, u, e0.elapsed_time(e1) * 1e-3, self.names.get(lab)) for k, lab, u, e0, e1 in self.rec]

    def summary(self):
        kinds, labels = {}, {}
        for kind, label, units, t, _ in self.times():
            u, s, n = kinds.get(kind, (0.0, 0.0, 0))
            kinds[kind] = (u + units, s + t, n + 1)
            u, s, n = labels.get((kind, label), (0.0, 0.0, 0))
            labels[(kind, label)] = (u + units, s + t, n + 1)
        return kinds, labels


def dense_gemm(tm, fgs, label, A, B, dt, out, fp8_mma=False):
    """One timed dense GEMM launch, recorded with its FLOPs and the name of
    the kernel instantiation it runs."""
    f = 2.0 * A.data.shape[0] * B.data.shape[0] * A.data.shape[1] * (2 if A.elem == fgs.ELEM_E2M1 else 1)
    return tm.run("gemm", label, f, lambda: fgs.gemm_block_scaled(A, B, dt, out=out, fp8_mma=fp8_mma),
                  kname=lambda: fgs.gemm_kernel_name(A, B, dt, fp8_mma=fp8_mma))


def gpu_normal(torch, shape, seed, sigma=1.0, outlier_cols=None):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    v = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    if sigma != 1.0:
        v *= sigma
    if outlier_cols is not None and len(outlier_cols):
        v[:, torch.as_tensor(outlier_cols, device="cuda")] *= 50.0
    return v.to(torch.bfloat16)


def gpu_t3(torch, shape, seed):
    """Student-t(3) scaled to std 1e-3: Z / sqrt(chi2_3 / 3) * 1e-3 / sqrt(3)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    z = torch.randn((4,) + tuple(shape), generator=g, device="cuda", dtype=torch.float32)
    v = (z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3.0
    return (z[0] / v.sqrt() * (1e-3 / math.sqrt(3.0))).to(torch.bfloat16)


# --------------------------------------------------------------------------
# headline: Llama-3-8B linear layers, both recipes
# --------------------------------------------------------------------------
class Llama8B:
    name = "llama3_8b_linears"
    fp8_mma = False

    def __init__(self, torch, fgs, synth, sets=INPUT_SETS):
        self.torch, self.fgs = torch, fgs
        t0 = time.time()
        self.out = {}
        base = {}
        for i, (name, K, N) in enumerate(LLAMA8B_LAYERS):
            # every layer its own seeded X, W and dY (tags per layer)
            x = synth.activations(LLAMA8B_M, K, seed=0, tag=synth.TAG_A + 16 * (1 + i))
            w = synth.weights(N, K, seed=0, tag=synth.TAG_W + 16 * (1 + i))
            dy = synth.gradients(LLAMA8B_M, N, seed=0, tag=synth.TAG_DY + 16 * (1 + i))
            base[name] = tuple(synth.to_torch_bf16(v).cuda() for v in (x, w, dy))
            for rname, _, _ in RECIPES:
                self.out[(rname, name, "y")] = torch.empty((LLAMA8B_M, N), dtype=torch.bfloat16, device="cuda")
                self.out[(rname, name, "dx")] = torch.empty((LLAMA8B_M, K), dtype=torch.bfloat16, device="cuda")
                self.out[(rname, name, "dw")] = torch.empty((N, K), dtype=torch.float32, device="cuda")
        # copies of the input set at distinct addresses, read in rotation
        self.sets = [base] + [{n: tuple(t.clone() for t in v) for n, v in base.items()} for _ in range(sets - 1)]
        self.step_no = 0
        torch.cuda.synchronize()
        nbytes = sum(t.numel() * t.element_size() for st in self.sets for v in st.values() for t in v)
        log(f"[bench] {self.name}: inputs generated and uploaded in {time.time() - t0:.1f} s "
            f"({len(self.sets)} input sets, {nbytes / 2**30:.2f} GiB)")

    def input_bytes(self):
        return sum(t.numel() * t.element_size() for st in self.sets for v in st.values() for t in v)

    def flops(self):
        return len(RECIPES) * sum(3 * 2.0 * LLAMA8B_M * N * K for _, K, N in LLAMA8B_LAYERS)

    def gemm_launches(self):
        """(label, M, N, K, A scale mode, B scale mode, out dtype) of every GEMM
        launch of one step: fwd X W^T, dgrad dY W, wgrad dY^T X."""
        torch = self.torch
        out = []
        for rname, amode, wmode in RECIPES:
            for name, K, N in LLAMA8B_LAYERS:
                M = LLAMA8B_M
                out.append((f"{rname}/{name}/fwd", M, N, K, amode, wmode, torch.bfloat16))
                out.append((f"{rname}/{name}/dgrad", M, K, N, amode, wmode, torch.bfloat16))
                out.append((f"{rname}/{name}/wgrad", N, K, M, amode, amode, torch.float32))
        return out

    @staticmethod
    def gemm_bytes_one(M, N, K, amode, bmode, out_bytes):
        """Algorithmic HBM bytes of one GEMM launch: operand codes and scales
        once, the output once."""
        sc = lambda r, c, mode: 4.0 * (r * c / 128 if mode == "tile" else
                                       r * c / 16384 if mode == "block" else 1)
        return M * K + N * K + sc(M, K, amode) + sc(N, K, bmode) + out_bytes * M * N

    def gemm_bytes(self):
        """Algorithmic HBM bytes of the step's GEMMs."""
        return sum(self.gemm_bytes_one(M, N, K, am, bm, 2 if dt == self.torch.bfloat16 else 4)
                   for _, M, N, K, am, bm, dt in self.gemm_launches())

    def gemm_only(self, steps):
        """Quantize once, then run only the step's GEMM launches `steps` times."""
        torch, fgs = self.torch, self.fgs
        ops = []
        for rname, amode, wmode in RECIPES:
            for name, K, N in LLAMA8B_LAYERS:
                X, W, dY = self.sets[0][name]
                qx = fgs.quantize_blockwise(X, amode, rowwise=True, colwise=True)
                qw = fgs.quantize_blockwise(W, wmode, rowwise=True, colwise=True)
                qdy = fgs.quantize_blockwise(dY, amode, rowwise=True, colwise=True)
                o = self.out
                ops.append((qx.rowwise(), qw.rowwise(), torch.bfloat16, o[(rname, name, "y")]))
                ops.append((qdy.rowwise(), qw.colwise(), torch.bfloat16, o[(rname, name, "dx")]))
                ops.append((qdy.colwise(), qx.colwise(), torch.float32, o[(rname, name, "dw")]))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            for a, b, dt, out in ops:
                fgs.gemm_block_scaled(a, b, dt, out=out)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        log(f"[bench] GEMM launches only: {dt / steps * 1e3:.2f} ms per step, "
            f"{self.flops() / (dt / steps) / 1e12:.1f} TFLOP/s")

    def gemm(self, tm, label, A, B, dt, out):
        dense_gemm(tm, self.fgs, label, A, B, dt, out, self.fp8_mma)

    def step(self, tm):
        torch, fgs = self.torch, self.fgs
        inputs = self.sets[self.step_no % len(self.sets)]
        self.step_no += 1
        for rname, amode, wmode in RECIPES:
            for name, K, N in LLAMA8B_LAYERS:
                X, W, dY = inputs[name]
                lab = f"{rname}/{name}"
                qx = tm.run("quant", lab + "/X", e4m3_bytes(LLAMA8B_M, K, amode),
                            lambda: fgs.quantize_blockwise(X, amode, rowwise=True, colwise=True))
                qw = tm.run("quant", lab + "/W", e4m3_bytes(N, K, wmode),
                            lambda: fgs.quantize_blockwise(W, wmode, rowwise=True, colwise=True))
                qdy = tm.run("quant", lab + "/dY", e4m3_bytes(LLAMA8B_M, N, amode),
                             lambda: fgs.quantize_blockwise(dY, amode, rowwise=True, colwise=True))
                o = self.out
                self.gemm(tm, lab + "/fwd", qx.rowwise(), qw.rowwise(), torch.bfloat16, o[(rname, name, "y")])
                self.gemm(tm, lab + "/dgrad", qdy.rowwise(), qw.colwise(), torch.bfloat16, o[(rname, name, "dx")])
                self.gemm(tm, lab + "/wgrad", qdy.colwise(), qx.colwise(), torch.float32, o[(rname, name, "dw")])


class Llama8BFp8Mma(Llama8B):
    """The headline step with every GEMM on the FP8 matrix instructions
    (fgs_gemm_block_scaled_fp8mma: the pages' own accumulation design, a
    looser error bound than the exact default)."""
    name = "llama3_8b_linears_fp8_mfma"
    fp8_mma = True


# --------------------------------------------------------------------------
# Llama-3-8B linear layers in the hybrid delayed-scaling recipe: per-tensor
# scales from a 16-step amax history, X and W in E4M3, dY in E5M2; one pass
# over each tensor (no amax pass first)
# --------------------------------------------------------------------------
class Hybrid8B:
    name = "llama3_8b_hybrid_delayed"
    HISTORY = 16

    def __init__(self, torch, fgs, synth):
        self.torch, self.fgs = torch, fgs
        self.x, self.w, self.dy, self.out, self.hist = {}, {}, {}, {}, {}
        for i, (name, K, N) in enumerate(LLAMA8B_LAYERS):
            # every layer its own X, W and dY
            self.x[name] = gpu_normal(torch, (LLAMA8B_M, K), 300 + i, outlier_cols=synth.outlier_channels(K, 0))
            self.w[name] = gpu_normal(torch, (N, K), 310 + i, sigma=0.02)
            self.dy[name] = gpu_t3(torch, (LLAMA8B_M, N), 320 + i)
            for role in ("x", "w", "dy"):
                self.hist[(name, role)] = torch.zeros(self.HISTORY, dtype=torch.float32, device="cuda")
            self.out[(name, "y")] = torch.empty((LLAMA8B_M, N), dtype=torch.bfloat16, device="cuda")
            self.out[(name, "dx")] = torch.empty((LLAMA8B_M, K), dtype=torch.bfloat16, device="cuda")
            self.out[(name, "dw")] = torch.empty((N, K), dtype=torch.float32, device="cuda")
        self.step_no = 0
        torch.cuda.synchronize()

    def flops(self):
        return sum(3 * 2.0 * LLAMA8B_M * N * K for _, K, N in LLAMA8B_LAYERS)

    def step(self, tm):
        torch, fgs = self.torch, self.fgs
        slot = self.step_no % self.HISTORY
        self.step_no += 1
        for name, K, N in LLAMA8B_LAYERS:
            X, W, dY, h, o = self.x[name], self.w[name], self.dy[name], self.hist, self.out
            qx = tm.run("quant", name + "/X", 4.0 * LLAMA8B_M * K, lambda: fgs.quantize_delayed(
                X, h[(name, "x")], slot, "e4m3", rowwise=True, colwise=True))
            qw = tm.run("quant", name + "/W", 4.0 * N * K, lambda: fgs.quantize_delayed(
                W, h[(name, "w")], slot, "e4m3", rowwise=True, colwise=True))
            qdy = tm.run("quant", name + "/dY", 4.0 * LLAMA8B_M * N, lambda: fgs.quantize_delayed(
                dY, h[(name, "dy")], slot, "e5m2", rowwise=True, colwise=True))
            dense_gemm(tm, fgs, name + "/fwd", qx.rowwise(), qw.rowwise(), torch.bfloat16, o[(name, "y")])
            dense_gemm(tm, fgs, name + "/dgrad", qdy.rowwise(), qw.colwise(), torch.bfloat16, o[(name, "dx")])
            dense_gemm(tm, fgs, name + "/wgrad", qdy.colwise(), qx.colwise(), torch.float32, o[(name, "dw")])


# --------------------------------------------------------------------------
# tiny blockwise GEMM (launch-bound; time only)
# --------------------------------------------------------------------------
class Tiny:
    name = "tiny_blockwise_128x256x256"

    def __init__(self, torch, fgs, synth):
        self.torch, self.fgs = torch, fgs
        self.a = synth.to_torch_bf16(synth.activations(128, 256, seed=0)).cuda()
        self.b = synth.to_torch_bf16(synth.weights(256, 256, seed=0)).cuda()
        self.c = torch.empty((128, 256), dtype=torch.float32, device="cuda")

    def flops(self):
        return 2.0 * 128 * 256 * 256

    def step(self, tm):
        fgs = self.fgs
        qa = tm.run("quant", "A", e4m3_bytes(128, 256, "tile", 1), lambda: fgs.quantize_blockwise(self.a, "tile"))
        qb = tm.run("quant", "B", e4m3_bytes(256, 256, "block", 1), lambda: fgs.quantize_blockwise(self.b, "block"))
        dense_gemm(tm, fgs, "fwd", qa.rowwise(), qb.rowwise(), self.torch.float32, self.c)


# --------------------------------------------------------------------------
# DeepSeek-V3 MoE: grouped GEMMs over 256 experts, Zipf(1.1) token counts:
# gate/up and down forward (the SwiGLU between them fused into the down
# projection's quantizer), their dgrad on the transposed expert weights, and
# their wgrad (one dW per expert, contraction over its tokens)
# --------------------------------------------------------------------------
class MoE:
    name = "deepseek_v3_moe_grouped"
    fp8_mma = False

    def __init__(self, torch, fgs, synth):
        import numpy as np
        self.torch, self.fgs = torch, fgs
        t0 = time.time()
        counts = synth.expert_counts(MOE_TOKENS, MOE_EXPERTS, 1.1, seed=0)
        self.counts = counts
        self.offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
        T, H, I, G = MOE_TOKENS, MOE_HIDDEN, MOE_INTER, MOE_EXPERTS
        # the tokens before dispatch and the routed row -> token map (seeded
        # random; the per-expert row counts are the Zipf draw above): the
        # dispatch gather is fused into the quantizer's read
        self.x_tok = gpu_normal(torch, (MOE_SOURCE_TOKENS, H), 101, outlier_cols=synth.outlier_channels(H, 0))
        gen = torch.Generator(device="cuda")
        gen.manual_seed(107)
        self.route = torch.randint(0, MOE_SOURCE_TOKENS, (T,), generator=gen, device="cuda", dtype=torch.int32)
        self.g1 = gpu_t3(torch, (T, 2 * I), 105)             # dY of gate+up
        self.g2 = gpu_t3(torch, (T, H), 106)                 # dY of down
        # expert weights, quantized once (128x128 blocks never straddle experts):
        # row-wise for the forward GEMMs, transposed for dgrad
        self.w1, self.w1t = self._expert_weights(G, 2 * I, H, 103)     # gate+up: 7168 -> 4096
        self.w2, self.w2t = self._expert_weights(G, H, I, 104)         # down:    2048 -> 7168
        self.y1 = torch.empty((T, 2 * I), dtype=torch.bfloat16, device="cuda")
        self.y2 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        self.dx1 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        self.dx2 = torch.empty((T, I), dtype=torch.bfloat16, device="cuda")
        # FP32 expert weight gradients: 256 x [4096 x 7168] and 256 x [7168 x 2048]
        self.dw1 = torch.empty((G, 2 * I, H), dtype=torch.float32, device="cuda")
        self.dw2 = torch.empty((G, H, I), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] {self.name}: expert weights generated and quantized in {time.time() - t0:.1f} s "
            f"(token counts max {counts.max()}, min {counts.min()}, {int((counts < 128).sum())} experts < 128)")

    def _expert_weights(self, G, N, K, seed):
        """Per-expert [N x K] weights: row-wise codes [G*N x K] for the forward
        GEMM and transposed codes [G*K x N] for dgrad, 128x128 blocks."""
        torch, fgs = self.torch, self.fgs
        codes = torch.empty((G * N, K), dtype=torch.uint8, device="cuda")
        scales = torch.empty((G * (N // 128), K // 128), dtype=torch.float32, device="cuda")
        codes_t = torch.empty((G * K, N), dtype=torch.uint8, device="cuda")
        scales_t = torch.empty((G * (K // 128), N // 128), dtype=torch.float32, device="cuda")
        for g in range(G):
            w = gpu_normal(torch, (N, K), seed * 1000 + g, sigma=0.02)
            q = fgs.quantize_blockwise(w, "block", rowwise=True, colwise=True)
            codes[g * N:(g + 1) * N] = q.q
            scales[g * (N // 128):(g + 1) * (N // 128)] = q.scales
            codes_t[g * K:(g + 1) * K] = q.qT
            scales_t[g * (K // 128):(g + 1) * (K // 128)] = q.scalesT
            del w, q
        return (fgs.Operand(codes, scales, fgs.SCALE_BLOCK_128x128),
                fgs.Operand(codes_t, scales_t, fgs.SCALE_BLOCK_128x128))

    def flops(self):
        return 3 * 2.0 * MOE_TOKENS * (2 * MOE_INTER * MOE_HIDDEN + MOE_HIDDEN * MOE_INTER)

    def gemm_bytes(self, N, K):
        """Algorithmic HBM bytes of one grouped GEMM: A codes and scales,
        the weights of every expert that has tokens, BF16 output."""
        active = int((self.counts > 0).sum())
        return MOE_TOKENS * K * (1 + 4 / 128) + active * N * K * (1 + 4 / 16384) + 2 * MOE_TOKENS * N

    def mfma_peak(self):
        """The matrix rate the GEMMs run at: FP16 (exact decode) or FP8."""
        return PEAK_FP8_MFMA if self.fp8_mma else PEAK_FP16_MFMA

    def roofline_seconds(self, N, K):
        """Sum over experts of max(MFMA time at the matrix peak, HBM time)."""
        t = 0.0
        for c in self.counts:
            if c == 0:
                continue
            fl = 2.0 * c * N * K
            by = c * K * (1 + 4 / 128) + N * K * (1 + 4 / 16384) + 2 * c * N
            t += max(fl / (self.mfma_peak() * 1e12), by / (PEAK_HBM * 1e9))
        return t

    def wgrad_bytes(self, M, N):
        """Algorithmic HBM bytes of one grouped wgrad: both operands' codes
        and 1x128 scales over the routed tokens, and every expert's FP32
        dW [M x N] (zeros for experts without tokens)."""
        return (M + N) * MOE_TOKENS * (1 + 4 / 128) + MOE_EXPERTS * 4.0 * M * N

    def wgrad_roofline_seconds(self, M, N):
        """Sum over experts of max(MFMA time at the matrix peak, HBM time)."""
        t = 0.0
        for c in self.counts:
            fl = 2.0 * c * M * N
            by = (M + N) * c * (1 + 4 / 128) + 4.0 * M * N
            t += max(fl / (self.mfma_peak() * 1e12), by / (PEAK_HBM * 1e9))
        return t

    def step(self, tm):
        torch, fgs = self.torch, self.fgs
        T, H, I = MOE_TOKENS, MOE_HIDDEN, MOE_INTER
        off = self.offsets
        mma = self.fp8_mma
        # each input is read once for its row-wise codes (fwd / dgrad) and its
        # per-expert transposed codes (wgrad)
        grouped = lambda x: fgs.quantize_grouped_colwise(x, off, rowwise=True)
        # dispatch: the routed rows gathered from the tokens inside the read
        # (algorithmic bytes: the tokens once, the index, both outputs)
        a1_bytes = e4m3_bytes(T, H, "tile", 2) - 2.0 * T * H + 2.0 * MOE_SOURCE_TOKENS * H + 4.0 * T
        qa1 = tm.run("quant", "A1", a1_bytes, lambda: fgs.quantize_grouped_colwise(
            self.x_tok, off, rowwise=True, row_index=self.route))
        tm.run("gemm", "gate_up", 2.0 * T * 2 * I * H, lambda: fgs.grouped_gemm_block_scaled(
            qa1.rowwise(), self.w1, off, 2 * I, torch.bfloat16, out=self.y1, fp8_mma=mma))
        # SwiGLU of the gate/up output fused into the down projection's quantizer
        a2_bytes = 2.0 * T * 2 * I + e4m3_bytes(T, I, "tile", 2) - 2.0 * T * I
        qa2 = tm.run("quant", "SwiGLU+A2", a2_bytes, lambda: fgs.swiglu_quantize_grouped(self.y1, off))
        tm.run("gemm", "down", 2.0 * T * H * I, lambda: fgs.grouped_gemm_block_scaled(
            qa2.rowwise(), self.w2, off, H, torch.bfloat16, out=self.y2, fp8_mma=mma))
        # dgrad: dZ = dY2 W2 (2048 outputs, contraction over 7168), dH = dY1 W1
        qg2 = tm.run("quant", "dY2", e4m3_bytes(T, H, "tile", 2), lambda: grouped(self.g2))
        tm.run("gemm", "down_dgrad", 2.0 * T * H * I, lambda: fgs.grouped_gemm_block_scaled(
            qg2.rowwise(), self.w2t, off, I, torch.bfloat16, out=self.dx2, fp8_mma=mma))
        qg1 = tm.run("quant", "dY1", e4m3_bytes(T, 2 * I, "tile", 2), lambda: grouped(self.g1))
        tm.run("gemm", "gate_up_dgrad", 2.0 * T * 2 * I * H, lambda: fgs.grouped_gemm_block_scaled(
            qg1.rowwise(), self.w1t, off, H, torch.bfloat16, out=self.dx1, fp8_mma=mma))
        # wgrad: dW2_g = dY2_g^T Z_g [7168 x 2048], dW1_g = dY1_g^T X_g [4096 x 7168]
        tm.run("gemm", "down_wgrad", 2.0 * T * H * I, lambda: fgs.grouped_wgrad_block_scaled(
            qg2.colwise(), qa2.colwise(), off, T, torch.float32, out=self.dw2, fp8_mma=mma))
        tm.run("gemm", "gate_up_wgrad", 2.0 * T * 2 * I * H, lambda: fgs.grouped_wgrad_block_scaled(
            qg1.colwise(), qa1.colwise(), off, T, torch.float32, out=self.dw1, fp8_mma=mma))


class MoEFp8Mma(MoE):
    """The MoE step with its grouped GEMMs on the FP8 matrix instructions."""
    name = "deepseek_v3_moe_grouped_fp8_mfma"
    fp8_mma = True


# --------------------------------------------------------------------------
# MXFP8 at Llama-3.1-405B shapes (one GPU's share, one layer): fwd + wgrad
# --------------------------------------------------------------------------
class MX405B:
    name = "llama31_405b_mxfp8"
    fp8_mma = False

    def __init__(self, torch, fgs, synth):
        self.torch, self.fgs = torch, fgs
        t0 = time.time()
        self.x, self.w, self.dy, self.out = {}, {}, {}, {}
        for i, (name, K, N) in enumerate(MX_LAYERS):
            self.x[name] = gpu_normal(torch, (MX_M, K), 200 + i)      # every layer its own X
            self.w[name] = gpu_normal(torch, (N, K), 210 + i, sigma=0.02)
            self.dy[name] = gpu_normal(torch, (MX_M, N), 220 + i)
            self.out[(name, "y")] = torch.empty((MX_M, N), dtype=torch.bfloat16, device="cuda")
            self.out[(name, "dw")] = torch.empty((N, K), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] {self.name}: inputs generated in {time.time() - t0:.1f} s")

    def flops(self):
        return sum(2 * 2.0 * MX_M * N * K for _, K, N in MX_LAYERS)

    def step(self, tm):
        torch, fgs = self.torch, self.fgs
        for name, K, N in MX_LAYERS:
            X, W, dY = self.x[name], self.w[name], self.dy[name]
            qx = tm.run("quant", name + "/X", mx_bytes(MX_M, K, 2), lambda: fgs.quantize_mx(X, rowwise=True, colwise=True))
            qw = tm.run("quant", name + "/W", mx_bytes(N, K, 1), lambda: fgs.quantize_mx(W))
            qdy = tm.run("quant", name + "/dY", mx_bytes(MX_M, N, 1),
                         lambda: fgs.quantize_mx(dY, rowwise=False, colwise=True))
            mma = self.fp8_mma
            dense_gemm(tm, fgs, name + "/fwd", qx.rowwise(), qw.rowwise(), torch.bfloat16, self.out[(name, "y")], mma)
            dense_gemm(tm, fgs, name + "/wgrad", qdy.colwise(), qx.colwise(), torch.float32, self.out[(name, "dw")], mma)


class MX405BFp8Mma(MX405B):
    """MXFP8 with the E8M0 scales applied by the scaled FP8 matrix
    instruction (fgs_gemm_block_scaled_fp8mma)."""
    name = "llama31_405b_mxfp8_fp8_mfma"
    fp8_mma = True


# --------------------------------------------------------------------------
# NVFP4 at 12B-hybrid-like shapes: fwd, dgrad, wgrad (RHT + SR on wgrad)
# --------------------------------------------------------------------------
class NV12B:
    name = "hybrid12b_nvfp4"

    def __init__(self, torch, fgs, synth):
        self.torch, self.fgs = torch, fgs
        self.rht_seed = synth.derived_seed(0, synth.TAG_RHT)
        self.sr_seed = synth.derived_seed(0, synth.TAG_SR)
        t0 = time.time()
        self.x, self.w, self.dy, self.out = {}, {}, {}, {}
        for i, (name, K, N) in enumerate(NV_LAYERS):
            self.x[name] = gpu_normal(torch, (NV_M, K), 300 + i)
            self.w[name] = gpu_normal(torch, (N, K), 310 + i, sigma=0.02)
            self.dy[name] = gpu_t3(torch, (NV_M, N), 320 + i)
            self.out[(name, "y")] = torch.empty((NV_M, N), dtype=torch.bfloat16, device="cuda")
            self.out[(name, "dx")] = torch.empty((NV_M, K), dtype=torch.bfloat16, device="cuda")
            self.out[(name, "dw")] = torch.empty((N, K), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] {self.name}: inputs generated in {time.time() - t0:.1f} s")

    def flops(self):
        return sum(3 * 2.0 * NV_M * N * K for _, K, N in NV_LAYERS)

    def step(self, tm):
        torch, fgs = self.torch, self.fgs
        for name, K, N in NV_LAYERS:
            X, W, dY = self.x[name], self.w[name], self.dy[name]
            qx = tm.run("quant", name + "/X", nvfp4_bytes(NV_M, K, 2), lambda: fgs.quantize_nvfp4(
                X, rowwise=True, colwise=True, rht_mask=2, rht_seed=self.rht_seed))
            qw = tm.run("quant", name + "/W", nvfp4_bytes(N, K, 2), lambda: fgs.quantize_nvfp4(
                W, rowwise=True, colwise=True))
            qdy = tm.run("quant", name + "/dY", nvfp4_bytes(NV_M, N, 2), lambda: fgs.quantize_nvfp4(
                dY, rowwise=True, colwise=True, rht_mask=2, rht_seed=self.rht_seed,
                stochastic=True, sr_seed=self.sr_seed))
            dense_gemm(tm, fgs, name + "/fwd", qx.rowwise(), qw.rowwise(), torch.bfloat16, self.out[(name, "y")])
            dense_gemm(tm, fgs, name + "/dgrad", qdy.rowwise(), qw.colwise(), torch.bfloat16, self.out[(name, "dx")])
            dense_gemm(tm, fgs, name + "/wgrad", qdy.colwise(), qx.colwise(), torch.float32, self.out[(name, "dw")])


WORKLOADS = {"llama3_8b": Llama8B, "hybrid8b": Hybrid8B, "tiny": Tiny, "moe": MoE, "mx405b": MX405B,
             "nv12b": NV12B, "llama3_8b_fp8mma": Llama8BFp8Mma, "mx405b_fp8mma": MX405BFp8Mma,
             "moe_fp8mma": MoEFp8Mma}


def measure(torch, wl, steps, warmup):
    """W untimed warm-up steps, then exactly `steps` timed steps between two
    device synchronisations; an event at every step boundary gives the
    per-step times."""
    for _ in range(warmup):
        wl.step(Timer(torch, enabled=False))
    torch.cuda.synchronize()
    tm = Timer(torch)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(steps):
        wl.step(tm)
        marks[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = [marks[i].elapsed_time(marks[i + 1]) * 1e-3 for i in range(steps)]
    kinds, labels = tm.summary()
    for (kind, label), (u, t, n) in labels.items():
        rate = f"{u / t / 1e12:8.1f} TFLOP/s" if kind == "gemm" else f"{u / t / 1e9:8.1f} GB/s"
        log(f"  {wl.name:28s} {label:24s} {t / n * 1e6:9.1f} us  {rate}  {tm.names.get(label, '')}")
    return wall, kinds, labels, step_s, tm


def step_stats(step_s):
    import numpy as np
    v = np.asarray(step_s) * 1e3
    return {"median": round(float(np.median(v)), 4), "p10": round(float(np.percentile(v, 10)), 4),
            "p90": round(float(np.percentile(v, 90)), 4), "mean": round(float(v.mean()), 4), "n": int(v.size)}


def kind_report(kinds, steps):
    out = {}
    if "gemm" in kinds:
        f, t, n = kinds["gemm"]
        out["gemm"] = {"TFLOP/s": round(f / t / 1e12, 2), "frac_fp16_mfma_peak": round(f / t / 1e12 / PEAK_FP16_MFMA, 4),
                       "frac_fp8_mfma_peak": round(f / t / 1e12 / PEAK_FP8_MFMA, 4),
                       "ms_per_step": round(t / steps * 1e3, 4)}
    if "quant" in kinds:
        b, t, n = kinds["quant"]
        out["quant"] = {"GB/s": round(b / t / 1e9, 1), "frac_hbm_peak": round(b / t / 1e9 / PEAK_HBM, 4),
                        "ms_per_step": round(t / steps * 1e3, 4)}
    return out


def instantiation_report(tm, steps):
    """Every GEMM kernel instantiation of a workload: launches per step, FLOPs
    per launch, average and median launch time, rate and its fraction of the
    matrix peak its instructions run at (FP8 for the FP8-instruction path, else
    FP16), and its share of the workload's GEMM time; sorted by share."""
    import numpy as np
    groups = {}
    for kind, label, units, t, name in tm.times():
        if kind != "gemm":
            continue
        g = groups.setdefault(name or label, {"flop": 0.0, "t": [], "labels": []})
        g["flop"] += units
        g["t"].append(t)
        if label not in g["labels"]:
            g["labels"].append(label)
    total = sum(sum(g["t"]) for g in groups.values()) or 1.0
    rows = []
    for name, g in groups.items():
        n, tt = len(g["t"]), sum(g["t"])
        rate = g["flop"] / tt / 1e12
        peak = PEAK_FP8_MFMA if name.endswith("true>") else PEAK_FP16_MFMA
        rows.append({"kernel": name, "launches_per_step": round(n / steps, 3),
                     "flop_per_launch": round(g["flop"] / n), "avg_us": round(tt / n * 1e6, 2),
                     "median_us": round(float(np.median(g["t"])) * 1e6, 2), "TFLOP/s": round(rate, 2),
                     "peak": peak, "frac_peak": round(rate / peak, 4), "share_of_gemm_time": round(tt / total, 4),
                     "launches": g["labels"]})
    rows.sort(key=lambda r: -r["share_of_gemm_time"])
    return rows


def quant_report(tm, steps, ceilings):
    """Quantizer rates per role (recipe / tensor, over the layers) and in
    total, against the HBM peak and the measured streaming ceilings."""
    groups = {}
    for kind, label, units, t, _ in tm.times():
        if kind != "quant":
            continue
        parts = label.split("/")
        key = "/".join([parts[0], parts[-1]]) if len(parts) > 2 else label
        b, tt = groups.get(key, (0.0, 0.0))
        groups[key] = (b + units, tt + t)
    out = {}
    for key, (b, tt) in sorted(groups.items()):
        r = b / tt / 1e9
        e = {"GB/s": round(r, 1), "frac_hbm_peak": round(r / PEAK_HBM, 4), "ms_per_step": round(tt / steps * 1e3, 4)}
        if ceilings:
            e["frac_copy_ceiling"] = round(r / ceilings["copy_GB/s"], 4)
            e["frac_read_ceiling"] = round(r / ceilings["read_GB/s"], 4)
        out[key] = e
    return out


def hbm_ceilings(torch, nbytes=1 << 30, reps=8):
    """What HBM sustains for this chip, measured by the in-tree streaming
    kernels (libfgs_hbm.so): a 1 GiB read reduced to one word per workgroup,
    and a 1 GiB copy (read + write bytes counted); each the best over the
    kernel variants (unroll depth, non-temporal access) and 1, 2, 4 or 8
    workgroups per compute unit, median of `reps` launches."""
    import ctypes
    import numpy as np
    if not os.path.exists(HBM_LIB):
        return None
    lib = ctypes.CDLL(HBM_LIB)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.fgs_hbm_read_grid.argtypes = [I32]
    lib.fgs_hbm_read.argtypes = [P, I64, P, I32, I32, P]
    lib.fgs_hbm_copy.argtypes = [P, P, I64, I32, I32, P]
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = {}
    for per_cu in (1, 2, 4, 8):
        out = torch.empty(lib.fgs_hbm_read_grid(per_cu), dtype=torch.int32, device="cuda")
        for variant in range(lib.fgs_hbm_variants()):
            for kind in ("read", "copy"):
                ts = []
                for r in range(reps + 2):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    if kind == "read":
                        rc = lib.fgs_hbm_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                              per_cu, variant, stream)
                    else:
                        rc = lib.fgs_hbm_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                              nbytes, per_cu, variant, stream)
                    e1.record()
                    if rc != 0:
                        raise RuntimeError(f"streaming kernel returned {rc}")
                    torch.cuda.synchronize()
                    if r >= 2:
                        ts.append(e0.elapsed_time(e1) * 1e-3)
                moved = nbytes * (1 if kind == "read" else 2)
                rate = moved / float(np.median(ts)) / 1e9
                if rate > best.get(kind, (0.0,))[0]:
                    best[kind] = (rate, per_cu, variant)
    del src, dst
    return {"read_GB/s": round(best["read"][0], 1), "read_config": {"workgroups_per_cu": best["read"][1],
                                                                    "variant": best["read"][2]},
            "copy_GB/s": round(best["copy"][0], 1), "copy_config": {"workgroups_per_cu": best["copy"][1],
                                                                    "variant": best["copy"][2]},
            "bytes": nbytes, "frac_hbm_peak_read": round(best["read"][0] / PEAK_HBM, 4),
            "frac_hbm_peak_copy": round(best["copy"][0] / PEAK_HBM, 4)}


# --------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters
# --------------------------------------------------------------------------
def gemm_source_digest():
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _kernel_short(name):
    name = name.replace("fgs::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0]


# the library's kernels (the counter tables leave out torch's and the bench's own)
LIB_KERNELS = ("gemm_block_scaled_kernel", "quant_", "amax_bf16", "nvfp4_", "delayed_scale_kernel")


def _counter_rows(d, counter):
    """{short kernel name: [per-dispatch values in KiB]} from a rocprofv3 --pmc
    csv directory."""
    out = {}
    files = [os.path.join(r, f) for r, _, fs in os.walk(d) for f in fs if f.endswith("counter_collection.csv")]
    if len(files) != 1:
        raise SystemExit(f"expected one *counter_collection.csv under {d}, found {len(files)}")
    with open(files[0], newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                out.setdefault(_kernel_short(row["Kernel_Name"]), []).append(float(row["Counter_Value"]))
    return out


def write_counter_profile(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, command, out=COUNTER_PROFILE):
    """Summarise FETCH_SIZE / WRITE_SIZE runs of the headline step (and of the
    1 GiB copy that calibrates both counters) into COUNTER_PROFILE, per kernel
    instantiation."""
    fetch, write = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")
    cf, cw = _counter_rows(cal_fetch_dir, "FETCH_SIZE"), _counter_rows(cal_write_dir, "WRITE_SIZE")
    copy = [k for k in cf if "copyBuffer" in k]
    if not copy:
        raise SystemExit("no copy kernel in the calibration runs")
    kib = CALIBRATION_BYTES / 1024.0
    f_fetch = kib / (sum(cf[copy[0]]) / len(cf[copy[0]]))
    f_write = kib / (sum(cw[copy[0]]) / len(cw[copy[0]]))
    lines = ["| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM bytes/dispatch (calibrated) |",
             "|---|---:|---:|---:|---:|"]
    kernels = {}
    for k in sorted(fetch):
        if not k.startswith(LIB_KERNELS):
            continue
        fv, wv = fetch[k], write.get(k, [])
        if len(fv) != len(wv):
            raise SystemExit(f"dispatch counts differ for {k}: {len(fv)} vs {len(wv)}")
        af, aw = sum(fv) / len(fv), sum(wv) / len(wv)
        fb, wb = 1024.0 * af * f_fetch, 1024.0 * aw * f_write
        lines.append(f"| `{k}` | {len(fv)} | {af:.1f} | {aw:.1f} | {(fb + wb) / 1e6:.2f} MB |")
        kernels[k] = {"dispatches": len(fv), "fetch_bytes_per_dispatch": round(fb), "write_bytes_per_dispatch": round(wb),
                      "traffic_bytes_per_dispatch": round(fb + wb)}
    if not any(k.startswith("gemm_block_scaled_kernel") for k in kernels):
        raise SystemExit("no gemm_block_scaled_kernel dispatches in the counter runs")
    summary = {"source_digest": gemm_source_digest(), "fetch_factor": round(f_fetch, 4),
               "write_factor": round(f_write, 4), "kernels": kernels}
    text = [
        "# HBM traffic of the headline step's kernels (rocprofv3 counters)",
        "",
        "Commands (repository root, one MI355X; each counter in a run of its own):",
        "",
        "```",
        *command,
        "```",
        "",
        f"Calibration: the 1 GiB device copy reads {kib / f_fetch:.1f} KiB of FETCH_SIZE and writes "
        f"{kib / f_write:.1f} KiB of WRITE_SIZE per dispatch, so FETCH_SIZE is scaled by {f_fetch:.4f} and "
        f"WRITE_SIZE by {f_write:.4f} to give bytes.",
        "",
        *lines,
        "",
        "Machine-readable summary (read by bench.py; `source_digest` is the SHA-256 prefix of the GEMM kernel's "
        "sources when the counters were taken, and bench.py reports traffic only while they still match):",
        "",
        "```json",
        json.dumps(summary),
        "```",
        "",
    ]
    with open(os.path.join(ROOT, out), "w") as f:
        f.write("\n".join(text))
    log(f"[bench] wrote {out}")


def _profile_json(path):
    """The machine-readable summary of a profile file, or None."""
    try:
        with open(os.path.join(ROOT, path)) as f:
            text = f.read()
        return json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None


def write_mfma_profile(csv_dir, command, out=MFMA_PROFILE):
    """Summarise a rocprofv3 --pmc run of MFMA_COUNTERS into MFMA_PROFILE, per
    GEMM kernel instantiation: MFMA busy (rocprof's MfmaUtil), the
    GUI-active clock the dispatches ran at, VALU and LDS instructions per
    MFMA, LDS bank conflicts."""
    files = [os.path.join(r, f) for r, _, fs in os.walk(csv_dir) for f in fs if f.endswith("counter_collection.csv")]
    if len(files) != 1:
        raise SystemExit(f"expected one *counter_collection.csv under {csv_dir}, found {len(files)}")
    agg = {}
    with open(files[0], newline="") as f:
        for row in csv.DictReader(f):
            k = _kernel_short(row["Kernel_Name"])
            if not k.startswith("gemm_block_scaled_kernel"):
                continue
            a = agg.setdefault(k, {"dur": {}, "c": {}})
            a["dur"][row["Dispatch_Id"]] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
            a["c"][row["Counter_Name"]] = a["c"].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    if not agg:
        raise SystemExit("no gemm_block_scaled_kernel dispatches in the counter run")
    lines = ["| kernel | dispatches | MFMA busy (rocprof MfmaUtil) | GUI-active clock | VALU per MFMA | "
             "LDS instr per MFMA | LDS bank conflicts |", "|---|---:|---:|---:|---:|---:|---:|"]
    kernels = {}
    for k, a in agg.items():
        c = a["c"]
        missing = [n for n in MFMA_COUNTERS if n not in c]
        if missing:
            raise SystemExit(f"counters missing for {k}: {missing}")
        gui = c["GRBM_GUI_ACTIVE"] / N_XCD              # the counter is summed over the XCDs
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * N_SIMD)
        clk = gui / sum(a["dur"].values()) / 1e9
        mf = c["SQ_INSTS_MFMA"]
        kernels[k] = {"dispatches": len(a["dur"]), "mfma_busy": round(busy, 4), "clock_ghz": round(clk, 3),
                      "valu_per_mfma": round(c["SQ_INSTS_VALU"] / mf, 3), "lds_per_mfma": round(c["SQ_INSTS_LDS"] / mf, 3),
                      "lds_bank_conflict_cycles": int(c["SQ_LDS_BANK_CONFLICT"])}
        lines.append(f"| `{k}` | {len(a['dur'])} | {100 * busy:.1f}% | {clk:.2f} GHz | {c['SQ_INSTS_VALU'] / mf:.2f} | "
                     f"{c['SQ_INSTS_LDS'] / mf:.2f} | {int(c['SQ_LDS_BANK_CONFLICT'])} |")
    clocks = [v["clock_ghz"] for v in kernels.values()]
    summary = {"source_digest": gemm_source_digest(), "kernels": kernels}
    text = [
        "# MFMA utilisation of the GEMM kernels (rocprofv3 counters)",
        "",
        "Command (repository root, one MI355X; one counter pass: 7 SQ counters and 1 GRBM counter):",
        "",
        "```",
        *command,
        "```",
        "",
        "The run is one warm-up and one timed step of the Llama-3-8B linears in both recipes on the exact path",
        "(`..., false>`), then the same step with every GEMM on the FP8 instructions (`..., true>`).",
        "",
        "How the columns are computed (summed over each kernel's dispatches):",
        "- **MFMA busy** is rocprof's `MfmaUtil`: `SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)`.",
        "  The counter file reports `GRBM_GUI_ACTIVE` summed over the 8 XCDs.",
        "- **GUI-active clock** is the per-XCD active cycle count divided by the dispatches' measured duration. It",
        "  is the clock the kernel ran at: the part is power-limited under sustained MFMA load, below its 2.4 GHz",
        "  maximum.",
        "- **VALU per MFMA** is the counter ratio `SQ_INSTS_VALU / SQ_INSTS_MFMA`, over the whole kernel (prologue and",
        "  epilogue included).",
        "  - In the exact path's K loop the VALU work is the FP16 decode and the promotion FMAs. On the 16x16",
        "    output tiles of the promoted 256 x 256 tile, an MFMA does a quarter of a 32x32 one's work, so the ratio",
        "    is not comparable across tile shapes.",
        "  - The 1x128 x 1x128 wgrad promotes with two scale factors per output.",
        "- **LDS bank conflicts** are `SQ_LDS_BANK_CONFLICT` cycles.",
        "",
        *lines,
        "",
        "Reading:",
        "- The exact per-tensor GEMM keeps the matrix units about 70% busy on the 256 x 256 tile (60% on the 256 x 128",
        "  tile) at the clock it runs at. Its K loop decodes half a k-step ahead of the MFMAs.",
        "- The promoted blockwise GEMM is about 52% busy on the 256 x 256 tile (16x16 output tiles) and about 49% on",
        "  the 1x128 x 1x128 wgrad's 256 x 128 tile. There, decode and promotion work exceeds what co-issues with the",
        "  MFMAs: the wgrad promotes with two scale factors per output, after each block's last k-step.",
        "- The FP8-instruction path reaches 45-52% at twice the FLOPs per busy cycle, except for its narrow-tile",
        "  1x128 x 1x128 wgrad, where promotion dominates.",
        "- There are no LDS bank conflicts in any kernel.",
        "",
        "The busy fractions are a property of the kernels and repeat from box to box; the clock (this run's",
        f"GUI-active clocks: {min(clocks):.2f}-{max(clocks):.2f} GHz) does not. The busier the matrix units, the lower",
        "the clock the part sustains, and the step's TFLOP/s follows the clock. bench.py reports the dominant",
        "instantiation's busy fraction and clock from this file, and its rate against the peak at that clock, while",
        "the GEMM sources still match the digest below.",
        "",
        "Machine-readable summary (read by bench.py; `source_digest` is the SHA-256 prefix of the GEMM kernel's "
        "sources when the counters were taken):",
        "",
        "```json",
        json.dumps(summary),
        "```",
        "",
    ]
    with open(os.path.join(ROOT, out), "w") as f:
        f.write("\n".join(text))
    log(f"[bench] wrote {out}")


def read_kernel_mfma(kernel, path=MFMA_PROFILE):
    """MFMA busy fraction and clock of one GEMM instantiation from
    MFMA_PROFILE, or None when the file is missing, holds no such kernel, or
    the GEMM kernel's sources changed since the counters were taken."""
    summary = _profile_json(path)
    if not summary or summary.get("source_digest") != gemm_source_digest():
        return None
    return summary.get("kernels", {}).get(kernel)


def read_kernel_traffic(kernel, path=COUNTER_PROFILE):
    """HBM bytes per dispatch of one kernel instantiation from
    COUNTER_PROFILE, or None when the file is missing, holds no such kernel,
    or the GEMM kernel's sources changed since the counters were taken."""
    summary = _profile_json(path)
    if not summary or summary.get("source_digest") != gemm_source_digest():
        return None
    return summary.get("kernels", {}).get(kernel)


def gpu_clocks():
    """Current shader and memory clock levels of the first AMD GPU, read from
    the amdgpu driver's DPM tables in sysfs (the level marked '*'); plain file
    reads, no child process.  None where the files are absent."""
    import glob
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
            out = {}
            for key in ("sclk", "mclk"):
                with open(os.path.join(dev, f"pp_dpm_{key}")) as f:
                    cur = [ln.split(":", 1)[1].strip(" *\n") for ln in f if ln.rstrip().endswith("*")]
                out[key] = cur[0] if cur else None
            return out
        except (OSError, IndexError):
            continue
    return None


def _cpu_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def _host_threads():
    """The host threads this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS where that is set (the GPU machine's CPU share)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        n = min(n, int(os.environ["OMP_NUM_THREADS"]))
    except (KeyError, ValueError):
        pass
    return max(1, n)


def _oracle_quant(pool, bits, mode, colwise, chunks):
    """The oracle's FP32-scaled E4M3 quantization of `bits`, split into
    128-row chunks run in parallel (bit-identical to one call: 1x128 tiles,
    128x128 blocks and the column-wise 128x1 tiles never cross a 128-row
    boundary; per-tensor scaling takes the tensor amax first, then quantizes
    each chunk with that amax as its only history entry, which is the same
    scale)."""
    import numpy as np
    import oracle
    rows = bits.shape[0]
    step = max(128, -(-rows // chunks) // 128 * 128)
    bounds = [(r, min(rows, r + step)) for r in range(0, rows, step)]
    axis = 1 if colwise else 0
    if mode == "tensor":
        am = max(pool.map(lambda b: int(np.max(bits[b[0]:b[1]] & 0x7FFF)), bounds))
        hist = np.array([am << 16], dtype=np.uint32).view(np.float32)
        parts = list(pool.map(lambda b: oracle.quant_delayed(bits[b[0]:b[1]], "e4m3", hist, colwise=colwise), bounds))
        return np.concatenate([p[0] for p in parts], axis=axis), np.array([[parts[0][1]]], dtype=np.float32)
    parts = list(pool.map(lambda b: oracle.quant_e4m3(bits[b[0]:b[1]], mode, colwise=colwise), bounds))
    return np.concatenate([p[0] for p in parts], axis=axis), np.concatenate([p[1] for p in parts], axis=axis)


def _oracle_sample(x, w, dy, threads):
    """One pass of the oracle over the sample: X, W, dY quantized row- and
    column-wise in both recipes, dequantized, and the three FP64 products."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with ThreadPoolExecutor(max_workers=threads) as pool, threadpool_limits(threads):
        for _, amode, wmode in RECIPES:
            qx, sx = _oracle_quant(pool, x, amode, False, threads)
            qxt, sxt = _oracle_quant(pool, x, amode, True, threads)
            qw, sw = _oracle_quant(pool, w, wmode, False, threads)
            qwt, swt = _oracle_quant(pool, w, wmode, True, threads)
            qd, sd = _oracle_quant(pool, dy, amode, False, threads)
            qdt, sdt = _oracle_quant(pool, dy, amode, True, threads)
            oracle.gemm_ref(oracle.dequant_e4m3(qx, sx, amode), oracle.dequant_e4m3(qw, sw, wmode))
            oracle.gemm_ref(oracle.dequant_e4m3(qd, sd, amode), oracle.dequant_e4m3(qwt, swt, wmode))
            oracle.gemm_ref(oracle.dequant_e4m3(qdt, sdt, amode), oracle.dequant_e4m3(qxt, sxt, amode))


def cpu_baseline(tokens=512):
    """The oracle, untuned, on a bounded sample of the headline workload: the
    QKV layer (K = 4096, N = 6144) with M cut to `tokens` tokens, both
    recipes: oracle quantization of X, W, dY (row-wise and column-wise,
    plain C, run in 128-row chunks on every host thread) and the three FP64
    numpy GEMMs (BLAS on every host thread); then the same on one thread.
    Reported in the metric's unit (GEMM TFLOP/s of the sample)."""
    from fine_grained_scaled_amd import synth
    K, N = 4096, 6144
    x = synth.activations(LLAMA8B_M, K, seed=0, tag=synth.TAG_A + 16, row_range=(0, tokens))
    w = synth.weights(N, K, seed=0, tag=synth.TAG_W + 16)
    dy = synth.gradients(LLAMA8B_M, N, seed=0, tag=synth.TAG_DY + 16, row_range=(0, tokens))
    flops = len(RECIPES) * 3 * 2.0 * tokens * N * K
    threads = _host_threads()
    t0 = time.perf_counter()
    _oracle_sample(x, w, dy, threads)
    dt = time.perf_counter() - t0
    t0 = time.perf_counter()
    _oracle_sample(x, w, dy, 1)
    dt1 = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"QKV layer (K=4096, N=6144) with M={tokens} of 8192 tokens, both recipes: oracle "
                       f"quantization (plain C in 128-row chunks) of X, W, dY row- and column-wise, dequantization "
                       f"and 3 FP64 numpy GEMMs per recipe; {threads} host threads, {dt:.1f} s wall"),
            "seconds": round(dt, 2),
            "single_thread": {"value": round(flops / dt1 / 1e12, 6), "seconds": round(dt1, 2)},
            "nproc": os.cpu_count(), "cpu_model": _cpu_info()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 12 timed steps keep the headline's timed region above 200 ms
    ap.add_argument("--steps", type=int, default=12)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", default="llama3_8b,hybrid8b,tiny,moe,mx405b,nv12b,llama3_8b_fp8mma,mx405b_fp8mma,moe_fp8mma",
                    help="comma list of " + ",".join(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference kernel that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--write-counter-profile", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="summarise four rocprofv3 --pmc csv directories (FETCH_SIZE and WRITE_SIZE of one headline "
                         "step, then of --copy-calibration) into " + COUNTER_PROFILE + " and exit (no GPU needed)")
    ap.add_argument("--counter-command", action="append", default=[],
                    help="command line recorded in the counter or MFMA profile (repeatable)")
    ap.add_argument("--write-mfma-profile", metavar="CSV_DIR",
                    help="summarise a rocprofv3 --pmc csv directory of the MFMA counters (" + " ".join(MFMA_COUNTERS) +
                         ") into " + MFMA_PROFILE + " and exit (no GPU needed)")
    ap.add_argument("--only", default=None,
                    help="comma list of workloads to run alone (no headline, no CPU baseline), reported on "
                         "stderr: for profiling runs")
    ap.add_argument("--gemm-only", action="store_true",
                    help="headline workload: quantize once, then time only the GEMM launches "
                         "(for counter collection on the GEMM kernel)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path has no cross-GPU exchange; run --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.write_counter_profile:
        write_counter_profile(*args.write_counter_profile, args.counter_command)
        return
    if args.write_mfma_profile:
        write_mfma_profile(args.write_mfma_profile, args.counter_command)
        return

    import torch
    import fine_grained_scaled_amd as fgs
    from fine_grained_scaled_amd import _lib, synth
    _lib.load()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 1 GiB 5 times (counter calibration)")
        return
    if args.gemm_only:
        head = Llama8B(torch, fgs, synth)
        head.gemm_only(args.steps)
        return
    log(f"[bench] device {torch.cuda.get_device_name(0)}; steps {args.steps} warmup {args.warmup}")
    names = [n for n in args.workloads.split(",") if n]
    if args.only:
        for n in args.only.split(","):
            wl = WORKLOADS[n](torch, fgs, synth)
            w_wall, w_kinds, _, w_steps, w_tm = measure(torch, wl, args.steps, args.warmup)
            log(f"[bench] {wl.name}: {kind_report(w_kinds, args.steps)}; step {step_stats(w_steps)}")
            del wl
            torch.cuda.empty_cache()
        return

    ceilings = hbm_ceilings(torch)
    log(f"[bench] HBM ceilings (in-tree streaming kernels): {ceilings}")

    head = Llama8B(torch, fgs, synth)
    clocks_before = gpu_clocks()
    wall, kinds, _, step_s, tm = measure(torch, head, args.steps, args.warmup)
    clocks_after = gpu_clocks()
    ms = wall * 1e3 / args.steps
    value = head.flops() / (wall / args.steps) / 1e12
    rep = kind_report(kinds, args.steps)
    inst = instantiation_report(tm, args.steps)
    quant = dict(rep.get("quant") or {})
    if ceilings:
        quant["frac_copy_ceiling"] = round(quant["GB/s"] / ceilings["copy_GB/s"], 4)
        quant["frac_read_ceiling"] = round(quant["GB/s"] / ceilings["read_GB/s"], 4)
    quant["roles"] = quant_report(tm, args.steps, ceilings)
    log(f"[bench] {head.name}: step {ms:.2f} ms, {value:.1f} TFLOP/s; {rep}")
    for r in inst:
        log(f"[bench]   {r['kernel']}: {r['launches_per_step']} launches/step, {r['avg_us']} us avg, "
            f"{r['TFLOP/s']} TFLOP/s = {r['frac_peak']} of peak, {r['share_of_gemm_time']} of GEMM time")

    extra = {}
    for n in names:
        if n == "llama3_8b":
            continue
        wl = WORKLOADS[n](torch, fgs, synth)
        w_wall, w_kinds, w_labels, w_steps, w_tm = measure(torch, wl, args.steps, args.warmup)
        r = kind_report(w_kinds, args.steps)
        r["ms_per_step"] = round(w_wall * 1e3 / args.steps, 4)
        r["step_ms"] = step_stats(w_steps)
        r["step_TFLOP/s"] = round(wl.flops() / (w_wall / args.steps) / 1e12, 2)
        if not isinstance(wl, MoE):
            r["instantiations"] = [{k: v for k, v in e.items() if k != "launches"}
                                   for e in instantiation_report(w_tm, args.steps)]
        if ceilings and "quant" in r:
            r["quant"]["frac_copy_ceiling"] = round(r["quant"]["GB/s"] / ceilings["copy_GB/s"], 4)
        if isinstance(wl, MoE):
            f, t, _ = w_kinds["gemm"]
            # forward (gate/up N=4096 K=7168, down N=7168 K=2048) and dgrad
            # (down N=2048 K=7168, gate/up N=7168 K=4096) on the row groups;
            # wgrad (dW [7168 x 2048] down, [4096 x 7168] gate/up) on the
            # token groups
            shapes = [(2 * MOE_INTER, MOE_HIDDEN), (MOE_HIDDEN, MOE_INTER), (MOE_INTER, MOE_HIDDEN),
                      (MOE_HIDDEN, 2 * MOE_INTER)]
            wshapes = [(MOE_HIDDEN, MOE_INTER), (2 * MOE_INTER, MOE_HIDDEN)]
            roof_rows = sum(wl.roofline_seconds(n, k) for n, k in shapes)
            roof_w = sum(wl.wgrad_roofline_seconds(m, n) for m, n in wshapes)
            by = sum(wl.gemm_bytes(n, k) for n, k in shapes) + sum(wl.wgrad_bytes(m, n) for m, n in wshapes)
            gemm_s = t / args.steps
            r["gemm"]["roofline_ms"] = round(float(roof_rows + roof_w) * 1e3, 4)
            r["gemm"]["frac_roofline"] = round(float(roof_rows + roof_w) / gemm_s, 4)
            r["gemm"]["GB/s"] = round(by / gemm_s / 1e9, 1)
            tw = sum(tt for (kind, lab), (_, tt, _) in w_labels.items() if kind == "gemm" and "wgrad" in lab)
            tw /= args.steps
            wby = sum(wl.wgrad_bytes(m, n) for m, n in wshapes)
            r["wgrad"] = {"ms_per_step": round(tw * 1e3, 4), "roofline_ms": round(float(roof_w) * 1e3, 4),
                          "frac_roofline": round(float(roof_w) / tw, 4), "GB/s": round(wby / tw / 1e9, 1)}
            tr = gemm_s - tw
            r["fwd_dgrad"] = {"ms_per_step": round(tr * 1e3, 4), "roofline_ms": round(float(roof_rows) * 1e3, 4),
                              "frac_roofline": round(float(roof_rows) / tr, 4)}
        log(f"[bench] {wl.name}: {r}")
        extra[wl.name] = r
        del wl
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample (CPU) ...")
        cpu = cpu_baseline()
        log(f"[bench] oracle sample: {cpu['value']} TFLOP/s; {cpu['sample']}; one thread "
            f"{cpu['single_thread']['value']} TFLOP/s ({cpu['single_thread']['seconds']} s)")

    g = rep["gemm"]
    dom = inst[0]
    # algorithmic bytes per launch of the dominant instantiation (its launches'
    # operand codes, scales and output, once each), and the HBM traffic its
    # dispatches made in the committed counter runs of the same sources
    shapes = {lab: (M, N, K, am, bm, dt) for lab, M, N, K, am, bm, dt in head.gemm_launches()}
    dl = [shapes[lab] for lab in dom["launches"]]
    alg = sum(head.gemm_bytes_one(M, N, K, am, bm, 2 if dt == torch.bfloat16 else 4) for M, N, K, am, bm, dt in dl) / len(dl)
    tr = read_kernel_traffic(dom["kernel"])
    traffic = tr["traffic_bytes_per_dispatch"] if tr else None
    if traffic is None:
        log(f"[bench] no traffic for {dom['kernel']}: {COUNTER_PROFILE} missing, without it, or taken on other sources")
    # its MFMA busy fraction and sustained clock in the committed counter run,
    # and this run's rate against the peak at that clock
    mf = read_kernel_mfma(dom["kernel"])
    at_clock = None
    if mf:
        at_clock = {"mfma_busy": mf["mfma_busy"], "clock_ghz": mf["clock_ghz"],
                    "peak_at_clock": round(PEAK_FP16_MFMA * mf["clock_ghz"] / MAX_SCLK_GHZ, 1),
                    "frac_at_clock": round(dom["TFLOP/s"] / (PEAK_FP16_MFMA * mf["clock_ghz"] / MAX_SCLK_GHZ), 4),
                    "source": MFMA_PROFILE}
    else:
        log(f"[bench] no MFMA profile for {dom['kernel']}: {MFMA_PROFILE} missing, without it, or taken on other sources")
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": step_stats(step_s),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 codes, fp16 mfma, fp32 accumulate",
        "data": "synthetic (seeded BF16: activations N(0,1) with x50 outlier channels, weights N(0,0.02), "
                "gradients Student-t(3) std 1e-3; each layer its own tensors, "
                f"{len(head.sets)} input sets in rotation, {head.input_bytes() / 2**30:.2f} GiB)",
        "config": {"workload": "llama3-8b linear layers fwd+dgrad+wgrad, blockwise 1x128/128x128 and per-tensor E4M3",
                   "tokens": LLAMA8B_M, "layers": {n: [K, N] for n, K, N in LLAMA8B_LAYERS},
                   "recipes": [r[0] for r in RECIPES], "step_gemm_tflop": round(head.flops() / 1e12, 4),
                   "input_sets": len(head.sets)},
        "roofline": {"bound": "mfma", "achieved": dom["TFLOP/s"], "peak": PEAK_FP16_MFMA, "unit": "TFLOP/s",
                     "frac": round(dom["TFLOP/s"] / PEAK_FP16_MFMA, 4), "traffic": traffic,
                     "kernel": dom["kernel"], "launches_per_step": dom["launches_per_step"],
                     "flop_per_launch": dom["flop_per_launch"], "avg_launch_us": dom["avg_us"],
                     "share_of_gemm_time": dom["share_of_gemm_time"],
                     "algorithmic_bytes_per_launch": round(alg),
                     "frac_of_fp8_peak": round(dom["TFLOP/s"] / PEAK_FP8_MFMA, 4),
                     "at_profiled_clock": at_clock},
        "gemm": dict(g, instantiations=[{k: v for k, v in e.items() if k != "launches"} for e in inst],
                     dominant=dom["kernel"]),
        "quant": quant,
        "hbm_ceiling": ceilings,
        "workloads": extra,
        "cpu_baseline": cpu,
        "clocks": {"before": clocks_before, "after": clocks_after},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
