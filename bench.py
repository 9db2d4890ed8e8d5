"""Benchmark: one NVFP4 linear-layer step (fprop + weight gradient) on one GPU.

Workload (synthetic stand-ins for a linear layer of the 12B hybrid model of
"Pretraining Large Language Models with NVFP4"): X bf16 [16384, 5120]
N(0,1) with 16 outlier channels x20, W bf16 [20480, 5120] N(0, 0.02^2),
dY bf16 [16384, 20480] Laplace(0, 1e-3). One step runs the whole hot path:

  1. nvfp4_quantize_row_rht(X)  both amaxes, then in one read: 1x16 RN row
                                copy (fprop A) and RHT + 16x1 RN (wgrad B)
  2. nvfp4_quantize(W)          tensor amax + 16x16 RN, W and W^T (fprop B)
  3. nvfp4_rht_quantize(dY)     RHT amax + RHT + 16x1 SR (Philox seed 7)
  4. nvfp4_gemm fprop           Y  [16384, 20480] = X W^T,  K = 5120,  bf16
  5. nvfp4_gemm wgrad           dW [20480, 5120] = dY^T X,  K = 16384, bf16

Two sets of input tensors alternate from step to step, so every call reads
inputs that the rest of a step (about 2 GB of traffic) has pushed out of the
caches. After the timed steps, and outside `value`: the dgrad path, X's two
copies as separate calls, the MXFP4 and FP8 comparisons, the workload
configurations c1-c4 and the dequantizer as standalone calls on rotated
input copies (`next.configs`), hand-written streaming read and copy kernels
(the memory system's rate for a kernel with no arithmetic), torch's copy and
bf16 GEMM as references, and the CPU oracle per call.

Prints one JSON line. `value` is the step's effective GEMM rate: the two
GEMMs' 2*M*N*K flops divided by the whole step time (quantizers included).
Per-call times come from HIP events recorded on the stream the library uses
(torch's current stream) inside the timed region. `traffic` (HBM bytes from
the FETCH_SIZE / WRITE_SIZE counters) and `counters` (VALU / MFMA busy)
come from the committed summaries in profiles/ and are null once the kernel
source has changed since they were taken. They are regenerated with:

  NEXT=mx_quantize_x,mx_quantize_w,mx_gemm_fprop,fp8_quantize_x,fp8_quantize_w,\
fp8_quantize_dy,fp8_gemm_fprop,fp8_gemm_wgrad
  rocprofv3 --kernel-trace --stats -d <d> -o run --output-format csv -- \
      python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --next-only $NEXT
  rocprofv3 --pmc FETCH_SIZE -d <d1> -o run --output-format csv -- \
      python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --next-only $NEXT \
      --copy-calibration-mib 1024
  rocprofv3 --pmc WRITE_SIZE -d <d2> ... (same command)
  rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_WAVES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU \
      SQ_INSTS_VALU SQ_INSTS_MFMA -d <d3> -o run --output-format csv -- \
      python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --next-only $NEXT
  python -m bit_block_scaled_bf16_amd.profiling stats|traffic|counters ...
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NVFP4 quantize GB/s (% HBM peak) + NVFP4 GEMM TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 MFMA, MI355X
FP4_MFMA_PEAK_TFLOPS = 10100.0  # dense FP4 MFMA (the MXFP4 comparison GEMM), MI355X
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense FP8 MFMA (the FP8 baseline GEMMs), MI355X

TOKENS, HIDDEN, FFN = 16384, 5120, 20480

# Committed counter summaries (profiles/): HBM traffic per call and busy
# fractions, each guarded by the SHA-256 of the kernel sources they cover.
TRAFFIC_SUMMARY = "linear_layer_traffic.md"
COUNTERS_SUMMARY = "linear_layer_counters.md"
# Kernels of each call, as (short-name fragment, dispatch index) in a
# profiled `--steps 1` run: a quantize call is an amax kernel and a
# quantize kernel; a GEMM call launches 256 x 256 tiles and, for a last
# partial round, 128 x 128 ones.
CALL_KERNELS = {
    "quantize_x_row_rht": (("rht_amax_mfma_kernel<true>", 0),
                           ("rht_quantize_mfma_kernel<true, false,", 0)),
    "quantize_w_16x16": (("amax_flat_kernel<unsigned short>", 0),
                         ("quantize_kernel<unsigned short, 1, false>", 0)),
    "rht_quantize_dy_sr": (("rht_amax_mfma_kernel<false>", 0),
                           ("rht_quantize_mfma_kernel<false, true,", 0)),
    "gemm_fprop": (("gemm_kernel<4, false, true,", 0), ("gemm_kernel<2, false, true,", 0)),
    "gemm_wgrad": (("gemm_kernel<4, false, false,", 0), ("gemm_kernel<2, false, false,", 0)),
}
CALL_SOURCE = {n: ("gemm_kernel" if n.startswith("gemm") else "quantize_kernel")
               for n in CALL_KERNELS}
# The same for calls after the step, in a profiled run with `--next-only`
# naming them: each runs once untimed, then once per timed round, in the
# order next_calls() lists them (so the two FP8 GEMMs alternate).
NEXT_KERNELS = {
    "mx_quantize_x": (("mx_quantize_kernel<unsigned short>", 2),),
    "mx_quantize_w": (("mx_quantize_kernel<unsigned short>", 3),),
    "mx_gemm_fprop": (("block_gemm_kernel<(Fmt)0", 1),),
    "fp8_gemm_fprop": (("block_gemm_kernel<(Fmt)1", 2),),
    "fp8_gemm_wgrad": (("block_gemm_kernel<(Fmt)1", 3),),
}
NEXT_SOURCE = {n: ("mxfp4" if n.startswith("mx_quantize") else "block_gemm_kernel")
               for n in NEXT_KERNELS}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="time only the step (profiling runs: the later calls share its kernels)")
    ap.add_argument("--next-only", default="",
                    help="comma-separated names of calls after the step: time only these, "
                         "and none of the later blocks (profiling runs of those kernels)")
    ap.add_argument("--tokens", type=int, default=TOKENS)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one copy-like kernel (torch.bitwise_not on int32) "
                         "over this many MiB, the reference for the traffic counters")
    return ap.parse_args()


def _q1(n):
    """Bytes of a 1x16 NVFP4 copy of n elements: codes + scale bytes."""
    return n * (0.5 + 1.0 / 16)


class Step:
    """Operands and outputs of one linear-layer step; `sets` copies of the
    inputs alternate from step to step."""

    def __init__(self, torch, nv, x_np, w_np, dy_np, sets=2):
        self.torch, self.nv = torch, nv
        dev = "cuda"
        u8 = torch.uint8
        t, h = x_np.shape
        f = w_np.shape[0]
        self.t, self.h, self.f = t, h, f
        bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
        x, w, dy = bf(x_np), bf(w_np), bf(dy_np)
        self.xs, self.ws, self.dys = [x], [w], [dy]
        for _ in range(sets - 1):
            self.xs.append(x.clone())
            self.ws.append(w.clone())
            self.dys.append(dy.clone())
        self.k = 0  # input set of the next step
        sc = lambda: torch.zeros(4, dtype=torch.float32, device=dev)
        ws = lambda: nv.amax_workspace(dev)
        e = lambda *s: torch.empty(s, dtype=u8, device=dev)
        # X row copy (fprop A)
        self.qx, self.sx, self.tx, self.ax = e(t, h // 2), e(t, h // 16), sc(), ws()
        # W 16x16: W and W^T codes, grid and grid^T
        self.qw, self.sw, self.qwt, self.swt = e(f, h // 2), e(f // 16, h // 16), e(h, f // 2), e(h // 16, f // 16)
        self.tw, self.aw = sc(), ws()
        # RHT copies (wgrad operands), stored [cols][tokens/2]
        self.qdy, self.sdy, self.tdy, self.ady = e(f, t // 2), e(f, t // 16), sc(), ws()
        self.qxt, self.sxt, self.txt, self.axt = e(h, t // 2), e(h, t // 16), sc(), ws()
        # dgrad: SR row copy of dY (A) and dX = dY W, whose B operand is W^T's copy
        self.qdyr, self.sdyr, self.tdyr, self.adyr = e(t, f // 2), e(t, f // 16), sc(), ws()
        self.dx = torch.empty((t, h), dtype=torch.bfloat16, device=dev)
        # MXFP4 comparison: X and W in 1x32 blocks, fprop on the FP4 MFMA
        self.mqx, self.msx = e(t, h // 2), e(t, h // 32)
        self.mqw, self.msw = e(f, h // 2), e(f, h // 32)
        # FP8 baseline (E4M3, per tensor): X row + column copies, W row copy,
        # dY column copy; fprop Y = X W^T and wgrad dW = dY^T X
        self.fx, self.fxt, self.ftx, self.fax = e(t, h), e(h, t), sc(), ws()
        self.fw, self.ftw, self.faw = e(f, h), sc(), ws()
        self.fdyt, self.ftdy, self.fady = e(f, t), sc(), ws()
        self.y = torch.empty((t, f), dtype=torch.bfloat16, device=dev)
        self.dw = torch.empty((f, h), dtype=torch.bfloat16, device=dev)
        self.status = torch.zeros(4, dtype=torch.int32, device=dev)
        self.offset = 0

    def advance(self):
        self.k = (self.k + 1) % len(self.xs)
        self.offset += 1

    @property
    def x(self):
        return self.xs[self.k]

    @property
    def w(self):
        return self.ws[self.k]

    @property
    def dy(self):
        return self.dys[self.k]

    def calls(self):
        nv = self.nv
        s = self
        return [
            ("quantize_x_row_rht", lambda: nv.nvfp4_quantize_row_rht(
                s.x, 7, nv.ROUND_RN, 0, 0, None, s.ax, s.qx, s.sx, s.tx, s.qxt, s.sxt, s.txt,
                s.status)),
            ("quantize_w_16x16", lambda: nv.nvfp4_quantize(
                s.w, nv.BLOCK_2D, nv.ROUND_RN, 0, 0, nv.OUT_ROW | nv.OUT_COL, None, s.aw, s.qw,
                s.sw, s.qwt, s.swt, s.tw, s.status)),
            ("rht_quantize_dy_sr", lambda: nv.nvfp4_rht_quantize(
                s.dy, 7, nv.ROUND_SR, 7, s.offset, None, s.ady, s.qdy, s.sdy, s.tdy, s.status)),
            ("gemm_fprop", lambda: nv.nvfp4_gemm(
                s.qx, s.sx, s.tx, nv.BLOCK_1D, s.qw, s.sw, s.tw, nv.BLOCK_2D, s.t, s.f, s.h,
                s.y)),
            ("gemm_wgrad", lambda: nv.nvfp4_gemm(
                s.qdy, s.sdy, s.tdy, nv.BLOCK_1D, s.qxt, s.sxt, s.txt, nv.BLOCK_1D, s.f, s.h,
                s.t, s.dw)),
        ]

    def next_calls(self):
        """Timed after the step, outside `value`: the dgrad path (the SR row
        copy of dY and dX = deq(Q_SR(dY)) deq(Q2D(W))), X's two copies as
        separate calls and its RHT copy with SR (the recipe rounds
        activations to nearest; the library offers both), the MXFP4
        comparison and the FP8 baseline."""
        nv = self.nv
        s = self
        return [
            ("quantize_dy_1x16_sr", lambda: nv.nvfp4_quantize(
                s.dy, nv.BLOCK_1D, nv.ROUND_SR, 7, s.offset, nv.OUT_ROW, None, s.adyr, s.qdyr,
                s.sdyr, None, None, s.tdyr, s.status)),
            ("gemm_dgrad", lambda: nv.nvfp4_gemm(
                s.qdyr, s.sdyr, s.tdyr, nv.BLOCK_1D, s.qwt, s.swt, s.tw, nv.BLOCK_2D, s.t, s.h,
                s.f, s.dx)),
            ("quantize_x_1x16", lambda: nv.nvfp4_quantize(
                s.x, nv.BLOCK_1D, nv.ROUND_RN, 0, 0, nv.OUT_ROW, None, s.ax, s.qx, s.sx, None,
                None, s.tx, s.status)),
            ("rht_quantize_x_rn", lambda: nv.nvfp4_rht_quantize(
                s.x, 7, nv.ROUND_RN, 0, 0, None, s.axt, s.qxt, s.sxt, s.txt, s.status)),
            ("rht_quantize_x_sr", lambda: nv.nvfp4_rht_quantize(
                s.x, 7, nv.ROUND_SR, 7, s.offset, None, s.axt, s.qxt, s.sxt, s.txt, s.status)),
            ("mx_quantize_x", lambda: nv.mxfp4_quantize(s.x, s.mqx, s.msx)),
            ("mx_quantize_w", lambda: nv.mxfp4_quantize(s.w, s.mqw, s.msw)),
            ("mx_gemm_fprop", lambda: nv.mxfp4_gemm(s.mqx, s.msx, s.mqw, s.msw, s.t, s.f, s.h,
                                                    s.y)),
            ("fp8_quantize_x", lambda: nv.fp8_quantize(s.x, nv.OUT_ROW | nv.OUT_COL, None, s.fax,
                                                       s.fx, s.fxt, s.ftx, s.status)),
            ("fp8_quantize_w", lambda: nv.fp8_quantize(s.w, nv.OUT_ROW, None, s.faw, s.fw, None,
                                                       s.ftw, s.status)),
            ("fp8_quantize_dy", lambda: nv.fp8_quantize(s.dy, nv.OUT_COL, None, s.fady, None,
                                                        s.fdyt, s.ftdy, s.status)),
            ("fp8_gemm_fprop", lambda: nv.fp8_gemm(s.fx, s.ftx, s.fw, s.ftw, s.t, s.f, s.h, s.y)),
            ("fp8_gemm_wgrad", lambda: nv.fp8_gemm(s.fdyt, s.ftdy, s.fxt, s.ftx, s.f, s.h, s.t,
                                                   s.dw)),
        ]

    def work(self):
        """Algorithmic bytes (quantizer calls, amax pass included) or flops."""
        t, h, f = self.t, self.h, self.f
        return {
            "quantize_x_row_rht": ("GB/s", t * h * 4 + 2 * _q1(t * h)),
            "quantize_x_1x16": ("GB/s", t * h * 4 + _q1(t * h)),
            "quantize_w_16x16": ("GB/s", f * h * (2 + 2 + 2 * (0.5 + 1.0 / 256))),
            "rht_quantize_dy_sr": ("GB/s", t * f * 4 + _q1(t * f)),
            "rht_quantize_x_rn": ("GB/s", t * h * 4 + _q1(t * h)),
            "gemm_fprop": ("TFLOP/s", 2.0 * t * f * h),
            "gemm_wgrad": ("TFLOP/s", 2.0 * f * h * t),
            "quantize_dy_1x16_sr": ("GB/s", t * f * 4 + _q1(t * f)),
            "rht_quantize_x_sr": ("GB/s", t * h * 4 + _q1(t * h)),
            "gemm_dgrad": ("TFLOP/s", 2.0 * t * h * f),
            # MXFP4: one pass (no tensor amax): bf16 in, codes + 1/32 scale bytes out
            "mx_quantize_x": ("GB/s", t * h * (2 + 0.5 + 1.0 / 32)),
            "mx_quantize_w": ("GB/s", f * h * (2 + 0.5 + 1.0 / 32)),
            "mx_gemm_fprop": ("FP4 TFLOP/s", 2.0 * t * f * h),
            # FP8: amax pass + quantize pass over bf16, one byte out per copy
            "fp8_quantize_x": ("GB/s", t * h * (2 + 2 + 2)),
            "fp8_quantize_w": ("GB/s", f * h * (2 + 2 + 1)),
            "fp8_quantize_dy": ("GB/s", t * f * (2 + 2 + 1)),
            "fp8_gemm_fprop": ("FP8 TFLOP/s", 2.0 * t * f * h),
            "fp8_gemm_wgrad": ("FP8 TFLOP/s", 2.0 * f * h * t),
        }


def time_calls(torch, call_list, reps, rotate=None):
    """Average microseconds of each call over `reps` rounds (HIP events on the
    current stream), after one untimed round. rotate() runs between rounds."""
    for _, fn in call_list:
        fn()
    if rotate:
        rotate()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in call_list] for _ in range(reps)]
    for k in range(reps):
        for i, (_, fn) in enumerate(call_list):
            evs[k][i][0].record()
            fn()
            evs[k][i][1].record()
        if rotate:
            rotate()
    torch.cuda.synchronize()
    return {name: 1e3 * sum(evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(reps)) / reps
            for i, (name, _) in enumerate(call_list)}


def rate_row(us, amount, unit, peak, traffic=None):
    per_s = amount / (us * 1e-6)
    achieved = per_s / (1e9 if unit.endswith("GB/s") else 1e12)
    row = {"us": round(us, 2), "achieved": round(achieved, 1), "unit": unit,
           "frac": round(achieved / peak, 4), "work": amount}
    if traffic is not None or unit == "GB/s":
        row["traffic"] = traffic
        row["traffic_GB/s"] = round(traffic / (us * 1e-6) / 1e9, 1) if traffic is not None else None
    return row


def config_rows(torch, nv, reps):
    """The workload configurations as standalone calls. Each input is cloned
    into enough copies that the copies a call cycles through total more than
    512 MB (twice the 256 MB Infinity Cache), so no call reads its input from
    a cache that the previous call filled. Amax-supplied rows pass the
    tensor's true amax (computed once, before timing) and time the quantize
    pass alone."""
    import workloads as wl

    dev = "cuda"
    u8 = torch.uint8
    e = lambda *s: torch.empty(s, dtype=u8, device=dev)
    sc = lambda: torch.zeros(4, dtype=torch.float32, device=dev)
    status = torch.zeros(4, dtype=torch.int32, device=dev)
    ws = nv.amax_workspace(dev)
    rows = {}

    def copies(a_np, dtype, min_total=1 << 29):
        t = torch.from_numpy(a_np).to(dtype).to(dev)
        n = max(1, -(-min_total // (t.numel() * t.element_size())))
        return [t] + [t.clone() for _ in range(n - 1)]

    def amax_of(t):
        return torch.tensor([float(t.float().abs().max()), 0, 0, 0], dtype=torch.float32,
                            device=dev)

    def run(name, fns, amount, unit="GB/s", peak=HBM_PEAK_GBS):
        state = {"i": 0}

        def call():
            fns[state["i"] % len(fns)]()

        def rotate():
            state["i"] += 1

        us = time_calls(torch, [(name, call)], reps, rotate)[name]
        rows[name] = rate_row(us, amount, unit, peak)
        rows[name]["copies"] = len(fns)

    # c1: fp32 256 x 1024, 1x16 RN quantize, then dequantize (launch-bound)
    x1 = torch.from_numpy(wl.fp32_outlier_matrix()).to(dev)
    q1, s1, t1 = e(256, 512), e(256, 64), sc()
    y1 = torch.empty((256, 1024), dtype=torch.float32, device=dev)
    run("c1_quantize_fp32_256x1024_rn", [lambda: nv.nvfp4_quantize(
        x1, nv.BLOCK_1D, nv.ROUND_RN, 0, 0, nv.OUT_ROW, None, ws, q1, s1, None, None, t1, status)],
        256 * 1024 * (4 + 4) + _q1(256 * 1024))
    run("c1_dequantize_fp32_256x1024", [lambda: nv.nvfp4_dequantize(
        q1, s1, t1, 256, 1024, nv.BLOCK_1D, y1)], _q1(256 * 1024) + 256 * 1024 * 4)
    del x1, y1

    # c2: bf16 activation 8192 x 5120, row + column copies from one read
    r, c = 8192, 5120
    xs = copies(wl.activation(r, c, seed=1), torch.bfloat16)
    a2 = amax_of(xs[0])
    q2r, s2r, q2c, s2c, t2 = e(r, c // 2), e(r, c // 16), e(c, r // 2), e(c, r // 16), sc()
    mk = lambda x, amax, w: (lambda: nv.nvfp4_quantize(
        x, nv.BLOCK_1D, nv.ROUND_RN, 0, 0, nv.OUT_ROW | nv.OUT_COL, amax, w, q2r, s2r, q2c, s2c,
        t2, status))
    run("c2_dual_rn_8192x5120", [mk(x, None, ws) for x in xs], r * c * 4 + 2 * _q1(r * c))
    run("c2_dual_rn_8192x5120_amax_in", [mk(x, a2, None) for x in xs], r * c * 2 + 2 * _q1(r * c))
    del xs

    # c3: bf16 weight 20480 x 5120, 16x16 blocks, both orientations
    r, c = 20480, 5120
    wts = copies(wl.weight(r, c, seed=2), torch.bfloat16)
    a3 = amax_of(wts[0])
    q3, s3, q3t, s3t, t3 = e(r, c // 2), e(r // 16, c // 16), e(c, r // 2), e(c // 16, r // 16), sc()
    mk = lambda x, amax, w: (lambda: nv.nvfp4_quantize(
        x, nv.BLOCK_2D, nv.ROUND_RN, 0, 0, nv.OUT_ROW | nv.OUT_COL, amax, w, q3, s3, q3t, s3t,
        t3, status))
    two_d = r * c * 2 * (0.5 + 1.0 / 256)
    run("c3_2d_rn_20480x5120", [mk(x, None, ws) for x in wts], r * c * 4 + two_d)
    run("c3_2d_rn_20480x5120_amax_in", [mk(x, a3, None) for x in wts], r * c * 2 + two_d)
    del wts

    # c4: wgrad inputs, RHT (seed 7) + 16x1: dY 8192 x 20480 with SR (Philox
    # seed 7), X 8192 x 5120 with RN
    r, c = 8192, 20480
    dys = copies(wl.gradient(r, c, seed=3), torch.bfloat16)
    q4, s4, t4 = e(c, r // 2), e(c, r // 16), sc()
    run("c4_rht_sr_dy_8192x20480", [
        (lambda x=x: nv.nvfp4_rht_quantize(x, 7, nv.ROUND_SR, 7, 0, None, ws, q4, s4, t4, status))
        for x in dys], r * c * 4 + _q1(r * c))
    # the transformed tensor's amax, from the call itself
    a4 = torch.zeros(4, dtype=torch.float32, device=dev)
    a4[0] = ws[0]
    run("c4_rht_sr_dy_8192x20480_amax_in", [
        (lambda x=x: nv.nvfp4_rht_quantize(x, 7, nv.ROUND_SR, 7, 0, a4, None, q4, s4, t4, status))
        for x in dys], r * c * 2 + _q1(r * c))
    del dys
    r, c = 8192, 5120
    xs = copies(wl.wgrad_activation(r, c, seed=4), torch.bfloat16)
    q5, s5, t5 = e(c, r // 2), e(c, r // 16), sc()
    run("c4_rht_rn_x_8192x5120", [
        (lambda x=x: nv.nvfp4_rht_quantize(x, 7, nv.ROUND_RN, 0, 0, None, ws, q5, s5, t5, status))
        for x in xs], r * c * 4 + _q1(r * c))
    del xs
    assert int(status[0]) == 0, "non-finite amax"
    return rows


def dequant_rows(torch, nv, step, reps):
    """c5's operands back to bf16: X's row copy [16384, 5120] and W's 16x16
    copy [20480, 5120] (reads codes and scale bytes, writes 2 bytes per
    element)."""
    t, h, f = step.t, step.h, step.f
    yx = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
    yw = torch.empty((f, h), dtype=torch.bfloat16, device="cuda")
    calls = [("dequantize_x_1x16_bf16", lambda: step.nv.nvfp4_dequantize(
                 step.qx, step.sx, step.tx, t, h, step.nv.BLOCK_1D, yx)),
             ("dequantize_w_16x16_bf16", lambda: step.nv.nvfp4_dequantize(
                 step.qw, step.sw, step.tw, f, h, step.nv.BLOCK_2D, yw))]
    us = time_calls(torch, calls, reps)
    out = {"dequantize_x_1x16_bf16": rate_row(us["dequantize_x_1x16_bf16"], _q1(t * h) + 2 * t * h,
                                              "GB/s", HBM_PEAK_GBS),
           "dequantize_w_16x16_bf16": rate_row(us["dequantize_w_16x16_bf16"],
                                               f * h * (0.5 + 1.0 / 256 + 2), "GB/s", HBM_PEAK_GBS)}
    del yx, yw
    return out


def stream_rows(torch, nv, reps):
    """The hand-written streaming references over 1 GiB: read only
    (nvfp4_stream_read) and read + write (nvfp4_stream_copy)."""
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(nv._lib.STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    us = time_calls(torch, [("read", lambda: nv.nvfp4_stream_read(src, n, sink)),
                            ("copy", lambda: nv.nvfp4_stream_copy(src, dst, n))], reps)
    del src, dst
    out = {}
    for name, nbytes in (("read", n), ("copy", 2 * n)):
        rate = nbytes / (us[name] * 1e-6) / 1e9
        out[name] = {"GB/s": round(rate, 1), "frac": round(rate / HBM_PEAK_GBS, 4),
                     "us": round(us[name], 1), "bytes": nbytes}
    return out


def hbm_copy_reference(torch, reps):
    """torch's copy_ between two 1 GiB buffers (ROCm's copy kernel), bytes
    read plus bytes written per average HIP-event duration."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    us = time_calls(torch, [("copy", lambda: dst.copy_(src))], reps)["copy"]
    del src, dst
    rate = 2 * n / (us * 1e-6) / 1e9
    return {"GB/s": round(rate, 1), "frac": round(rate / HBM_PEAK_GBS, 4), "us": round(us, 1),
            "bytes": 2 * n, "what": "torch copy_ of a 1 GiB device buffer (read + write)"}


def dense_gemm_reference(torch, reps, t, h, f):
    """What ROCm's BLAS reaches on a plain bf16 GEMM of the fprop shape
    (torch.mm of contiguous random [t, h] and [h, f] operands, fp32
    accumulation): a reference for the NVFP4 GEMM's fraction of the dense
    MFMA peak, not a measurement of it."""
    a = torch.randn(t, h, device="cuda").to(torch.bfloat16)
    b = torch.randn(h, f, device="cuda").to(torch.bfloat16)
    out = torch.empty(t, f, device="cuda", dtype=torch.bfloat16)
    us = time_calls(torch, [("mm", lambda: torch.mm(a, b, out=out))], reps)["mm"]
    del a, b, out
    rate = 2.0 * t * h * f / (us * 1e-6) / 1e12
    return {"TFLOP/s": round(rate, 1), "frac": round(rate / MFMA_PEAK_TFLOPS, 4),
            "us": round(us, 1),
            "what": f"torch.mm bf16 [{t},{h}] x [{h},{f}], random operands (ROCm BLAS)"}


CPU_TOKENS, CPU_FFN = 4096, 8192


def cpu_baseline(x_np, w_np, dy_np):
    """The oracle, call by call, on a fixed slice of the step's own input
    tensors: X[:4096] (4096 x 5120), W[:8192] (8192 x 5120) and
    dY[:4096, :8192], i.e. one linear-layer step at tokens 4096, ffn 8192.
    Each call's rate uses the same algorithmic bytes / flops as the GPU rows;
    `value` is the slice step's effective GEMM rate, like the GPU's."""
    import numpy as np

    import oracle as o

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    t, h, f = CPU_TOKENS, x_np.shape[1], CPU_FFN
    xs, wsl = x_np[:t], w_np[:f]
    dys = np.ascontiguousarray(dy_np[:t, :f])
    timings = {}

    def timed(name, fn):
        t0 = time.perf_counter()
        out = fn()
        timings[name] = time.perf_counter() - t0
        return out

    qx = timed("quantize_x_1x16", lambda: o.quantize(xs, outputs=("row",))["row"])
    qxt = timed("rht_quantize_x_rn", lambda: o.rht_quantize(xs, 7, rounding="rn"))
    qw = timed("quantize_w_16x16", lambda: o.quantize_2d(wsl))["row"]
    qdy = timed("rht_quantize_dy_sr", lambda: o.rht_quantize(dys, 7, rounding="sr", seed=7))
    timed("gemm_fprop", lambda: o.gemm(qx.codes, qx.scales, qx.tensor_scale, "1d", qw.codes,
                                       qw.scales, qw.tensor_scale, "2d"))
    timed("gemm_wgrad", lambda: o.gemm(qdy.codes, qdy.scales, qdy.tensor_scale, "1d", qxt.codes,
                                       qxt.scales, qxt.tensor_scale, "1d"))
    work = {
        "quantize_x_1x16": ("GB/s", t * h * 4 + _q1(t * h)),
        "rht_quantize_x_rn": ("GB/s", t * h * 4 + _q1(t * h)),
        "quantize_w_16x16": ("GB/s", f * h * (2 + 2 + 2 * (0.5 + 1.0 / 256))),
        "rht_quantize_dy_sr": ("GB/s", t * f * 4 + _q1(t * f)),
        "gemm_fprop": ("TFLOP/s", 2.0 * t * f * h),
        "gemm_wgrad": ("TFLOP/s", 2.0 * f * h * t),
    }
    calls = {}
    for name, sec in timings.items():
        unit, amount = work[name]
        rate = amount / sec / (1e9 if unit == "GB/s" else 1e12)
        calls[name] = {"seconds": round(sec, 3), "achieved": round(rate, 4), "unit": unit}
    total = sum(timings.values())
    flops = work["gemm_fprop"][1] + work["gemm_wgrad"][1]
    return {
        "value": flops / total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"the oracle call by call on a slice of the step's own tensors: X[:{t}], "
                  f"W[:{f}], dY[:{t}, :{f}] (a linear-layer step at tokens={t}, hidden={h}, "
                  f"ffn={f}); elementwise numpy single-threaded, float64 BLAS matmul with "
                  f"{blas_threads} threads; {total:.1f} s; value = the two GEMMs' flops / the "
                  f"slice step's time",
        "calls": calls,
        "seconds": round(total, 3),
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: a data-parallel "
              "run would shard the tokens and reduce the weight gradient across GPUs, which this "
              "library does not do", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import bit_block_scaled_bf16_amd as nv
    import workloads as wl
    from bit_block_scaled_bf16_amd import profiling

    nv.load()
    torch.cuda.set_device(0)
    t = args.tokens
    x_np, w_np, dy_np = wl.linear_layer(tokens=t)
    step = Step(torch, nv, x_np, w_np, dy_np)
    if args.no_cpu_baseline:
        del x_np, w_np, dy_np
    calls = step.calls()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
        step.advance()
    torch.cuda.synchronize()

    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in calls] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for i, (_, fn) in enumerate(calls):
            events[k][i][0].record()
            fn()
            events[k][i][1].record()
        step.advance()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert int(step.status.cpu()[0]) == 0, "non-finite amax"

    ms_step = elapsed * 1e3 / args.steps
    work = step.work()
    profiles = os.path.join(ROOT, "profiles")
    traffic_md = os.path.join(profiles, TRAFFIC_SUMMARY)
    counters_md = os.path.join(profiles, COUNTERS_SUMMARY)

    kernels = {}
    for i, (name, _) in enumerate(calls):
        us = 1e3 * float(np.mean([events[k][i][0].elapsed_time(events[k][i][1])
                                  for k in range(args.steps)]))
        unit, amount = work[name]
        peak = HBM_PEAK_GBS if unit == "GB/s" else MFMA_PEAK_TFLOPS
        traffic = profiling.kernel_traffic(traffic_md, CALL_KERNELS[name], CALL_SOURCE[name])
        kernels[name] = rate_row(us, amount, unit, peak, traffic)
        kernels[name]["traffic"] = traffic
        kernels[name]["traffic_GB/s"] = (round(traffic / (us * 1e-6) / 1e9, 1)
                                         if traffic is not None else None)
        kernels[name]["counters"] = profiling.kernel_counters(counters_md, CALL_KERNELS[name],
                                                              CALL_SOURCE[name])

    next_block = None
    if not args.no_next:
        reps = max(args.steps, 5)
        nxt = step.next_calls()
        only = [n for n in args.next_only.split(",") if n]
        if only:
            unknown = set(only) - {n for n, _ in nxt}
            if unknown:
                sys.exit(f"--next-only: unknown calls {sorted(unknown)}")
            nxt = [c for c in nxt if c[0] in only]
        us = time_calls(torch, nxt, reps, rotate=step.advance)
        rows = {}
        for name, _ in nxt:
            unit, amount = work[name]
            peak = (FP4_MFMA_PEAK_TFLOPS if unit.startswith("FP4") else
                    FP8_MFMA_PEAK_TFLOPS if unit.startswith("FP8") else
                    HBM_PEAK_GBS if unit == "GB/s" else MFMA_PEAK_TFLOPS)
            traffic = (profiling.kernel_traffic(traffic_md, NEXT_KERNELS[name], NEXT_SOURCE[name])
                       if name in NEXT_KERNELS else None)
            rows[name] = rate_row(us[name], amount, unit, peak, traffic)
            if name in NEXT_KERNELS:
                rows[name]["counters"] = profiling.kernel_counters(
                    counters_md, NEXT_KERNELS[name], NEXT_SOURCE[name])
        assert int(step.status.cpu()[0]) == 0, "non-finite amax"
    if not args.no_next and only:
        next_block = {"selected": rows}
    elif not args.no_next:
        next_block = {
            "dgrad": {k: rows[k] for k in ("quantize_dy_1x16_sr", "gemm_dgrad")},
            "variants": {k: rows[k] for k in ("quantize_x_1x16", "rht_quantize_x_rn",
                                              "rht_quantize_x_sr")},
            "mxfp4": {k: v for k, v in rows.items() if k.startswith("mx_")},
            "fp8": {k: v for k, v in rows.items() if k.startswith("fp8_")},
            "dequantize": dequant_rows(torch, nv, step, reps),
        }
        # the step's tensors are no longer needed: room for the config copies
        del step
        torch.cuda.empty_cache()
        next_block["configs"] = config_rows(torch, nv, reps)
        next_block["stream"] = stream_rows(torch, nv, reps)
        next_block["hbm_copy"] = hbm_copy_reference(torch, reps)
        next_block["dense_bf16_gemm"] = dense_gemm_reference(torch, reps, t, HIDDEN, FFN)

    gemm_flops = work["gemm_fprop"][1] + work["gemm_wgrad"][1]
    value = gemm_flops / (ms_step * 1e-3) / 1e12
    q_names = [n for n in kernels if kernels[n]["unit"] == "GB/s"]
    q_bytes = sum(work[n][1] for n in q_names)
    q_us = sum(kernels[n]["us"] for n in q_names)
    g_us = kernels["gemm_fprop"]["us"] + kernels["gemm_wgrad"]["us"]
    dom = max(("gemm_fprop", "gemm_wgrad"), key=lambda n: kernels[n]["us"])
    roofline = {
        "bound": "mfma",
        "kernel": dom,
        "achieved": kernels[dom]["achieved"],
        "peak": MFMA_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": kernels[dom]["frac"],
        "traffic": kernels[dom]["traffic"],
    }
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands (e2m1 x e4m3, exact in f16), f16 MFMA, f32 accumulate; f32 quantizer",
        "data": "synthetic",
        "config": {
            "workload": f"nvfp4_linear_layer_fprop_wgrad tokens={t} hidden={HIDDEN} ffn={FFN}",
            "x": "bf16 N(0,1), 16 outlier channels x20, seed 5",
            "w": "bf16 N(0,0.02^2), seed 2, 16x16 blocks",
            "dy": "bf16 Laplace(0,1e-3), seed 6, RHT seed 7, SR Philox seed 7",
            "input_sets": 2,
        },
        "quantize": {"GB/s": round(q_bytes / (q_us * 1e-6) / 1e9, 1),
                     "frac": round(q_bytes / (q_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "us": round(q_us, 1)},
        "gemm": {"TFLOP/s": round(gemm_flops / (g_us * 1e-6) / 1e12, 1),
                 "frac": round(gemm_flops / (g_us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                 "us": round(g_us, 1)},
        "kernels": kernels,
        "next": next_block,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x_np, w_np, dy_np)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
