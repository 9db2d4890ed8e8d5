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

X's two copies are also timed as separate calls (nvfp4_quantize row copy,
nvfp4_rht_quantize RN) after the step, with the dgrad path and the
MXFP4 / FP8 comparisons.

Prints one JSON line. `value` is the step's effective GEMM rate: the two
GEMMs' 2*M*N*K flops divided by the whole step time (quantizers included).
Per-call times come from HIP events recorded on the stream the library uses
(torch's current stream) inside the timed region. `cpu_baseline` times the
CPU oracle on a bounded slice of the same workload.
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

# HBM traffic per GEMM launch comes from the committed counter summary below
# (null when it is missing or the GEMM source changed since it was taken).
TRAFFIC_SUMMARY = "linear_layer_traffic.md"
# Kernels of each call, as (short-name fragment, dispatch index within one
# step) in the counter summary: a quantize call is an amax kernel and a
# quantize kernel; a GEMM call launches 256 x 256 tiles and, for a last
# partial round, 128 x 128 ones.
CALL_KERNELS = {
    "quantize_x_row_rht": (("amax_tile_kernel<unsigned short, true, false, true>", 0),
                           ("quantize_kernel<unsigned short, 3, false>", 0)),
    "quantize_w_16x16": (("amax_flat_kernel<unsigned short>", 0),
                         ("quantize_kernel<unsigned short, 1, false>", 0)),
    "rht_quantize_dy_sr": (("amax_tile_kernel<unsigned short, true, false, false>", 0),
                           ("quantize_kernel<unsigned short, 2, true>", 0)),
    "gemm_fprop": (("gemm_kernel<4, false, true,", 0), ("gemm_kernel<2, false, true,", 0)),
    "gemm_wgrad": (("gemm_kernel<4, false, false,", 0), ("gemm_kernel<2, false, false,", 0)),
    # the dgrad path, run after the step
    "quantize_dy_1x16_sr": (("amax_flat_kernel<unsigned short>", 1),
                            ("quantize_rows_kernel<unsigned short, true>", 0)),
    "gemm_dgrad": (("gemm_kernel<4, false, true,", 1), ("gemm_kernel<2, false, true,", 1)),
    # X's two copies as separate calls, and its RHT copy with SR (after the step)
    "quantize_x_1x16": (("amax_flat_kernel<unsigned short>", 2),
                        ("quantize_rows_kernel<unsigned short, false>", 0)),
    "rht_quantize_x_rn": (("amax_tile_kernel<unsigned short, true, false, false>", 1),
                          ("quantize_kernel<unsigned short, 2, false>", 0)),
    "rht_quantize_x_sr": (("amax_tile_kernel<unsigned short, true, false, false>", 2),
                          ("quantize_kernel<unsigned short, 2, true>", 1)),
    "mx_quantize_x": (("mx_quantize_kernel<unsigned short>", 0),),
    "mx_quantize_w": (("mx_quantize_kernel<unsigned short>", 1),),
    "mx_gemm_fprop": (("block_gemm_kernel<(Fmt)0", 0),),
    "fp8_quantize_x": (("amax_flat_kernel<unsigned short>", 3),
                       ("fp8_quantize_kernel<unsigned short>", 0)),
    "fp8_quantize_w": (("amax_flat_kernel<unsigned short>", 4),
                       ("fp8_quantize_kernel<unsigned short>", 1)),
    "fp8_quantize_dy": (("amax_flat_kernel<unsigned short>", 5),
                        ("fp8_quantize_kernel<unsigned short>", 2)),
    "fp8_gemm_fprop": (("block_gemm_kernel<(Fmt)1", 0),),
    "fp8_gemm_wgrad": (("block_gemm_kernel<(Fmt)1", 1),),
}


def _call_source(name):
    if name.startswith("mx_gemm") or name.startswith("fp8_gemm"):
        return "f8f6f4_gemm"
    if name.startswith("mx_"):
        return "mxfp4"
    if name.startswith("fp8_"):
        return ("fp8", "quantize_kernel")  # its amax pass is the NVFP4 quantizer's
    return "gemm_kernel" if name.startswith("gemm") else "quantize_kernel"


CALL_SOURCE = {n: _call_source(n) for n in CALL_KERNELS}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the dgrad calls timed after the step (they share the fprop GEMM's "
                         "kernel, whose per-kernel profile statistics would then mix both)")
    ap.add_argument("--tokens", type=int, default=TOKENS)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one copy-like kernel (torch.bitwise_not on int32) "
                         "over this many MiB, the reference for the traffic counters")
    return ap.parse_args()


class Step:
    """Pre-allocated operands and outputs of one linear-layer step."""

    def __init__(self, torch, nv, x_np, w_np, dy_np):
        self.torch, self.nv = torch, nv
        dev = "cuda"
        u8 = torch.uint8
        t, h = x_np.shape
        f = w_np.shape[0]
        self.t, self.h, self.f = t, h, f
        bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
        self.x, self.w, self.dy = bf(x_np), bf(w_np), bf(dy_np)
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
        """The dgrad path, timed apart from the step (it is not one of the
        step's rows): the SR row copy of dY and dX = deq(Q_SR(dY)) deq(Q2D(W))."""
        nv = self.nv
        s = self
        return [
            ("quantize_dy_1x16_sr", lambda: nv.nvfp4_quantize(
                s.dy, nv.BLOCK_1D, nv.ROUND_SR, 7, s.offset, nv.OUT_ROW, None, s.adyr, s.qdyr,
                s.sdyr, None, None, s.tdyr, s.status)),
            ("gemm_dgrad", lambda: nv.nvfp4_gemm(
                s.qdyr, s.sdyr, s.tdyr, nv.BLOCK_1D, s.qwt, s.swt, s.tw, nv.BLOCK_2D, s.t, s.h,
                s.f, s.dx)),
        ]

    def variant_calls(self):
        """X's two copies as separate calls (the row copy, then the RHT RN
        copy), and its RHT copy with SR (the recipe rounds activations to
        nearest; the library offers both), timed apart from the step into the
        step's own X-copy buffers after the step's GEMMs have read them."""
        nv = self.nv
        s = self
        return [
            ("quantize_x_1x16", lambda: nv.nvfp4_quantize(
                s.x, nv.BLOCK_1D, nv.ROUND_RN, 0, 0, nv.OUT_ROW, None, s.ax, s.qx, s.sx, None,
                None, s.tx, s.status)),
            ("rht_quantize_x_rn", lambda: nv.nvfp4_rht_quantize(
                s.x, 7, nv.ROUND_RN, 0, 0, None, s.axt, s.qxt, s.sxt, s.txt, s.status)),
            ("rht_quantize_x_sr", lambda: nv.nvfp4_rht_quantize(
                s.x, 7, nv.ROUND_SR, 7, s.offset, None, s.axt, s.qxt, s.sxt, s.txt, s.status)),
        ]

    def mx_calls(self):
        """The MXFP4 comparison path, timed apart from the step."""
        nv = self.nv
        s = self
        return [
            ("mx_quantize_x", lambda: nv.mxfp4_quantize(s.x, s.mqx, s.msx)),
            ("mx_quantize_w", lambda: nv.mxfp4_quantize(s.w, s.mqw, s.msw)),
            ("mx_gemm_fprop", lambda: nv.mxfp4_gemm(s.mqx, s.msx, s.mqw, s.msw, s.t, s.f, s.h,
                                                    s.y)),
        ]

    def fp8_calls(self):
        """The FP8 baseline (fprop and wgrad), timed apart from the step."""
        nv = self.nv
        s = self
        return [
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
        q1 = 0.5 + 1.0 / 16  # codes + 1x16 scale bytes per element
        return {
            "quantize_x_row_rht": ("GB/s", t * h * (2 + 2 + 2 * q1)),
            "quantize_x_1x16": ("GB/s", t * h * (2 + 2 + q1)),
            "quantize_w_16x16": ("GB/s", f * h * (2 + 2 + 2 * (0.5 + 1.0 / 256))),
            "rht_quantize_dy_sr": ("GB/s", t * f * (2 + 2 + q1)),
            "rht_quantize_x_rn": ("GB/s", t * h * (2 + 2 + q1)),
            "gemm_fprop": ("TFLOP/s", 2.0 * t * f * h),
            "gemm_wgrad": ("TFLOP/s", 2.0 * f * h * t),
            "quantize_dy_1x16_sr": ("GB/s", t * f * (2 + 2 + q1)),
            "rht_quantize_x_sr": ("GB/s", t * h * (2 + 2 + q1)),
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


def cpu_baseline():
    """The oracle on a bounded slice of the step: 4096 tokens, the first
    10240 rows of W; same operations and seeds. Returns its effective TFLOP/s."""
    import numpy as np

    import oracle as o
    import workloads as wl

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    t, h, f = 4096, HIDDEN, 10240
    x = wl.normal((t, h), seed=5, outlier_channels=16)
    w = wl.weight(f, h, seed=2)
    dy = wl.laplace((t, f), seed=6)
    t0 = time.perf_counter()
    qx = o.quantize(x, outputs=("row",))["row"]
    qw = o.quantize_2d(w)
    qdy = o.rht_quantize(dy, 7, rounding="sr", seed=7)
    qxt = o.rht_quantize(x, 7, rounding="rn")
    o.gemm(qx.codes, qx.scales, qx.tensor_scale, "1d", qw["row"].codes, qw["row"].scales,
           qw["row"].tensor_scale, "2d")
    o.gemm(qdy.codes, qdy.scales, qdy.tensor_scale, "1d", qxt.codes, qxt.scales, qxt.tensor_scale,
           "1d")
    dt = time.perf_counter() - t0
    flops = 2 * (2.0 * t * f * h)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"one linear-layer step of the oracle at tokens={t}, hidden={h}, ffn={f} "
                  f"(first {f} rows of the weight); elementwise numpy single-threaded, float64 "
                  f"BLAS matmul with {blas_threads} threads; {dt:.1f} s; value = the two GEMMs' "
                  f"flops / step time",
        "seconds": dt,
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
    }


def hbm_copy_reference(torch, reps):
    """The streaming rate a plain device-to-device copy reaches on this GPU:
    torch's copy_ between two 1 GiB buffers (ROCm's copy kernel), bytes read
    plus bytes written per average HIP-event duration. A reference for the
    quantizers' fractions of the 8 TB/s peak, not a measurement of them."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(max(reps, 1))]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / len(ev)
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
    torch.mm(a, b, out=out)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(max(reps, 1))]
    for e0, e1 in ev:
        e0.record()
        torch.mm(a, b, out=out)
        e1.record()
    torch.cuda.synchronize()
    us = 1e3 * sum(e0.elapsed_time(e1) for e0, e1 in ev) / len(ev)
    del a, b, out
    rate = 2.0 * t * h * f / (us * 1e-6) / 1e12
    return {"TFLOP/s": round(rate, 1), "frac": round(rate / MFMA_PEAK_TFLOPS, 4),
            "us": round(us, 1),
            "what": f"torch.mm bf16 [{t},{h}] x [{h},{f}], random operands (ROCm BLAS)"}


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

    nv.load()
    torch.cuda.set_device(0)
    t = args.tokens
    x_np, w_np, dy_np = wl.linear_layer(tokens=t)
    step = Step(torch, nv, x_np, w_np, dy_np)
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
        step.offset += 1
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
        step.offset += 1
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert int(step.status.cpu()[0]) == 0, "non-finite amax"

    # the dgrad path, after the timed step and outside it
    next_calls = [] if args.no_next else (step.next_calls() + step.variant_calls() + step.mx_calls()
                                          + step.fp8_calls())
    for _ in range(min(args.warmup, 1)):
        for _, fn in next_calls:
            fn()
    next_events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in next_calls] for _ in range(args.steps)]
    for k in range(args.steps):
        for i, (_, fn) in enumerate(next_calls):
            next_events[k][i][0].record()
            fn()
            next_events[k][i][1].record()
    torch.cuda.synchronize()
    assert int(step.status.cpu()[0]) == 0, "non-finite amax"
    copy_ref = hbm_copy_reference(torch, args.steps)
    gemm_ref = dense_gemm_reference(torch, args.steps, t, HIDDEN, FFN)

    ms_step = elapsed * 1e3 / args.steps
    work = step.work()
    from bit_block_scaled_bf16_amd import profiling

    summary = os.path.join(ROOT, "profiles", TRAFFIC_SUMMARY)

    def call_stats(call_list, evs):
        res = {}
        for i, (name, _) in enumerate(call_list):
            ms = [evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps)]
            avg_ms = float(np.mean(ms))
            unit, amount = work[name]
            if unit == "GB/s":
                rate = amount / (avg_ms * 1e-3) / 1e9
                peak = HBM_PEAK_GBS
            else:
                rate = amount / (avg_ms * 1e-3) / 1e12
                peak = (FP4_MFMA_PEAK_TFLOPS if unit.startswith("FP4") else
                        FP8_MFMA_PEAK_TFLOPS if unit.startswith("FP8") else MFMA_PEAK_TFLOPS)
            traffic = profiling.kernel_traffic(summary, CALL_KERNELS[name], CALL_SOURCE[name])
            res[name] = {"us": round(avg_ms * 1e3, 2), "achieved": round(rate, 1), "unit": unit,
                         "frac": round(rate / peak, 4), "work": amount, "traffic": traffic,
                         # the counted HBM bytes over the same time (null with traffic)
                         "traffic_GB/s": (round(traffic / (avg_ms * 1e-3) / 1e9, 1)
                                          if traffic is not None else None)}
        return res

    kernels = call_stats(calls, events)
    next_rows = call_stats(next_calls, next_events)

    gemm_flops = work["gemm_fprop"][1] + work["gemm_wgrad"][1]
    value = gemm_flops / (ms_step * 1e-3) / 1e12
    q_names = [n for n in kernels if kernels[n]["unit"] == "GB/s"]
    q_bytes = sum(work[n][1] for n in q_names)
    q_us = sum(kernels[n]["us"] for n in q_names)
    g_us = kernels["gemm_fprop"]["us"] + kernels["gemm_wgrad"]["us"]
    dom = max(("gemm_fprop", "gemm_wgrad"), key=lambda n: kernels[n]["us"])
    traffic = kernels[dom]["traffic"]
    roofline = {
        "bound": "mfma",
        "kernel": dom,
        "achieved": kernels[dom]["achieved"],
        "peak": MFMA_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": kernels[dom]["frac"],
        "traffic": traffic,
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
        },
        "quantize": {"GB/s": round(q_bytes / (q_us * 1e-6) / 1e9, 1),
                     "frac": round(q_bytes / (q_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "us": round(q_us, 1)},
        "gemm": {"TFLOP/s": round(gemm_flops / (g_us * 1e-6) / 1e12, 1),
                 "frac": round(gemm_flops / (g_us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                 "us": round(g_us, 1)},
        "kernels": kernels,
        "next": ({"dgrad": {k: v for k, v in next_rows.items()
                            if k in ("quantize_dy_1x16_sr", "gemm_dgrad")},
                  "variants": {k: v for k, v in next_rows.items()
                               if k in ("quantize_x_1x16", "rht_quantize_x_rn",
                                        "rht_quantize_x_sr")},
                  "mxfp4": {k: v for k, v in next_rows.items() if k.startswith("mx_")},
                  "fp8": {k: v for k, v in next_rows.items() if k.startswith("fp8_")}}
                 if next_rows else None),
        "roofline": roofline,
        "hbm_copy": copy_ref,
        "dense_bf16_gemm": gemm_ref,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
