#!/usr/bin/env python3
"""Benchmark of the quantized-GEMM hot path on one MI355X.

One step is one pass of every kernel of the path over one batch of
synthetic, HBM-resident inputs: weight preparation and the decode-sized
GEMMs first, the prefill GEMM last:

  1. quantize_rows   fp16 fused-QKV weight [12288, 4096] -> int8 codes + fp16 scales
  2. gemm w8a8       those codes, M = 64 (streaming matrix-core path)
  3. pack_int4       int4 weight values [4096, 4096] -> [4096, 2048] bytes
  4. gemm w4a8       decode GEMV, M = 1, N = K = 4096
  5. pack_int2       ternary weight values [4096, 4096] -> [4096, 1024] bytes
  6. gemm w2a8       ternary, M = 1 and M = 128, N = K = 4096
  7. gemm w4a8       prefill, M = 4096, N = K = 4096 (tiled matrix-core path)

Memory-bound steps read their inputs from rings of distinct buffers larger
than twice the 256 MB Infinity Cache, so every timed read comes from HBM.

Timing.  This process never touches the GPU; it runs two children on it:
  * a plain run: the timed steps back to back (HIP events around the whole
    region give ms_per_step), the same steps with HIP events around every
    kernel (a secondary per-kernel figure, which also brackets the
    dispatch), the rows built on the same kernels ("extras"), the box's
    achievable ceilings, and the CPU oracle baseline;
  * the same launches again under `rocprofv3 --kernel-trace`, each dispatch
    labelled, so that every kernel's primary duration is its own begin->end
    time on the GPU (median over the timed launches, with p10 / p90).
`value` is the int8 TOP/s of the M = 4096 W4A8 GEMM from that kernel-trace
median.  If rocprofv3 is unavailable (or this process already runs under a
profiler, or --no-trace), the HIP-event figures are reported as primary and
the line says so.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import shutil
import subprocess
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized GEMM TOPS (M=4096) + GEMV HBM GB/s (M=1), % of MI355X roofline"
MALL_BYTES = 256 << 20
HOLD_CYCLES = 50_000_000
# The step's kernels in launch order: weight preparation and the decode
# GEMVs first, the M = 4096 GEMM last.  Right after that GEMM the clock is
# still recovering from its matrix-core load (a W2A8 decode GEMV launched
# directly after it measured 4.7 against 4.0 us), so it does not precede a
# GEMV in the cycle.
STEP_NAMES = ["quantize_rows", "gemm_w8a8_m64", "pack_int4", "gemm_w4a8_m1",
              "pack_int2", "gemm_w2a8_m1", "gemm_w2a8_m128", "gemm_w4a8_m4096"]
# same-size cold reads beside the decode GEMVs (algorithmic bytes of W2A8 and
# W4A8 at M = 1, N = K = 4096, and W4A8 at N = 11008)
READ_SIZES = {"gemm_w2a8_m1": 4214784, "gemm_w4a8_m1": 8409088, "gemm_w4a8_m1_n11008": 22592512}
# iterations of the W4A8-data matrix-core loop (32 instructions each)
STREAM_ITERS = 500


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-trace", action="store_true",
                   help="do not run the kernel-trace child (HIP events become the primary timing)")
    p.add_argument("--sustained", action="store_true",
                   help="also time the M=4096 GEMM back to back for a few milliseconds "
                        "(continuous matrix-core load)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the timed steps, run a plain 512 MiB device copy three times "
                        "(the known-size reference for the HBM byte counters)")
    p.add_argument("--child", choices=["measure", "trace"], default=None, help=argparse.SUPPRESS)
    p.add_argument("--out", default=None, help=argparse.SUPPRESS)
    return p.parse_args(argv)


# Kernel sources of the tiled matrix-core GEMM; the committed HBM-traffic
# summary is used only while their code (comments and blank space aside) and
# the compiler flags are unchanged.
TILED_SOURCES = ["gemm_tiled.hip", "lds_dma.h", "unpack.h", "bq_internal.h", "nf4_decode.h", "nf4_table.h", "gelu_fit.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w4a8_m4096_hbm_traffic.txt")


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace (string literals kept)."""
    token = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\])*"|\s+', re.S)
    return token.sub(lambda m: m.group(0) if m.group(0).startswith('"') else "", text)


def tiled_source_hash() -> str:
    import hashlib

    from bit_mixed_precision_amd import _build

    h = hashlib.sha256()
    for f in TILED_SOURCES:
        with open(os.path.join(ROOT, "bit_mixed_precision_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    h.update(" ".join(_build.FLAGS).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the M=4096 W4A8 GEMM from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by the copy-kernel factors), or
    None if there is none or the kernel sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    try:
        if vals.get("source_sha256_16") != tiled_source_hash():
            return None
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def ring_len(nbytes: int, minimum: int = 2) -> int:
    """Copies needed so that a ring of buffers spans > 2x the MALL."""
    return max(minimum, -(-2 * MALL_BYTES // max(nbytes, 1)) + 1)


# ---------------------------------------------------------------------------
# kernel-trace parsing (host only)
# ---------------------------------------------------------------------------

def is_bench_kernel(name: str) -> bool:
    """Dispatches the trace child labels: the library's and the calibration
    kernels (namespace bq); torch's own kernels are not labelled."""
    return "bq::" in name


def trace_durations(csv_path: str, labels: list) -> dict:
    """Per-label lists of kernel durations (us) from a rocprofv3 kernel-trace
    CSV: the rows of bench kernels, in dispatch order, paired one to one with
    the labels the trace child recorded for its launches."""
    rows = []
    with open(csv_path, newline="") as fh:
        for r in csv.DictReader(fh):
            if is_bench_kernel(r["Kernel_Name"]):
                rows.append(r)
    rows.sort(key=lambda r: int(r.get("Dispatch_Id") or 0))
    if len(rows) != len(labels):
        raise ValueError(f"{len(rows)} bench kernel dispatches in the trace, {len(labels)} labels")
    out = {}
    for r, lab in zip(rows, labels):
        out.setdefault(lab, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    return out


def stats(us: list) -> dict:
    a = np.asarray(us, dtype=np.float64)
    p10, p50, p90 = np.percentile(a, [10, 50, 90])
    return {"us": round(float(p50), 3), "us_mean": round(float(a.mean()), 3), "us_min": round(float(a.min()), 3),
            "us_p10": round(float(p10), 3), "us_p90": round(float(p90), 3), "n": int(a.size)}


def under_profiler() -> bool:
    pre = os.environ.get("LD_PRELOAD", "") + os.environ.get("HSA_TOOLS_LIB", "")
    return "rocprof" in pre or any(k.startswith("ROCPROF") for k in os.environ)


# ---------------------------------------------------------------------------
# the GPU children
# ---------------------------------------------------------------------------

class Runner:
    """Runs the benchmark's launches in one of two modes: "measure" brackets
    repetitions with HIP events on the launch stream and returns the mean us;
    "trace" only launches, recording one label per library dispatch (each
    timed function makes exactly one), for the kernel trace."""

    def __init__(self, mode, torch, steps, warmup):
        self.mode, self.torch, self.steps, self.warmup = mode, torch, steps, warmup
        self.labels = []

    def hold(self):
        # A device-side spin ahead of the timed work lets the host enqueue the
        # whole timed region before the GPU reaches it, so host launch
        # overhead never leaves the GPU idle between timed kernels.
        try:
            self.torch.cuda._sleep(HOLD_CYCLES)
            return True
        except Exception:
            return False

    def timed(self, label, fn, reps=None, warm=None):
        """fn(i) makes one library launch; reps timed launches after warm
        untimed ones.  Returns the mean us (measure) or None (trace)."""
        torch = self.torch
        reps = self.steps if reps is None else reps
        warm = self.warmup if warm is None else warm
        for i in range(warm):
            if self.mode == "trace":
                self.labels.append("warm")
            fn(i)
        torch.cuda.synchronize()
        if self.mode == "trace":
            for i in range(reps):
                self.labels.append(label)
                fn(warm + i)
            torch.cuda.synchronize()
            return None
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        self.hold()
        for i in range(reps):
            ev[i][0].record()
            fn(warm + i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3

    def untimed(self, fn, n=1):
        for i in range(n):
            if self.mode == "trace":
                self.labels.append("setup")
            fn(i)


def child(args):
    import torch

    from bit_mixed_precision_amd import _build, bq, roofline, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = Runner(args.child, torch, args.steps, args.warmup)
    res = {"mode": args.child}

    def up(a):
        if a.dtype == np.uint16:
            a = a.view(np.float16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def ring(t, n):
        return [t] + [t.clone() for _ in range(n - 1)]

    # ---------------- inputs (host draws, uploaded once) ----------------
    K = 4096
    W, A64 = synth.bminf_case(M=64, rows=3 * 4096, cols=K, seed=0)
    A4096, B4v, s4 = synth.w4a8_case(4096, 4096, K, seed=0)
    A1 = A4096[:1].copy()
    A2, B2v, s2 = synth.w2a8_case(128, 4096, K, seed=0)
    A2_1 = A2[:1].copy()

    W_d = ring(up(W), ring_len(W.nbytes))
    A64_d = up(A64)
    q_ring = [torch.empty(W.shape, dtype=torch.int8, device=dev) for _ in range(ring_len(W.size))]
    s_ring = [torch.empty(W.shape[0], dtype=torch.float16, device=dev) for _ in q_ring]
    B4v_d = ring(up(B4v), ring_len(B4v.nbytes))
    B4p_ring = [torch.empty((4096, K // 2), dtype=torch.uint8, device=dev) for _ in range(ring_len(4096 * K // 2))]
    B2v_d = ring(up(B2v), ring_len(B2v.nbytes))
    B2p_ring = [torch.empty((4096, K // 4), dtype=torch.uint8, device=dev) for _ in range(ring_len(4096 * K // 4))]
    s4_d, s2_d = up(s4), up(s2)
    A4096_d, A1_d, A2_d, A2_1_d = up(A4096), up(A1), up(A2), up(A2_1)
    C64 = torch.empty((64, W.shape[0]), dtype=torch.float16, device=dev)
    C1 = torch.empty((1, 4096), dtype=torch.float16, device=dev)
    C4096 = torch.empty((4096, 4096), dtype=torch.float16, device=dev)
    C2_1 = torch.empty((1, 4096), dtype=torch.float16, device=dev)
    C2_128 = torch.empty((128, 4096), dtype=torch.float16, device=dev)

    # fill every ring slot once (packed weights and codes) before timing
    R.untimed(lambda i: bq.quantize_rows(W_d[i % len(W_d)], q_ring[i], s_ring[i]), len(q_ring))
    R.untimed(lambda i: bq.pack_int4(B4v_d[i % len(B4v_d)], B4p_ring[i]), len(B4p_ring))
    R.untimed(lambda i: bq.pack_int2(B2v_d[i % len(B2v_d)], B2p_ring[i]), len(B2p_ring))
    torch.cuda.synchronize()

    # ---------------- the step ----------------
    def step(i, mark=None):
        def run(j, fn):
            if R.mode == "trace":
                R.labels.append(STEP_NAMES[j] if mark != "warm" else "warm")
            if callable(mark):
                mark(j)
            fn()
        qi = i % len(q_ring)
        qj = (i + len(q_ring) // 2) % len(q_ring)  # codes written a while ago
        pi = i % len(B4p_ring)
        pj = (i + len(B4p_ring) // 2) % len(B4p_ring)
        ri = i % len(B2p_ring)
        rj = (i + len(B2p_ring) // 2) % len(B2p_ring)
        run(0, lambda: bq.quantize_rows(W_d[i % len(W_d)], q_ring[qi], s_ring[qi]))
        run(1, lambda: bq.gemm_w8a8_dequant(A64_d, q_ring[qj], s_ring[qj], C64))
        run(2, lambda: bq.pack_int4(B4v_d[i % len(B4v_d)], B4p_ring[pi]))
        run(3, lambda: bq.gemm_w4a8_dequant(A1_d, B4p_ring[pj], s4_d, C1))
        run(4, lambda: bq.pack_int2(B2v_d[i % len(B2v_d)], B2p_ring[ri]))
        run(5, lambda: bq.gemm_w2a8_dequant(A2_1_d, B2p_ring[rj], s2_d, C2_1))
        run(6, lambda: bq.gemm_w2a8_dequant(A2_d, B2p_ring[rj], s2_d, C2_128))
        run(7, lambda: bq.gemm_w4a8_dequant(A4096_d, B4p_ring[pj], s4_d, C4096))

    for i in range(args.warmup):
        step(i, "warm")
    torch.cuda.synchronize()

    if R.mode == "measure":
        # (a) the timed steps back to back, events around the whole region
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        held = R.hold()
        e0.record()
        for i in range(args.steps):
            step(args.warmup + i)
        e1.record()
        torch.cuda.synchronize()
        res["wall_ms_per_step"] = (time.perf_counter() - t0) * 1e3 / args.steps
        res["ms_per_step"] = e0.elapsed_time(e1) / args.steps
        res["launch_queue_prefilled"] = held
        # (b) the same steps with events around every kernel (secondary)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STEP_NAMES) + 1)] for _ in range(args.steps)]
        R.hold()
        for i in range(args.steps):
            ev = evs[i]
            step(args.warmup + args.steps + i, lambda j: ev[j].record())
            ev[-1].record()
        torch.cuda.synchronize()
        dur = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) * 1e3 for j in range(len(STEP_NAMES))]
                        for i in range(args.steps)])
        res["events"] = {n: stats(dur[:, j]) for j, n in enumerate(STEP_NAMES)}
    else:
        for i in range(args.steps):
            step(args.warmup + i)
        torch.cuda.synchronize()

    ev = {}  # label -> event mean us (measure mode)

    def timed(label, fn, reps=None, warm=None):
        us = R.timed(label, fn, reps, warm)
        if us is not None:
            ev[label] = round(us, 3)

    # Sustained decode GEMV: back-to-back launches over the ring of packed
    # weights (each launch reads a different 8 MiB buffer from HBM), events
    # around the whole run.
    if R.mode == "measure":
        reps = 4 * len(B4p_ring)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        R.hold()
        g0.record()
        for r in range(reps):
            bq.gemm_w4a8_dequant(A1_d, B4p_ring[r % len(B4p_ring)], s4_d, C1)
        g1.record()
        torch.cuda.synchronize()
        res["gemv_sustained_us"] = g0.elapsed_time(g1) * 1e3 / reps
        if args.sustained:
            reps_big = 2 * len(B4p_ring)
            R.hold()
            g0.record()
            for r in range(reps_big):
                bq.gemm_w4a8_dequant(A4096_d, B4p_ring[r % len(B4p_ring)], s4_d, C4096)
            g1.record()
            torch.cuda.synchronize()
            res["gemm_m4096_sustained_us"] = g0.elapsed_time(g1) * 1e3 / reps_big

    # ---------------- rows after the path, outside the step ----------------
    # W8A8 linear layer with per-token activation quantization: fp16 X [64, 4096]
    # -> int8 codes + token scales, then the two-scale GEMM with the quantized
    # fused-QKV weight [12288, 4096] (codes and scales of the step).
    _, Xl = synth.bminf_linear_case(M=64)
    Xl_d = up(Xl)
    ql = torch.empty(Xl.shape, dtype=torch.int8, device=dev)
    sl = torch.empty((Xl.shape[0],), dtype=torch.float16, device=dev)
    Cl = torch.empty((Xl.shape[0], W.shape[0]), dtype=torch.float16, device=dev)
    timed("linear_quantize", lambda i: bq.quantize_rows(Xl_d, ql, sl))
    timed("linear_gemm", lambda i: bq.gemm_dual_scale(ql, q_ring[i % len(q_ring)], 8, s_ring[i % len(q_ring)],
                                                      sl, Cl))
    # Batched fused-QKV GEMM: the three [4096, 4096] int8 weights of the same
    # quantized matrix in one launch, the M = 64 per-token codes broadcast.
    Cq = torch.empty((3, Xl.shape[0], 4096), dtype=torch.float16, device=dev)
    timed("qkv_batched_w8a8", lambda i: bq.gemm_batched(ql, q_ring[i % len(q_ring)].view(3, 4096, K), 8,
                                                        s_ring[i % len(q_ring)].view(3, 4096), sl, out=Cq))
    # The M = 4096 W4A8 GEMM with GELU fused into the epilogue (the Pallas
    # page's fused-activation experiment).
    timed("gemm_w4a8_m4096_gelu", lambda i: bq.gemm_act(A4096_d, B4p_ring[(i + len(B4p_ring) // 2) % len(B4p_ring)],
                                                        4, s4_d, None, act="gelu", out=C4096))
    # int4 weight preparation from fp16: quantize to the int4 code range then
    # pack (two launches), and the same in one pass (bq_quantize_pack).
    q4 = torch.empty(W.shape, dtype=torch.int8, device=dev)
    s4q = torch.empty((W.shape[0],), dtype=torch.float16, device=dev)
    p4 = torch.empty((W.shape[0], W.shape[1] // 2), dtype=torch.uint8, device=dev)
    timed("prep_quantize_int4", lambda i: bq.quantize_rows_bits(W_d[i % len(W_d)], 4, q4, s4q))
    timed("prep_pack_int4", lambda i: bq.pack_int4(q4, p4))
    timed("prep_fused_int4", lambda i: bq.quantize_pack(W_d[i % len(W_d)], 4, p4, s4q))

    # W4A16 with NF4 weight codes, per-row scale and zero point: decode (M = 1)
    # and prefill (M = 4096), N = K = 4096, code rings past the MALL.
    g16 = np.random.default_rng(7)
    s_nf = up(g16.uniform(0.001, 0.01, 4096).astype(np.float16))
    z_nf = up(g16.uniform(-0.05, 0.05, 4096).astype(np.float16))
    codes_nf = torch.from_numpy(g16.integers(0, 256, (4096, K // 2), dtype=np.uint8)).to(dev)
    nf_ring = ring(codes_nf, ring_len(codes_nf.numel()))
    for Mn in (1, 4096):
        A_nf = up(g16.standard_normal((Mn, K)).astype(np.float16))
        C_nf = torch.empty((Mn, 4096), dtype=torch.float16, device=dev)
        timed(f"w4a16_nf4_m{Mn}", lambda i: bq.gemm_nf4_a16(A_nf, nf_ring[i % len(nf_ring)], s_nf, z_nf, out=C_nf))
        if Mn == 4096 and R.mode == "measure":
            # context: the vendor library's dense fp16 GEMM (torch.matmul, i.e.
            # hipBLASLt, fp32 accumulation) on the same activations and the
            # fp16 weights these codes decode to (the library's product with
            # the identity gives them exactly): the matrix cores' clock depends
            # on the values they multiply, so the comparison takes the same ones
            eye = torch.eye(K, dtype=torch.float16, device=dev)
            Wt = [bq.gemm_nf4_a16(eye, nf_ring[r], s_nf, z_nf) for r in range(2)]  # [K, N]: W[n, k] at [k, n]
            del eye
            timed("vendor_fp16_gemm_4096_nf4_values", lambda i: torch.matmul(A_nf, Wt[i % 2], out=C_nf))
            del Wt
        del A_nf, C_nf
    del nf_ring, codes_nf

    # The rest of the W4A8 M sweep at N = K = 4096 (M = 1 and 4096 are in the
    # step), each launch on a different packed B of a ring past the MALL.
    for Ms in (16, 64, 256, 1024):
        A_s = A4096_d[:Ms]
        C_s = torch.empty((Ms, 4096), dtype=torch.float16, device=dev)
        timed(f"gemm_w4a8_m{Ms}", lambda i: bq.gemm_w4a8_dequant(A_s, B4p_ring[i % len(B4p_ring)], s4_d, C_s))
        del C_s
    # W2A8 at M = 256 and the fused-QKV W8A8 shape at M = 128 (mid-M sweep)
    C2_256 = torch.empty((256, 4096), dtype=torch.float16, device=dev)
    A2_256 = up(np.concatenate([A2, A2]))
    timed("gemm_w2a8_m256", lambda i: bq.gemm_w2a8_dequant(A2_256, B2p_ring[i % len(B2p_ring)], s2_d, C2_256))
    # the decode GEMV at N = 11008
    _, B11v, s11h = synth.w4a8_case(1, 11008, K, seed=0)
    s11 = up(s11h)
    B11 = torch.empty((11008, K // 2), dtype=torch.uint8, device=dev)
    R.untimed(lambda i: bq.pack_int4(up(B11v), B11))
    B11_ring = ring(B11, ring_len(B11.numel()))
    C11 = torch.empty((1, 11008), dtype=torch.float16, device=dev)
    timed("gemm_w4a8_m1_n11008", lambda i: bq.gemm_w4a8_dequant(A1_d, B11_ring[i % len(B11_ring)], s11, C11))
    del B11_ring, B11
    # The small W4A8 case, M = 16, N = 256, K = 256 (launch-bound: time only).
    A0, B0v, s0 = synth.w4a8_case(16, 256, 256, seed=0)
    A0_d, s0_d = up(A0), up(s0)
    B0 = torch.empty((256, 128), dtype=torch.uint8, device=dev)
    R.untimed(lambda i: bq.pack_int4(up(B0v), B0))
    C0 = torch.empty((16, 256), dtype=torch.float16, device=dev)
    timed("gemm_w4a8_16x256x256", lambda i: bq.gemm_w4a8_dequant(A0_d, B0, s0_d, C0))
    # Decode with the three projections of a fused QKV weight in one launch.
    Bqkv = torch.stack([B4p_ring[0], B4p_ring[1], B4p_ring[2]])
    Bqkv_ring = ring(Bqkv, ring_len(Bqkv.numel()))
    sqkv = torch.stack([s4_d, s4_d, s4_d])
    Cqkv = torch.empty((3, 1, 4096), dtype=torch.float16, device=dev)
    timed("gemm_w4a8_m1_qkv_batched", lambda i: bq.gemm_batched(A1_d, Bqkv_ring[i % len(Bqkv_ring)], 4, sqkv,
                                                                out=Cqkv))
    del Bqkv_ring, Bqkv

    # ---------------- achievable ceilings of the box ----------------
    # libbq_calib.so (measurement kernels only): an int8 matrix-core loop on
    # register operands, streaming reads of 1 GiB and of the decode GEMVs'
    # sizes (each launch on a different part of a buffer past the MALL).
    import ctypes

    calib = ctypes.CDLL(_build.CALIB_LIB)
    cstream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cal_out = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    loop_blocks, loop_iters = 1024, 4000

    def mfma_loop(i):
        rc = calib.bq_calib_mfma_loop(loop_blocks, loop_iters, ctypes.c_void_p(cal_out.data_ptr()), cstream)
        if rc != 0:
            raise RuntimeError(f"bq_calib_mfma_loop: hip error {rc}")

    def mfma_w4a8_stream(i):
        rc = calib.bq_calib_mfma_w4a8_stream(loop_blocks, STREAM_ITERS, ctypes.c_void_p(cal_out.data_ptr()), cstream)
        if rc != 0:
            raise RuntimeError(f"bq_calib_mfma_w4a8_stream: hip error {rc}")

    rd_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)

    def reader(nbytes, blocks):
        step_b = (nbytes + 4095) // 4096 * 4096
        slots = max(1, rd_buf.numel() // step_b)

        def fn(i):
            off = (i % slots) * step_b
            rc = calib.bq_calib_read_stream(ctypes.c_void_p(rd_buf.data_ptr() + off), ctypes.c_int64(nbytes),
                                            blocks, ctypes.c_void_p(cal_out.data_ptr()), cstream)
            if rc != 0:
                raise RuntimeError(f"bq_calib_read_stream: hip error {rc}")
        return fn

    timed("mfma_i8_loop", mfma_loop, reps=10, warm=2)
    timed("mfma_i8_loop_w4a8_data", mfma_w4a8_stream, reps=10, warm=2)
    timed("read_stream_1GiB", reader(1 << 30, 2048), reps=10, warm=2)
    for key, nbytes in READ_SIZES.items():
        timed(f"read_{nbytes}", reader(nbytes, 2048))
    if R.mode == "measure":
        # a plain 512 MiB device copy (read + write) and the vendor library's
        # int8 GEMM at M = N = K = 4096 (torch._int_mm, i.e. hipBLASLt) beside
        # this library's: measurement context only, not used by the path
        cp_src = torch.empty(256 << 20, dtype=torch.float16, device=dev).fill_(1.0)
        cp_dst = torch.empty_like(cp_src)
        timed("device_copy_512MiB", lambda i: cp_dst.copy_(cp_src), reps=10, warm=2)
        del cp_src, cp_dst
        B8 = q_ring[0][:4096]
        timed("vendor_int8_gemm_4096", lambda i: torch._int_mm(A4096_d, B8.t()))
        C32 = torch.empty((4096, 4096), dtype=torch.int32, device=dev)
        timed("own_w8a8_i32_4096", lambda i: bq.gemm_w8a8_i32(A4096_d, B8, out=C32))
        if args.copy_calibration:
            src = torch.empty(256 << 20, dtype=torch.float16, device=dev).fill_(1.0)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
    del rd_buf, cal_out

    res["events_extra"] = ev
    # the automatic path of every GEMM shape reported (host-side rule)
    res["paths"] = {f"{M_}x{N_}x{k_}x{b_}": bq.select_path(M_, N_, k_, b_)
                    for (M_, N_, k_, b_) in [(64, 12288, K, 8), (1, 4096, K, 4), (4096, 4096, K, 4), (1, 4096, K, 2),
                                             (128, 4096, K, 2), (16, 4096, K, 4), (64, 4096, K, 4),
                                             (256, 4096, K, 4), (1024, 4096, K, 4), (256, 4096, K, 2),
                                             (1, 11008, K, 4), (16, 256, 256, 4), (64, 4096, K, 8)]}
    if R.mode == "trace":
        res["labels"] = R.labels
    elif not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(A4096, B4v, s4, args.cpu_seconds)
        res["cpu_oracle_configs"] = cpu_oracle_configs(W, A64, A1, B4v, A2, B2v, s4, s2)
    with open(args.out, "w") as fh:
        json.dump(res, fh)


# ---------------------------------------------------------------------------
# the CPU oracle baseline (measure child)
# ---------------------------------------------------------------------------

def cpu_cores() -> int:
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))
    return cores


def cpu_baseline(A, Bv, s, budget_s):
    """The oracle (unpack -> integer GEMM -> dequant, as it stands) on a
    bounded sample of rows of the M = 4096 W4A8 workload, on the host cores."""
    import oracle

    Bp = oracle.pack_int4(Bv)

    def run(rows):
        t = time.perf_counter()
        oracle.gemm_wxa8_dequant(np.ascontiguousarray(A[:rows]), Bp, s, 4)
        return time.perf_counter() - t

    # Rows of A grow fourfold while a run takes under a third of the budget;
    # when the whole workload fits, it is repeated until the budget is spent.
    rows = min(64, A.shape[0])
    t = run(rows)
    while rows < A.shape[0] and t < budget_s / 3:
        rows = min(A.shape[0], rows * 4)
        t = run(rows)
    reps = 1
    while rows == A.shape[0] and reps < 10 and t * (reps + 1) / reps <= budget_s:
        t += run(rows)
        reps += 1
    ops = 2 * rows * Bv.shape[0] * Bv.shape[1] * reps
    return {"value": round(ops / t / 1e12, 6), "unit": "TOPS", "cores": cpu_cores(), "kind": "oracle",
            "sample": f"{rows} of {A.shape[0]} rows of A (M={rows}, N={Bv.shape[0]}, K={Bv.shape[1]}, "
                      f"w4a8 dequant) x {reps}, {t:.1f} s"}


def cpu_oracle_configs(W, A64, A1, B4v, A2, B2v, s4, s2):
    """The oracle (as it stands, all host cores) on the other workloads of the
    step, each the median of three runs."""
    import oracle

    from bit_mixed_precision_amd import synth

    out = {}

    def timed(name, fn):
        ts = []
        for _ in range(3):
            t = time.perf_counter()
            fn()
            ts.append((time.perf_counter() - t) * 1e3)
        out[name] = {"oracle_ms": round(float(np.median(ts)), 2)}

    codes = {}
    timed("quantize_rows", lambda: codes.update(zip(("q", "s"), oracle.quantize_rows(W))))
    timed("gemm_w8a8_m64", lambda: oracle.gemm_wxa8_dequant(A64, codes["q"], codes["s"], 8))
    B4p = oracle.pack_int4(B4v)
    B2p = oracle.pack_int2(B2v)
    timed("pack_int4", lambda: oracle.pack_int4(B4v))
    timed("gemm_w4a8_m1", lambda: oracle.gemm_wxa8_dequant(A1, B4p, s4, 4))
    timed("pack_int2", lambda: oracle.pack_int2(B2v))
    timed("gemm_w2a8_m1", lambda: oracle.gemm_wxa8_dequant(np.ascontiguousarray(A2[:1]), B2p, s2, 2))
    timed("gemm_w2a8_m128", lambda: oracle.gemm_wxa8_dequant(A2, B2p, s2, 2))
    _, B11v, s11 = synth.w4a8_case(1, 11008, W.shape[1], seed=0)
    B11p = oracle.pack_int4(B11v)
    timed("gemm_w4a8_m1_n11008", lambda: oracle.gemm_wxa8_dequant(A1, B11p, s11, 4))
    out["cores"] = cpu_cores()
    # single-thread times of the quantize and the M <= 64 workloads, in a
    # child process (the thread count of the oracle's OpenMP is fixed at load)
    code = (
        "import sys, time, json, numpy as np; sys.path.insert(0, %r)\n"
        "import oracle; from bit_mixed_precision_amd import synth\n"
        "W, A64 = synth.bminf_case(M=64, rows=3 * 4096, cols=4096, seed=0)\n"
        "A, B4v, s4 = synth.w4a8_case(1, 4096, 4096, seed=0)\n"
        "B4p = oracle.pack_int4(B4v); r = {}\n"
        "t = time.perf_counter(); q, s = oracle.quantize_rows(W); r['quantize_rows'] = time.perf_counter() - t\n"
        "t = time.perf_counter(); oracle.gemm_wxa8_dequant(A64, q, s, 8); r['gemm_w8a8_m64'] = time.perf_counter() - t\n"
        "t = time.perf_counter(); oracle.gemm_wxa8_dequant(A, B4p, s4, 4); r['gemm_w4a8_m1'] = time.perf_counter() - t\n"
        "print(json.dumps(r))\n" % ROOT)
    try:
        res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                             env={**os.environ, "OMP_NUM_THREADS": "1"})
        one = json.loads(res.stdout.strip().splitlines()[-1])
        for k, v in one.items():
            out[k]["oracle_ms_1thread"] = round(v * 1e3, 2)
    except Exception as e:  # reported, not fatal: the all-cores times stand
        out["single_thread_error"] = str(e)[:200]
    return out


# ---------------------------------------------------------------------------
# the parent: runs both children and writes the line
# ---------------------------------------------------------------------------

def _child_cmd(args, mode, out):
    cmd = [sys.executable, os.path.abspath(__file__), "--child", mode, "--out", out,
           "--steps", str(args.steps), "--warmup", str(args.warmup), "--cpu-seconds", str(args.cpu_seconds)]
    if args.no_cpu_baseline:
        cmd.append("--no-cpu-baseline")
    if args.sustained:
        cmd.append("--sustained")
    if args.copy_calibration:
        cmd.append("--copy-calibration")
    return cmd


def run_trace_child(args, tmp):
    """The launches again under rocprofv3's kernel trace; returns (per-label
    durations, None) or (None, reason)."""
    if args.no_trace:
        return None, "--no-trace"
    if under_profiler():
        return None, "already under a profiler"
    rp = shutil.which("rocprofv3") or ("/opt/rocm/bin/rocprofv3" if os.path.exists("/opt/rocm/bin/rocprofv3")
                                       else None)
    if rp is None:
        return None, "rocprofv3 not found"
    out = os.path.join(tmp, "trace.json")
    tdir = os.path.join(tmp, "trace")
    cmd = [rp, "--kernel-trace", "--output-format", "csv", "-d", tdir, "-o", "bench", "--",
           *_child_cmd(args, "trace", out)]
    r = subprocess.run(cmd, cwd=tmp, env={**os.environ, "TMPDIR": tmp}, capture_output=True, text=True,
                       timeout=900)
    found = glob.glob(os.path.join(tdir, "**", "bench_kernel_trace.csv"), recursive=True)
    if not os.path.exists(out) or not found:
        tail = (r.stdout + r.stderr).strip().splitlines()[-3:]
        return None, f"trace child rc {r.returncode}: {' | '.join(tail)[:300]}"
    # rocprofv3 may end with its own fault after the program has finished and
    # the files are whole: the results count when both are present
    labels = json.load(open(out))["labels"]
    try:
        return trace_durations(found[0], labels), None
    except ValueError as e:
        return None, str(e)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: every kernel of the path is measured on a single "
              "GPU (the path is not sharded across GPUs); --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    if args.child:
        child(args)
        return

    from bit_mixed_precision_amd import _build, bq

    if not os.path.exists(bq.LIB_PATH) or not os.path.exists(_build.CALIB_LIB):
        import __graft_entry__

        __graft_entry__.build()
    tmp = tempfile.mkdtemp(prefix="bq_bench_")
    try:
        a_out = os.path.join(tmp, "measure.json")
        r = subprocess.run(_child_cmd(args, "measure", a_out), timeout=1200)
        if r.returncode != 0 or not os.path.exists(a_out):
            print(f"bench.py: the measuring run failed (rc {r.returncode})", file=sys.stderr)
            sys.exit(r.returncode or 1)
        meas = json.load(open(a_out))
        trace, why = run_trace_child(args, tmp)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    print(json.dumps(build_line(args, meas, trace, why)), flush=True)


def build_line(args, meas, trace, why):
    """The JSON line from the measuring run's figures and the kernel-trace
    durations (primary when present)."""
    from bit_mixed_precision_amd import roofline

    K = 4096
    paths = meas["paths"]

    def select_path(M_, N_, k_, b_):
        return paths[f"{M_}x{N_}x{k_}x{b_}"]

    timing = ("kernel trace: rocprofv3 --kernel-trace begin->end of each launch, median over the timed "
              "launches of this run (HIP events: secondary, *_events)") if trace else \
        f"HIP events around each launch (kernel trace unavailable: {why})"

    def primary(label, ev_us):
        """(us, stats) of a label: the trace median, else the events figure."""
        if trace and label in trace:
            st = stats(trace[label])
            return st["us"], st
        return ev_us, None

    def perf(M_, N_, us, bits):
        ops, nbytes = roofline.gemm_ops(M_, N_, K), roofline.gemm_bytes(M_, N_, K, bits)
        b, _ = roofline.bound(ops, nbytes)
        gbs, tops = nbytes / (us * 1e-6), ops / (us * 1e-6)
        return {"GB_per_s": round(gbs / 1e9, 1), "TOPS": round(tops / 1e12, 2), "bound": b,
                "frac_of_bound": round(gbs / roofline.HBM_PEAK_BYTES_PER_S if b == "hbm"
                                       else tops / roofline.INT8_MFMA_PEAK_OPS_PER_S, 4)}

    work = {
        "quantize_rows": dict(shape=[12288, 4096], bytes=roofline.quantize_bytes(12288, 4096), ops=0, path="quantize"),
        "gemm_w8a8_m64": dict(shape=[64, 12288, 4096], bits=8),
        "pack_int4": dict(shape=[4096, 4096], bytes=roofline.pack_bytes(4096, K, 4), ops=0, path="pack"),
        "gemm_w4a8_m1": dict(shape=[1, 4096, 4096], bits=4),
        "gemm_w4a8_m4096": dict(shape=[4096, 4096, 4096], bits=4),
        "pack_int2": dict(shape=[4096, 4096], bytes=roofline.pack_bytes(4096, K, 2), ops=0, path="pack"),
        "gemm_w2a8_m1": dict(shape=[1, 4096, 4096], bits=2),
        "gemm_w2a8_m128": dict(shape=[128, 4096, 4096], bits=2),
    }
    kernels = {}
    for n in STEP_NAMES:
        w = work[n]
        evst = meas["events"][n]
        us, st = primary(n, evst["us_mean"])
        k = {"shape": w["shape"], "us": us}
        if st:
            k.update({x: st[x] for x in ("us_mean", "us_p10", "us_p90", "n")})
        k["us_events"] = evst["us_mean"]
        if "bits" in w:
            M_, N_, _ = w["shape"]
            k["path"] = select_path(M_, N_, K, w["bits"])
            k.update(perf(M_, N_, us, w["bits"]))
        else:
            gbs = w["bytes"] / (us * 1e-6)
            k.update({"path": w["path"], "GB_per_s": round(gbs / 1e9, 1), "bound": "hbm",
                      "frac_of_bound": round(gbs / roofline.HBM_PEAK_BYTES_PER_S, 4)})
        kernels[n] = k

    ev = meas["events_extra"]

    def read_us(nbytes):
        return primary(f"read_{nbytes}", ev.get(f"read_{nbytes}"))[0]

    for n in ("gemm_w4a8_m1", "gemm_w2a8_m1"):
        r_us = read_us(READ_SIZES[n])
        kernels[n]["read_same_size_us"] = r_us
        kernels[n]["vs_same_size_read"] = round(kernels[n]["us"] / r_us, 4) if r_us else None

    head = kernels["gemm_w4a8_m4096"]
    gemv = kernels["gemm_w4a8_m1"]
    traffic = measured_traffic()
    roof = {
        "bound": "mfma", "kernel": "gemm_w4a8_m4096 (gemm_tiled_kernel, 256x256 tile, 8 waves)",
        "achieved": head["TOPS"], "peak": roofline.INT8_MFMA_PEAK_OPS_PER_S / 1e12, "unit": "TOPS",
        "frac": head["frac_of_bound"], "us_per_launch": head["us"],
        "us_per_launch_events": head["us_events"],
        "traffic": traffic,
        "traffic_source": ("profiles/gemm_w4a8_m4096_hbm_traffic.txt: rocprofv3 FETCH_SIZE and WRITE_SIZE of this "
                           "kernel's sources, scaled by a plain copy's counts (voided when the sources change)"),
        "algorithmic_bytes": roofline.gemm_bytes(4096, 4096, K, 4),
        "timing": "kernel trace" if trace else "HIP events",
    }

    # extras: the rows built on the same kernels, timed after the step
    def extra(label, M_=None, N_=None, bits=None, nbytes=None, ops=None, peak=None):
        us, st = primary(label, ev.get(label))
        if us is None:
            return None
        e = {"us": us, "us_events": ev.get(label)}
        if st:
            e["us_p10"], e["us_p90"] = st["us_p10"], st["us_p90"]
        if M_ is not None:
            e["shape"] = [M_, N_, K]
            e["path"] = select_path(M_, N_, K, bits)
            e.update(perf(M_, N_, us, bits))
        if nbytes is not None:
            e["GB_per_s"] = round(nbytes / (us * 1e-6) / 1e9, 1)
            e["frac_of_hbm_peak"] = round(nbytes / (us * 1e-6) / roofline.HBM_PEAK_BYTES_PER_S, 4)
        if ops is not None:
            e["TOPS"] = round(ops / (us * 1e-6) / 1e12, 2)
            if peak:
                e["frac_of_peak"] = round(ops / (us * 1e-6) / peak, 4)
        return e

    Ml, Nl = 64, 12288
    lin_q = extra("linear_quantize", nbytes=roofline.quantize_bytes(Ml, K))
    lin_g = extra("linear_gemm", nbytes=roofline.gemm_bytes(Ml, Nl, K, 8) + 2 * Ml)
    sweep = {f"gemm_w4a8_m{m}": extra(f"gemm_w4a8_m{m}", m, 4096, 4) for m in (16, 64, 256, 1024)}
    sweep["gemm_w2a8_m256"] = extra("gemm_w2a8_m256", 256, 4096, 2)
    n11 = extra("gemm_w4a8_m1_n11008", 1, 11008, 4)
    r11 = read_us(READ_SIZES["gemm_w4a8_m1_n11008"])
    n11["read_same_size_us"] = r11
    n11["vs_same_size_read"] = round(n11["us"] / r11, 4) if r11 else None
    sweep["gemm_w4a8_m1_n11008"] = n11
    sweep["gemm_w4a8_16x256x256"] = dict(extra("gemm_w4a8_16x256x256"), shape=[16, 256, 256], bound="launch",
                                         path=select_path(16, 256, 256, 4))
    sweep["gemm_w4a8_m1_qkv_batched"] = dict(
        extra("gemm_w4a8_m1_qkv_batched", nbytes=3 * roofline.gemm_bytes(1, 4096, K, 4) - 2 * K),
        shape=[3, 1, 4096, K], path=select_path(1, 4096, K, 4))
    gelu = extra("gemm_w4a8_m4096_gelu", ops=roofline.gemm_ops(4096, 4096, K),
                 peak=roofline.INT8_MFMA_PEAK_OPS_PER_S)
    gelu["vs_plain_epilogue"] = round(head["us"] / gelu["us"], 4)
    prep_bytes = roofline.quantize_bytes(12288, K) + roofline.pack_bytes(12288, K, 4)
    pq, pp, pf = extra("prep_quantize_int4"), extra("prep_pack_int4"), extra("prep_fused_int4")
    extras = {
        "w4a16_nf4_m1": dict(extra("w4a16_nf4_m1", nbytes=roofline.nf4_gemm_bytes(1, 4096, K)),
                             shape=[1, 4096, K], kernel="gemv_nf4_kernel"),
        "w4a16_nf4_m4096": dict(extra("w4a16_nf4_m4096", ops=roofline.gemm_ops(4096, 4096, K),
                                      peak=roofline.FP16_MFMA_PEAK_FLOPS),
                                shape=[4096, 4096, K], kernel="gemm_tiled_kernel (NF4 mode)"),
        "w4a8_sweep": sweep,
        "weight_prep_int4": {
            "shape": [12288, K], "quantize_us": pq["us"], "pack_us": pp["us"],
            "GB_per_s": round(prep_bytes / ((pq["us"] + pp["us"]) * 1e-6) / 1e9, 1),
            "fused_us": pf["us"],
            "fused_GB_per_s": round((12288 * K * 2 + 12288 * K // 2 + 2 * 12288) / (pf["us"] * 1e-6) / 1e9, 1),
        },
        "gemm_w4a8_m4096_gelu": dict(gelu, shape=[4096, 4096, K]),
        "qkv_batched_w8a8": dict(extra("qkv_batched_w8a8", nbytes=roofline.gemm_bytes(Ml, Nl, K, 8) + 2 * Ml),
                                 shape=[3, Ml, 4096, K], path=select_path(Ml, 4096, K, 8)),
        "linear_w8a8_per_token": {
            "shape": [Ml, Nl, K], "path": select_path(Ml, Nl, K, 8), "quantize_us": lin_q["us"],
            "gemm_us": lin_g["us"], "total_us": round(lin_q["us"] + lin_g["us"], 3),
            "GB_per_s": round((roofline.quantize_bytes(Ml, K) + roofline.gemm_bytes(Ml, Nl, K, 8) + 2 * Ml)
                              / ((lin_q["us"] + lin_g["us"]) * 1e-6) / 1e9, 1)},
    }

    loop_us = primary("mfma_i8_loop", ev.get("mfma_i8_loop"))[0]
    loop_tops = 1024 * 4 * 4000 * 4 * 65536 / (loop_us * 1e-6) / 1e12
    data_us = primary("mfma_i8_loop_w4a8_data", ev.get("mfma_i8_loop_w4a8_data"))[0]
    # 2^21 operations per wavefront per iteration: one 128-k stage of the
    # M = 4096 GEMM's wavefront (64 instructions of 16 x 16 x 64)
    data_tops = 1024 * 4 * STREAM_ITERS * (1 << 21) / (data_us * 1e-6) / 1e12
    rd_us = primary("read_stream_1GiB", ev.get("read_stream_1GiB"))[0]
    rd_gbs = (1 << 30) / (rd_us * 1e-6) / 1e9
    ceilings = {
        "mfma_i8_loop": {"us": round(loop_us, 2), "TOPS": round(loop_tops, 2),
                         "frac_of_int8_peak": round(loop_tops * 1e12 / roofline.INT8_MFMA_PEAK_OPS_PER_S, 4)},
        "read_stream_1GiB": {"us": round(rd_us, 2), "GB_per_s": round(rd_gbs, 1),
                             "frac_of_hbm_peak": round(rd_gbs * 1e9 / roofline.HBM_PEAK_BYTES_PER_S, 4)},
        "read_same_size": {str(nb): {"us": read_us(nb), "GB_per_s": round(nb / (read_us(nb) * 1e-6) / 1e9, 1)}
                           for nb in READ_SIZES.values()},
        # the W4A8 GEMM's matrix-core instruction stream on operands drawn like
        # the workload's: the clock the matrix cores hold depends on the bits
        # they multiply, so this, not the constant-operand loop, is the
        # matrix-core rate the GEMM can reach on this data
        "mfma_i8_loop_w4a8_data": {"us": round(data_us, 2), "TOPS": round(data_tops, 2),
                                   "frac_of_int8_peak": round(data_tops * 1e12 / roofline.INT8_MFMA_PEAK_OPS_PER_S, 4)},
        "value_frac_of_mfma_loop": round(head["TOPS"] / loop_tops, 4),
        "value_frac_of_mfma_w4a8_data_loop": round(head["TOPS"] / data_tops, 4),
    }
    if "device_copy_512MiB" in ev:
        cp_us = ev["device_copy_512MiB"]
        ceilings["device_copy_512MiB_events"] = {"us": cp_us, "GB_per_s": round(2 * (512 << 20) / (cp_us * 1e-6) / 1e9, 1)}
    if "vendor_int8_gemm_4096" in ev:
        ops = roofline.gemm_ops(4096, 4096, K)
        v_us, o_us = ev["vendor_int8_gemm_4096"], ev["own_w8a8_i32_4096"]
        ceilings["vendor_int8_gemm_4096_events"] = {"kernel": "torch._int_mm (hipBLASLt), int8 x int8 -> int32",
                                                    "us": v_us, "TOPS": round(ops / (v_us * 1e-6) / 1e12, 2)}
        ceilings["own_w8a8_i32_4096_events"] = {"us": o_us, "TOPS": round(ops / (o_us * 1e-6) / 1e12, 2),
                                                "vs_vendor": round(v_us / o_us, 4)}
    if "vendor_fp16_gemm_4096_nf4_values" in ev:
        ops = roofline.gemm_ops(4096, 4096, K)
        v_us, o_us = ev["vendor_fp16_gemm_4096_nf4_values"], ev["w4a16_nf4_m4096"]
        ceilings["vendor_fp16_gemm_4096_nf4_values_events"] = {
            "kernel": "torch.matmul (hipBLASLt), fp16 x fp16 -> fp16, the NF4 GEMM's activations and decoded weights",
            "us": v_us, "TFLOPS": round(ops / (v_us * 1e-6) / 1e12, 2),
            "own_nf4_us": o_us, "own_nf4_vs_vendor": round(v_us / o_us, 4)}

    cpu = meas.get("cpu_baseline")
    cfgs = meas.get("cpu_oracle_configs")
    if cfgs:
        gpu_us = {k: v["us"] for k, v in kernels.items()}
        gpu_us["gemm_w4a8_m1_n11008"] = n11["us"]
        for k, v in cfgs.items():
            if isinstance(v, dict) and k in gpu_us:
                v["gpu_us"] = gpu_us[k]
                v["speedup"] = round(v["oracle_ms"] * 1e3 / gpu_us[k], 1)

    return {
        "metric": METRIC,
        "value": head["TOPS"],
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(meas["ms_per_step"], 4),
        "wall_ms_per_step": round(meas["wall_ms_per_step"], 4),
        "launch_queue_prefilled": meas.get("launch_queue_prefilled"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "timing": timing,
        "config": {
            "workload": "w4a8 dequant GEMM M=4096 N=4096 K=4096 within one pass of the path "
                        "(quantize 12288x4096, w8a8 M=64 N=12288, pack int4, w4a8 M=1, pack int2, "
                        "w2a8 M=1 and 128, w4a8 M=4096)",
            "M": 4096, "N": 4096, "K": 4096, "weight_bits": 4,
        },
        "gemv_m1": {"us": gemv["us"], "GB_per_s": gemv["GB_per_s"], "frac_of_hbm_peak": gemv["frac_of_bound"],
                    "shape": gemv["shape"], "read_same_size_us": gemv["read_same_size_us"],
                    "vs_same_size_read": gemv["vs_same_size_read"], "us_events": gemv["us_events"],
                    "sustained_us_events": round(meas["gemv_sustained_us"], 3)},
        "roofline": roof,
        "gemm_m4096_sustained_us_events": meas.get("gemm_m4096_sustained_us"),
        "cpu_baseline": cpu,
        "cpu_oracle_configs": cfgs,
        "kernels": kernels,
        "extras": extras,
        "ceilings": ceilings,
    }


if __name__ == "__main__":
    main()
