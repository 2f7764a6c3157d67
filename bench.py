#!/usr/bin/env python3
"""Benchmark of the quantized-GEMM hot path on one MI355X.

One step is one pass of every kernel of the path over one batch of
synthetic, HBM-resident inputs, in the order a model would run them:

  1. quantize_rows   fp16 fused-QKV weight [12288, 4096] -> int8 codes + fp16 scales
  2. gemm w8a8       those codes, M = 64 (tiled matrix-core path, 64x64 tiles)
  3. pack_int4       int4 weight values [4096, 4096] -> [4096, 2048] bytes
  4. gemm w4a8       decode GEMV, M = 1, N = K = 4096 (dot-product GEMV path)
  5. gemm w4a8       prefill, M = 4096, N = K = 4096 (tiled matrix-core path)
  6. pack_int2       ternary weight values [4096, 4096] -> [4096, 1024] bytes
  7. gemm w2a8       ternary, M = 1 and M = 128, N = K = 4096

Memory-bound steps read their inputs from rings of distinct buffers larger
than twice the 256 MB Infinity Cache, so every timed read comes from HBM.
Each kernel is timed with HIP events recorded on the stream it runs on;
`value` is the headline: int8 TOPS of the M = 4096 W4A8 GEMM.  The decode
GEMV's HBM GB/s and every other kernel's rate are reported under "kernels".
After the step, "extras" times the rest of the W4A8 M sweep (M = 16, 64,
256, 1024), the decode GEMV at N = 11008, and the rows built on the same
kernels (per-token linear, batched QKV, fused GELU, int4 weight preparation,
W4A16 NF4), none of which enter `value` or `ms_per_step`; "ceilings" puts
a plain device copy and the vendor library's int8 GEMM, measured in the same
run, beside this library's kernels.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized GEMM TOPS (M=4096) + GEMV HBM GB/s (M=1), % of MI355X roofline"
MALL_BYTES = 256 << 20
HOLD_CYCLES = 50_000_000


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--sustained", action="store_true",
                   help="also time the M=4096 GEMM back to back for a few milliseconds "
                        "(continuous matrix-core load)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the timed steps, run a plain 512 MiB device copy three times "
                        "(the known-size reference for the HBM byte counters)")
    return p.parse_args()


# Kernel sources of the tiled matrix-core GEMM; the committed HBM-traffic
# summary is used only while their code (comments and blank space aside) and
# the compiler flags are unchanged.
TILED_SOURCES = ["gemm_tiled.hip", "unpack.h", "bq_internal.h", "nf4_table.h", "erfc_fit.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w4a8_m4096_hbm_traffic.txt")


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace (string literals kept)."""
    import re

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


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: every kernel of the path is measured on a single "
              "GPU (the path is not sharded across GPUs); --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_mixed_precision_amd import bq, roofline, synth

    from bit_mixed_precision_amd import _build as lib_build

    if not os.path.exists(bq.LIB_PATH) or not os.path.exists(lib_build.CALIB_LIB):
        import __graft_entry__

        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

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
    B4p_ring = [torch.empty((4096, K // 2), dtype=torch.uint8, device=dev)
                for _ in range(ring_len(4096 * K // 2))]
    B2v_d = ring(up(B2v), ring_len(B2v.nbytes))
    B2p_ring = [torch.empty((4096, K // 4), dtype=torch.uint8, device=dev)
                for _ in range(ring_len(4096 * K // 4))]
    s4_d, s2_d = up(s4), up(s2)
    A4096_d, A1_d, A2_d, A2_1_d = up(A4096), up(A1), up(A2), up(A2_1)
    C64 = torch.empty((64, W.shape[0]), dtype=torch.float16, device=dev)
    C1 = torch.empty((1, 4096), dtype=torch.float16, device=dev)
    C4096 = torch.empty((4096, 4096), dtype=torch.float16, device=dev)
    C2_1 = torch.empty((1, 4096), dtype=torch.float16, device=dev)
    C2_128 = torch.empty((128, 4096), dtype=torch.float16, device=dev)

    # fill every ring slot once (packed weights and codes) before timing
    for i in range(len(q_ring)):
        bq.quantize_rows(W_d[i % len(W_d)], q_ring[i], s_ring[i])
    for i in range(len(B4p_ring)):
        bq.pack_int4(B4v_d[i % len(B4v_d)], B4p_ring[i])
    for i in range(len(B2p_ring)):
        bq.pack_int2(B2v_d[i % len(B2v_d)], B2p_ring[i])
    torch.cuda.synchronize()

    # ---------------- the step ----------------
    names = ["quantize_rows", "gemm_w8a8_m64", "pack_int4", "gemm_w4a8_m1",
             "gemm_w4a8_m4096", "pack_int2", "gemm_w2a8_m1", "gemm_w2a8_m128"]

    def step(i, ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record()
        mark(0)
        qi = i % len(q_ring)
        bq.quantize_rows(W_d[i % len(W_d)], q_ring[qi], s_ring[qi])
        mark(1)
        qj = (i + len(q_ring) // 2) % len(q_ring)  # codes written a while ago
        bq.gemm_w8a8_dequant(A64_d, q_ring[qj], s_ring[qj], C64)
        mark(2)
        pi = i % len(B4p_ring)
        bq.pack_int4(B4v_d[i % len(B4v_d)], B4p_ring[pi])
        mark(3)
        pj = (i + len(B4p_ring) // 2) % len(B4p_ring)
        bq.gemm_w4a8_dequant(A1_d, B4p_ring[pj], s4_d, C1)
        mark(4)
        bq.gemm_w4a8_dequant(A4096_d, B4p_ring[pj], s4_d, C4096)
        mark(5)
        ri = i % len(B2p_ring)
        bq.pack_int2(B2v_d[i % len(B2v_d)], B2p_ring[ri])
        mark(6)
        rj = (i + len(B2p_ring) // 2) % len(B2p_ring)
        bq.gemm_w2a8_dequant(A2_1_d, B2p_ring[rj], s2_d, C2_1)
        mark(7)
        bq.gemm_w2a8_dequant(A2_d, B2p_ring[rj], s2_d, C2_128)
        mark(8)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def hold_gpu():
        # A device-side spin ahead of the timed work lets the host enqueue the
        # whole timed region before the GPU reaches it, so host launch
        # overhead never leaves the GPU idle between timed kernels.
        try:
            torch.cuda._sleep(HOLD_CYCLES)
            return True
        except Exception:
            return False

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    held = hold_gpu()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    dur_ms = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(len(names))]
                       for i in range(args.steps)])
    mean_ms = dur_ms.mean(axis=0)
    gpu_ms_per_step = evs[0][0].elapsed_time(evs[-1][-1]) / args.steps

    # Sustained decode GEMV: back-to-back launches over the ring of packed
    # weights (each launch reads a different 8 MiB buffer from HBM).
    reps = 4 * len(B4p_ring)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold_gpu()
    g0.record()
    for r in range(reps):
        bq.gemm_w4a8_dequant(A1_d, B4p_ring[r % len(B4p_ring)], s4_d, C1)
    g1.record()
    torch.cuda.synchronize()
    gemv_sustained_us = g0.elapsed_time(g1) * 1e3 / reps

    # Optionally, the M = 4096 GEMM back to back over the same ring (each
    # launch reads a different packed B) for a few milliseconds: the rate
    # under continuous matrix-core load, where the power limit lowers the
    # clock further than within the step.
    big_sustained_us = None
    if args.sustained:
        reps_big = 2 * len(B4p_ring)
        torch.cuda.synchronize()
        hold_gpu()
        g0.record()
        for r in range(reps_big):
            bq.gemm_w4a8_dequant(A4096_d, B4p_ring[r % len(B4p_ring)], s4_d, C4096)
        g1.record()
        torch.cuda.synchronize()
        big_sustained_us = g0.elapsed_time(g1) * 1e3 / reps_big

    # ---------------- rows after the path, timed outside the step ----------------
    # W8A8 linear layer with per-token activation quantization: fp16 X [64, 4096]
    # -> int8 codes + token scales (quantize_rows), then the two-scale GEMM with
    # the quantized fused-QKV weight [12288, 4096] (codes and scales of the step).
    Wl, Xl = synth.bminf_linear_case(M=64)
    del Wl
    Xl_d = up(Xl)
    ql = torch.empty(Xl.shape, dtype=torch.int8, device=dev)
    sl = torch.empty((Xl.shape[0],), dtype=torch.float16, device=dev)
    Cl = torch.empty((Xl.shape[0], W.shape[0]), dtype=torch.float16, device=dev)
    lin_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.warmup):
        bq.quantize_rows(Xl_d, ql, sl)
        bq.gemm_dual_scale(ql, q_ring[i % len(q_ring)], 8, s_ring[i % len(q_ring)], sl, Cl)
    torch.cuda.synchronize()
    hold_gpu()
    for i in range(args.steps):
        qj = i % len(q_ring)
        lin_ev[i][0].record()
        bq.quantize_rows(Xl_d, ql, sl)
        lin_ev[i][1].record()
        bq.gemm_dual_scale(ql, q_ring[qj], 8, s_ring[qj], sl, Cl)
        lin_ev[i][2].record()
    torch.cuda.synchronize()
    lin_q_us = float(np.mean([e[0].elapsed_time(e[1]) for e in lin_ev])) * 1e3
    lin_g_us = float(np.mean([e[1].elapsed_time(e[2]) for e in lin_ev])) * 1e3
    Ml, Kl, Nl = Xl.shape[0], Xl.shape[1], W.shape[0]
    lin_q_bytes = roofline.quantize_bytes(Ml, Kl)
    lin_g_bytes = roofline.gemm_bytes(Ml, Nl, Kl, 8) + 2 * Ml
    # Batched fused-QKV GEMM: the three [4096, 4096] int8 weights of the same
    # quantized [12288, 4096] matrix in one launch, the M = 64 per-token codes
    # broadcast to all three, two-scale epilogue.
    Cq = torch.empty((3, Xl.shape[0], 4096), dtype=torch.float16, device=dev)
    qkv_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.warmup):
        bq.gemm_batched(ql, q_ring[i % len(q_ring)].view(3, 4096, Kl), 8,
                        s_ring[i % len(q_ring)].view(3, 4096), sl, out=Cq)
    torch.cuda.synchronize()
    hold_gpu()
    for i in range(args.steps):
        qj = i % len(q_ring)
        qkv_ev[i][0].record()
        bq.gemm_batched(ql, q_ring[qj].view(3, 4096, Kl), 8, s_ring[qj].view(3, 4096), sl, out=Cq)
        qkv_ev[i][1].record()
    torch.cuda.synchronize()
    qkv_us = float(np.mean([e[0].elapsed_time(e[1]) for e in qkv_ev])) * 1e3
    qkv_bytes = roofline.gemm_bytes(Ml, Nl, Kl, 8) + 2 * Ml  # A once, the three weights, scales, C
    # The M = 4096 W4A8 GEMM with GELU fused into the epilogue (the Pallas
    # page's fused-activation experiment: utilization with the activation
    # against without it, the plain launch being the step's).
    act_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.warmup):
        bq.gemm_act(A4096_d, B4p_ring[i % len(B4p_ring)], 4, s4_d, None, act="gelu", out=C4096)
    torch.cuda.synchronize()
    hold_gpu()
    for i in range(args.steps):
        pj = (i + len(B4p_ring) // 2) % len(B4p_ring)
        act_ev[i][0].record()
        bq.gemm_act(A4096_d, B4p_ring[pj], 4, s4_d, None, act="gelu", out=C4096)
        act_ev[i][1].record()
    torch.cuda.synchronize()
    gelu_us = float(np.mean([e[0].elapsed_time(e[1]) for e in act_ev])) * 1e3

    # int4 weight preparation from fp16: the fused-QKV weight [12288, 4096]
    # quantized to the int4 code range, then packed (two launches).
    q4 = torch.empty(W.shape, dtype=torch.int8, device=dev)
    s4q = torch.empty((W.shape[0],), dtype=torch.float16, device=dev)
    p4 = torch.empty((W.shape[0], W.shape[1] // 2), dtype=torch.uint8, device=dev)
    prep_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.warmup):
        bq.quantize_rows_bits(W_d[i % len(W_d)], 4, q4, s4q)
        bq.pack_int4(q4, p4)
    torch.cuda.synchronize()
    hold_gpu()
    for i in range(args.steps):
        prep_ev[i][0].record()
        bq.quantize_rows_bits(W_d[i % len(W_d)], 4, q4, s4q)
        prep_ev[i][1].record()
        bq.pack_int4(q4, p4)
        prep_ev[i][2].record()
    torch.cuda.synchronize()
    prep_q_us = float(np.mean([e[0].elapsed_time(e[1]) for e in prep_ev])) * 1e3
    prep_p_us = float(np.mean([e[1].elapsed_time(e[2]) for e in prep_ev])) * 1e3
    prep_bytes = roofline.quantize_bytes(*W.shape) + roofline.pack_bytes(W.shape[0], W.shape[1], 4)
    # the same preparation in one pass (bq_quantize_pack): fp16 read once,
    # packed bytes and scales written once
    p4f = torch.empty_like(p4)
    s4f = torch.empty_like(s4q)
    for i in range(args.warmup):
        bq.quantize_pack(W_d[i % len(W_d)], 4, p4f, s4f)
    fused_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    hold_gpu()
    for i in range(args.steps):
        fused_ev[i][0].record()
        bq.quantize_pack(W_d[i % len(W_d)], 4, p4f, s4f)
        fused_ev[i][1].record()
    torch.cuda.synchronize()
    fused_us = float(np.mean([e[0].elapsed_time(e[1]) for e in fused_ev])) * 1e3
    fused_bytes = W.size * 2 + W.size // 2 + 2 * W.shape[0]

    # W4A16 with NF4 weight codes, per-row scale and zero point: decode
    # (M = 1, a stream over the codes, bound by HBM) and prefill (M = 4096,
    # fp16 matrix cores), N = K = 4096, code rings past the MALL.
    nf4_res = {}
    g16 = np.random.default_rng(7)
    s_nf = up(g16.uniform(0.001, 0.01, 4096).astype(np.float16))
    z_nf = up(g16.uniform(-0.05, 0.05, 4096).astype(np.float16))
    codes_nf = torch.from_numpy(g16.integers(0, 256, (4096, K // 2), dtype=np.uint8)).to(dev)
    nf_ring = ring(codes_nf, ring_len(codes_nf.numel()))
    for Mn in (1, 4096):
        A_nf = up(g16.standard_normal((Mn, K)).astype(np.float16))
        C_nf = torch.empty((Mn, 4096), dtype=torch.float16, device=dev)
        nf_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.warmup):
            bq.gemm_nf4_a16(A_nf, nf_ring[i % len(nf_ring)], s_nf, z_nf, out=C_nf)
        torch.cuda.synchronize()
        hold_gpu()
        for i in range(args.steps):
            nf_ev[i][0].record()
            bq.gemm_nf4_a16(A_nf, nf_ring[i % len(nf_ring)], s_nf, z_nf, out=C_nf)
            nf_ev[i][1].record()
        torch.cuda.synchronize()
        us = float(np.mean([e[0].elapsed_time(e[1]) for e in nf_ev])) * 1e3
        nbytes = roofline.nf4_gemm_bytes(Mn, 4096, K)
        flops = roofline.gemm_ops(Mn, 4096, K)
        key = "w4a16_nf4_m%d" % Mn
        if Mn == 1:
            nf4_res[key] = {"shape": [Mn, 4096, K], "kernel": "gemv_nf4_kernel", "us": round(us, 2),
                            "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / roofline.HBM_PEAK_BYTES_PER_S, 4)}
        else:
            nf4_res[key] = {"shape": [Mn, 4096, K], "kernel": "gemm_tiled_kernel (NF4 mode)", "us": round(us, 2),
                            "TFLOP_per_s": round(flops / (us * 1e-6) / 1e12, 1),
                            "frac_of_fp16_mfma_peak": round(flops / (us * 1e-6) / roofline.FP16_MFMA_PEAK_FLOPS, 4)}
        del A_nf, C_nf
    del nf_ring, codes_nf

    # The rest of the W4A8 M sweep at N = K = 4096 (M = 1 and 4096 are in the
    # step) and the decode GEMV at N = 11008, each launch on a different
    # packed B of a ring past the MALL, timed one launch at a time.
    def time_launches(fn, nring):
        for i in range(args.warmup):
            fn(i % nring)
        torch.cuda.synchronize()
        evs_l = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        hold_gpu()
        for i in range(args.steps):
            evs_l[i][0].record()
            fn((i + nring // 2) % nring)
            evs_l[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in evs_l])) * 1e3

    def perf(M_, N_, us, bits=4):
        ops, nbytes = roofline.gemm_ops(M_, N_, K), roofline.gemm_bytes(M_, N_, K, bits)
        b, _ = roofline.bound(ops, nbytes)
        gbs, tops = nbytes / (us * 1e-6), ops / (us * 1e-6)
        return {"shape": [M_, N_, K], "path": bq.select_path(M_, N_, K, bits), "us": round(us, 2),
                "GB_per_s": round(gbs / 1e9, 1), "TOPS": round(tops / 1e12, 2), "bound": b,
                "frac_of_bound": round(gbs / roofline.HBM_PEAK_BYTES_PER_S if b == "hbm"
                                       else tops / roofline.INT8_MFMA_PEAK_OPS_PER_S, 4)}

    sweep = {}
    for Ms in (16, 64, 256, 1024):
        A_s = A4096_d[:Ms]
        C_s = torch.empty((Ms, 4096), dtype=torch.float16, device=dev)
        us = time_launches(lambda r: bq.gemm_w4a8_dequant(A_s, B4p_ring[r], s4_d, C_s), len(B4p_ring))
        sweep["gemm_w4a8_m%d" % Ms] = perf(Ms, 4096, us)
        del C_s
    _, B11v, s11h = synth.w4a8_case(1, 11008, K, seed=0)
    s11 = up(s11h)
    B11 = torch.empty((11008, K // 2), dtype=torch.uint8, device=dev)
    bq.pack_int4(up(B11v), B11)
    del B11v
    B11_ring = ring(B11, ring_len(B11.numel()))
    C11 = torch.empty((1, 11008), dtype=torch.float16, device=dev)
    us = time_launches(lambda r: bq.gemm_w4a8_dequant(A1_d, B11_ring[r], s11, C11), len(B11_ring))
    sweep["gemm_w4a8_m1_n11008"] = perf(1, 11008, us)
    del B11_ring, B11
    # The small W4A8 case, M = 16, N = 256, K = 256 (launch-bound: time only).
    A0, B0v, s0 = synth.w4a8_case(16, 256, 256, seed=0)
    A0_d, s0_d = up(A0), up(s0)
    B0 = torch.empty((256, 128), dtype=torch.uint8, device=dev)
    bq.pack_int4(up(B0v), B0)
    C0 = torch.empty((16, 256), dtype=torch.float16, device=dev)
    us = time_launches(lambda r: bq.gemm_w4a8_dequant(A0_d, B0, s0_d, C0), 1)
    sweep["gemm_w4a8_16x256x256"] = {"shape": [16, 256, 256], "path": bq.select_path(16, 256, 256, 4),
                                     "us": round(us, 2), "bound": "launch"}
    del A0_d, B0, C0
    # Decode with the three projections of a fused QKV weight in one launch:
    # three int4 [4096, 4096] weights, one activation row broadcast to all.
    Bqkv = torch.stack([B4p_ring[0], B4p_ring[1], B4p_ring[2]])
    Bqkv_ring = ring(Bqkv, ring_len(Bqkv.numel()))
    sqkv = torch.stack([s4_d, s4_d, s4_d])
    Cqkv = torch.empty((3, 1, 4096), dtype=torch.float16, device=dev)
    us = time_launches(lambda r: bq.gemm_batched(A1_d, Bqkv_ring[r], 4, sqkv, out=Cqkv), len(Bqkv_ring))
    qkv1_bytes = 3 * roofline.gemm_bytes(1, 4096, K, 4) - 2 * K  # the activation row is read once
    sweep["gemm_w4a8_m1_qkv_batched"] = {
        "shape": [3, 1, 4096, K], "path": bq.select_path(1, 4096, K, 4), "us": round(us, 2),
        "GB_per_s": round(qkv1_bytes / (us * 1e-6) / 1e9, 1),
        "frac_of_bound": round(qkv1_bytes / (us * 1e-6) / roofline.HBM_PEAK_BYTES_PER_S, 4), "bound": "hbm"}
    del Bqkv_ring, Bqkv

    extras = {
        **nf4_res,
        "w4a8_sweep": sweep,
        "weight_prep_int4": {
            "shape": list(W.shape), "quantize_us": round(prep_q_us, 2), "pack_us": round(prep_p_us, 2),
            "GB_per_s": round(prep_bytes / ((prep_q_us + prep_p_us) * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(prep_bytes / ((prep_q_us + prep_p_us) * 1e-6)
                                      / roofline.HBM_PEAK_BYTES_PER_S, 4),
            "fused_us": round(fused_us, 2),
            "fused_GB_per_s": round(fused_bytes / (fused_us * 1e-6) / 1e9, 1),
            "fused_frac_of_hbm_peak": round(fused_bytes / (fused_us * 1e-6) / roofline.HBM_PEAK_BYTES_PER_S, 4),
        },
        "gemm_w4a8_m4096_gelu": {
            "shape": [4096, 4096, 4096], "us": round(gelu_us, 2),
            "TOPS": round(roofline.gemm_ops(4096, 4096, K) / (gelu_us * 1e-6) / 1e12, 2),
            "vs_plain_epilogue": round(mean_ms[names.index("gemm_w4a8_m4096")] * 1e3 / gelu_us, 4),
        },
        "qkv_batched_w8a8": {
            "shape": [3, Ml, 4096, Kl], "path": bq.select_path(Ml, 4096, Kl, 8), "us": round(qkv_us, 2),
            "GB_per_s": round(qkv_bytes / (qkv_us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(qkv_bytes / (qkv_us * 1e-6) / roofline.HBM_PEAK_BYTES_PER_S, 4),
        },
        "linear_w8a8_per_token": {
            "shape": [Ml, Nl, Kl], "path": bq.select_path(Ml, Nl, Kl, 8),
            "quantize_us": round(lin_q_us, 2), "gemm_us": round(lin_g_us, 2),
            "total_us": round(lin_q_us + lin_g_us, 2),
            "GB_per_s": round((lin_q_bytes + lin_g_bytes) / ((lin_q_us + lin_g_us) * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round((lin_q_bytes + lin_g_bytes) / ((lin_q_us + lin_g_us) * 1e-6)
                                      / roofline.HBM_PEAK_BYTES_PER_S, 4),
        },
    }

    kernel_path = {
        "quantize_rows": "quantize", "pack_int4": "pack", "pack_int2": "pack",
        "gemm_w8a8_m64": bq.select_path(64, 12288, K, 8),
        "gemm_w4a8_m1": bq.select_path(1, 4096, K, 4),
        "gemm_w4a8_m4096": bq.select_path(4096, 4096, K, 4),
        "gemm_w2a8_m1": bq.select_path(1, 4096, K, 2),
        "gemm_w2a8_m128": bq.select_path(128, 4096, K, 2),
    }

    # ---------------- algorithmic work per kernel ----------------
    work = {
        "quantize_rows": dict(shape=[12288, 4096], bytes=roofline.quantize_bytes(12288, 4096), ops=0),
        "gemm_w8a8_m64": dict(shape=[64, 12288, 4096], bytes=roofline.gemm_bytes(64, 12288, K, 8),
                              ops=roofline.gemm_ops(64, 12288, K)),
        "pack_int4": dict(shape=[4096, 4096], bytes=roofline.pack_bytes(4096, K, 4), ops=0),
        "gemm_w4a8_m1": dict(shape=[1, 4096, 4096], bytes=roofline.gemm_bytes(1, 4096, K, 4),
                             ops=roofline.gemm_ops(1, 4096, K)),
        "gemm_w4a8_m4096": dict(shape=[4096, 4096, 4096], bytes=roofline.gemm_bytes(4096, 4096, K, 4),
                                ops=roofline.gemm_ops(4096, 4096, K)),
        "pack_int2": dict(shape=[4096, 4096], bytes=roofline.pack_bytes(4096, K, 2), ops=0),
        "gemm_w2a8_m1": dict(shape=[1, 4096, 4096], bytes=roofline.gemm_bytes(1, 4096, K, 2),
                             ops=roofline.gemm_ops(1, 4096, K)),
        "gemm_w2a8_m128": dict(shape=[128, 4096, 4096], bytes=roofline.gemm_bytes(128, 4096, K, 2),
                               ops=roofline.gemm_ops(128, 4096, K)),
    }
    kernels = {}
    for j, n in enumerate(names):
        w = work[n]
        t = mean_ms[j] * 1e-3
        b, _ = roofline.bound(w["ops"], w["bytes"])
        gbs = w["bytes"] / t / 1e9
        tops = w["ops"] / t / 1e12
        p10, p50, p90 = np.percentile(dur_ms[:, j] * 1e3, [10, 50, 90])
        kernels[n] = {
            "shape": w["shape"], "us": round(mean_ms[j] * 1e3, 2),
            "us_min": round(dur_ms[:, j].min() * 1e3, 2),
            "us_p10": round(float(p10), 2), "us_p50": round(float(p50), 2), "us_p90": round(float(p90), 2),
            "GB_per_s": round(gbs, 1), "TOPS": round(tops, 2), "bound": b,
            "frac_of_bound": round(gbs * 1e9 / roofline.HBM_PEAK_BYTES_PER_S if b == "hbm"
                                   else tops * 1e12 / roofline.INT8_MFMA_PEAK_OPS_PER_S, 4),
        }

    head = kernels["gemm_w4a8_m4096"]
    gemv = kernels["gemm_w4a8_m1"]
    head_tops = head["TOPS"]
    roof = {
        "bound": "mfma", "kernel": "gemm_w4a8_m4096 (gemm_tiled_kernel, 256x256 tile, 8 waves)",
        "achieved": head_tops, "peak": roofline.INT8_MFMA_PEAK_OPS_PER_S / 1e12,
        "unit": "TOPS", "frac": round(head_tops * 1e12 / roofline.INT8_MFMA_PEAK_OPS_PER_S, 4),
        "us_per_launch": head["us"],
        "traffic": measured_traffic(),
        "algorithmic_bytes": work["gemm_w4a8_m4096"]["bytes"],
    }

    # Measured ceilings in the same run (box-to-box differences cancel in the
    # ratios): a plain 512 MiB device copy (read + write bytes), and the vendor
    # library's int8 GEMM at M = N = K = 4096 (torch._int_mm, i.e. hipBLASLt,
    # int8 x int8 -> int32; measurement context only, not used by the path)
    # beside this library's int8 x int8 -> int32 and W4A8 -> fp16 GEMMs, each
    # launch timed alone between two 64 MiB copies, as in the step.
    gap_src = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    gap_dst = torch.empty_like(gap_src)

    def time_alone(fn):
        for _ in range(args.warmup):
            fn()
        evs_c = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        hold_gpu()
        for i in range(args.steps):
            gap_dst.copy_(gap_src)
            evs_c[i][0].record()
            fn()
            evs_c[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in evs_c])) * 1e3

    cp_src = torch.empty(256 << 20, dtype=torch.float16, device=dev).fill_(1.0)
    cp_dst = torch.empty_like(cp_src)
    copy_us = time_alone(lambda: cp_dst.copy_(cp_src))
    copy_gbs = 2 * cp_src.numel() * 2 / (copy_us * 1e-6) / 1e9
    del cp_src, cp_dst
    B8 = q_ring[0][:4096]                      # int8 codes [4096, 4096]
    C32 = torch.empty((4096, 4096), dtype=torch.int32, device=dev)
    ops4096 = roofline.gemm_ops(4096, 4096, K)
    vendor_us = time_alone(lambda: torch._int_mm(A4096_d, B8.t()))
    own_i32_us = time_alone(lambda: bq.gemm_w8a8_i32(A4096_d, B8, out=C32))
    own_w4_us = time_alone(lambda: bq.gemm_w4a8_dequant(A4096_d, B4p_ring[0], s4_d, C4096))
    # Achievable ceilings of the box itself (libbq_calib.so, measurement
    # kernels only): int8 matrix-core instructions on register operands
    # (1024 workgroups of four wavefronts, four independent accumulators
    # each), and a plain streaming read of 1 GiB.
    import ctypes

    calib = ctypes.CDLL(lib_build.CALIB_LIB)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cal_out = torch.empty(2048 * 256, dtype=torch.int32, device=dev)
    loop_blocks, loop_iters = 1024, 4000

    def mfma_loop():
        rc = calib.bq_calib_mfma_loop(loop_blocks, loop_iters, ctypes.c_void_p(cal_out.data_ptr()), stream)
        if rc != 0:
            raise RuntimeError(f"bq_calib_mfma_loop: hip error {rc}")

    rd_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)

    def read_stream():
        rc = calib.bq_calib_read_stream(ctypes.c_void_p(rd_buf.data_ptr()), ctypes.c_int64(rd_buf.numel()), 2048,
                                        ctypes.c_void_p(cal_out.data_ptr()), stream)
        if rc != 0:
            raise RuntimeError(f"bq_calib_read_stream: hip error {rc}")

    loop_us = time_alone(mfma_loop)
    loop_tops = loop_blocks * 4 * loop_iters * 4 * 65536 / (loop_us * 1e-6) / 1e12
    read_us = time_alone(read_stream)
    read_gbs = rd_buf.numel() / (read_us * 1e-6) / 1e9
    del rd_buf, cal_out, C32, gap_src, gap_dst
    gemv_sus_gbs = work["gemm_w4a8_m1"]["bytes"] / (gemv_sustained_us * 1e-6) / 1e9
    ceilings = {
        "mfma_i8_loop": {"us": round(loop_us, 2), "TOPS": round(loop_tops, 2),
                         "frac_of_int8_peak": round(loop_tops * 1e12 / roofline.INT8_MFMA_PEAK_OPS_PER_S, 4)},
        "read_stream_1GiB": {"us": round(read_us, 2), "GB_per_s": round(read_gbs, 1),
                             "frac_of_hbm_peak": round(read_gbs * 1e9 / roofline.HBM_PEAK_BYTES_PER_S, 4)},
        "value_frac_of_mfma_loop": round(head_tops / loop_tops, 4),
        "gemv_m1_sustained_frac_of_read_stream": round(gemv_sus_gbs / read_gbs, 4),
        "device_copy_512MiB": {"us": round(copy_us, 2), "GB_per_s": round(copy_gbs, 1),
                               "frac_of_hbm_peak": round(copy_gbs * 1e9 / roofline.HBM_PEAK_BYTES_PER_S, 4)},
        "vendor_int8_gemm_4096": {"kernel": "torch._int_mm (hipBLASLt), int8 x int8 -> int32",
                                  "us": round(vendor_us, 2), "TOPS": round(ops4096 / (vendor_us * 1e-6) / 1e12, 2)},
        "own_w8a8_i32_4096": {"us": round(own_i32_us, 2), "TOPS": round(ops4096 / (own_i32_us * 1e-6) / 1e12, 2),
                              "vs_vendor": round(vendor_us / own_i32_us, 4)},
        "own_w4a8_f16_4096": {"us": round(own_w4_us, 2), "TOPS": round(ops4096 / (own_w4_us * 1e-6) / 1e12, 2),
                              "vs_vendor": round(vendor_us / own_w4_us, 4)},
        "gemv_m1_sustained_vs_copy": round(
            work["gemm_w4a8_m1"]["bytes"] / (gemv_sustained_us * 1e-6) / 1e9 / copy_gbs, 4),
        "quantize_vs_copy": round(kernels["quantize_rows"]["GB_per_s"] / copy_gbs, 4),
    }

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for n in names:
        kernels[n]["path"] = kernel_path[n]

    cpu = None
    cpu_configs = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(A4096, B4v, s4, args.cpu_seconds)
        gpu_us = {k: v["us"] for k, v in kernels.items()}
        gpu_us["gemm_w4a8_m1_n11008"] = sweep["gemm_w4a8_m1_n11008"]["us"]
        cpu_configs = cpu_oracle_configs(W, A64, A1, B4v, A2, B2v, s4, s2, gpu_us)

    line = {
        "metric": METRIC,
        "value": head_tops,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(gpu_ms_per_step, 4),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "launch_queue_prefilled": held,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "w4a8 dequant GEMM M=4096 N=4096 K=4096 within one pass of the path "
                        "(quantize 12288x4096, w8a8 M=64, pack int4/int2, w4a8 M=1 and 4096, "
                        "w2a8 M=1 and 128)",
            "M": 4096, "N": 4096, "K": 4096, "weight_bits": 4,
        },
        "gemv_m1": {"GB_per_s": gemv["GB_per_s"], "frac_of_hbm_peak": gemv["frac_of_bound"],
                    "us": gemv["us"], "shape": gemv["shape"],
                    "sustained_us": round(gemv_sustained_us, 3),
                    "sustained_GB_per_s": round(work["gemm_w4a8_m1"]["bytes"] / (gemv_sustained_us * 1e-6) / 1e9, 1)},
        "roofline": roof,
        "gemm_m4096_sustained": None if big_sustained_us is None else {
            "us": round(big_sustained_us, 2),
            "TOPS": round(work["gemm_w4a8_m4096"]["ops"] / (big_sustained_us * 1e-6) / 1e12, 2)},
        "cpu_baseline": cpu,
        "cpu_oracle_configs": cpu_configs,
        "kernels": kernels,
        "extras": extras,
        "ceilings": ceilings,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(A, Bv, s, budget_s):
    """The oracle (unpack -> integer GEMM -> dequant, as it stands) on a
    bounded sample of rows of the M = 4096 W4A8 workload, on the host cores."""
    import oracle

    Bp = oracle.pack_int4(Bv)
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))

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
    return {"value": round(ops / t / 1e12, 6), "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {A.shape[0]} rows of A (M={rows}, N={Bv.shape[0]}, K={Bv.shape[1]}, "
                      f"w4a8 dequant) x {reps}, {t:.1f} s"}


def cpu_oracle_configs(W, A64, A1, B4v, A2, B2v, s4, s2, gpu_us):
    """The oracle (as it stands, all host cores) on the other workloads of the
    step, each timed once beside the GPU kernel's in-step time."""
    import oracle

    from bit_mixed_precision_amd import synth

    out = {}

    def timed(name, fn, extra=""):
        t = time.perf_counter()
        fn()
        ms = (time.perf_counter() - t) * 1e3
        g = gpu_us.get(name)
        out[name] = {"oracle_ms": round(ms, 2), "gpu_us": g,
                     "speedup": round(ms * 1e3 / g, 1) if g else None}
        if extra:
            out[name]["note"] = extra

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
    # single-thread times of the quantize and the M <= 64 workloads, in a
    # child process (the thread count of the oracle's OpenMP is fixed at load)
    import subprocess

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


if __name__ == "__main__":
    main()
