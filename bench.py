"""Benchmark of the 4-bit GEMV / GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sections decode,gemm,affine,affine8,small,llama,cpu]
                    (also: crossover, calib; not in the default run)

A step is one decode token through the decode-GEMV workload (Q4_0 W
[12288, 4096], one bf16 activation [1, 4096] ~ N(0,1)): q4_gemv_act on W and
q4_gemv_fused2_act on a (gate, up) pair of the same shape, each quantising
the activation to Q8_1 on chip (the same bits as q8_1_quantize_act, whose
three-launch step is timed beside it under "extra").  The weights rotate through enough distinct copies
(>= 538 MB) that every step streams them from HBM, not from the 256 MB
last-level cache.  Steps run as replays of a HIP graph (as a decode loop
would), and `value` is the step's algorithmic bytes over the wall-clock time
of exactly K steps between two synchronisations (GB/s).  The roofline object
is q4_gemv_fused2_act's, the step's longest kernel: its mean duration over
back-to-back launches queued behind a GPU hold, bracketed by HIP events on
the launching stream.

The other sections add, under "extra": the prefill GEMM (Q4_0, M=2048,
TFLOP/s) against dequantise-then-GEMM, the affine-4 group-64 sweep over
M in {1, 32, 512, 2048, 8192} with its crossover, the same sweep for affine
8-bit weights, the small-M paths, and the Llama-3.2-1B-shaped
16-layer stack (aggregate tokens/s).  The CPU oracle is timed on the host
cores on bounded samples of the decode workload (`cpu_baseline`) and of the
prefill GEMM (under `extra.gemm_roofline`), at N=1 only.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from gemv_q4_affine_amd import binding as B  # noqa: E402
from gemv_q4_affine_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, TFLOP/s


# HBM bytes per launch of the roofline kernel (q4_gemv_fused2_act at the
# decode shape, k_q4_gemv<1,2,4,2,2,bf16>), from the rocprofv3 FETCH_SIZE /
# WRITE_SIZE passes summarised in profiles/q4_gemv_n12288_k4096_hbm_traffic.md.
# They hold only for the sources they were taken on: with any other source the
# figure is reported as null until the counters are taken again.
MEASURED_TRAFFIC = {"sources": ["gemv_q4_affine_amd/csrc/gemv.hip", "gemv_q4_affine_amd/csrc/device_common.hpp"],
                    "sha256_prefix": "c13c4d93c6d549bc", "bytes_per_launch": 56857411}


def sources_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    ok = sources_hash(MEASURED_TRAFFIC["sources"]) == MEASURED_TRAFFIC["sha256_prefix"]
    return MEASURED_TRAFFIC["bytes_per_launch"] if ok else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_dev(x_f32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(synth.bf16_bits(x_f32).view(np.int16)).cuda().view(torch.bfloat16)


def hold_gpu(us: float):
    """Keep the GPU busy for at least `us` microseconds (a spin kernel counting
    core cycles, sized for the highest clock) so that the host can queue a
    whole timed region behind it: the region then runs without launch gaps."""
    torch.cuda._sleep(int(us * 1e-6 * 2.4e9))


def region_us(fn, n: int, warmup: int = 3, hold_us: float | None = None) -> float:
    """Mean microseconds per call of fn(i), i < n, queued back to back behind a
    hold and bracketed by events on the current stream."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    hold = hold_us if hold_us is not None else 50.0 * n + 2000.0
    for _attempt in range(3):
        hold_gpu(hold)
        t0 = time.perf_counter()
        s.record()
        for i in range(n):
            fn(i)
        e.record()
        enqueue_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        if enqueue_us < 0.8 * hold:
            break
        hold = 2.0 * enqueue_us      # the host fell behind the hold: queue again with a longer one
    return s.elapsed_time(e) * 1e3 / n


def steady_us(fn, n: int, busy_ms: float = 150.0) -> float:
    """Mean microseconds per call of fn(i), i < n, in steady state: the same
    calls run back to back for about busy_ms first and the timed calls follow
    with no idle gap.  For long compute-bound kernels: after an idle or
    spinning GPU the clock takes milliseconds to settle under the power limit,
    which a short region behind a hold would include.  The host must queue a
    call faster than the GPU runs it (true above some tens of microseconds)."""
    fn(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(3):
        fn(i % n)
    torch.cuda.synchronize()
    one = max((time.perf_counter() - t0) / 3, 1e-6)
    for i in range(max(1, int(busy_ms * 1e-3 / one))):
        fn(i % n)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(n):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e3 / n


def graph_of(fns, stream):
    """A HIP graph of the launches made by fns() on `stream`."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fns:
            f()
    return g


def graph_region_us(g, launches_per_replay: int, replays: int) -> float:
    """Mean microseconds per launch over `replays` back-to-back replays of g."""
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    hold_gpu(20.0 * replays + 1000.0)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e3 / (replays * launches_per_replay)


# ---------------------------------------------------------------------------
# decode step (the headline workload)
# ---------------------------------------------------------------------------

def decode_section(steps: int, warmup: int, copies: int):
    wl = synth.DECODE
    N, K = wl.N, wl.K
    log(f"[decode] generating W [{N},{K}] x3 and x [1,{K}]")
    rng = np.random.default_rng(wl.seed)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, 1, K)
    Wg = synth.weights(rng, N, K)
    Wu = synth.weights(rng, N, K)
    x = bf16_dev(X)
    mats = []
    for Wm in (W, Wg, Wu):
        qs, d = B.q4_quantize(torch.from_numpy(Wm).cuda())
        mats.append((qs, d))
    del W, Wg, Wu
    # distinct copies so every step streams its weights from HBM
    rot = [[(qs.clone(), d.clone()) for (qs, d) in mats] for _ in range(copies)]
    torch.cuda.synchronize()
    xq = torch.empty((1, K), dtype=torch.int8, device="cuda")
    xd = torch.empty((1, K // 32, 2), dtype=torch.int16, device="cuda")
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y0 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")

    ya = torch.empty((1, N), dtype=torch.float32, device="cuda")
    ya0 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    ya1 = torch.empty((1, N), dtype=torch.float32, device="cuda")

    wbytes = N * K // 2 + N * (K // 32) * 2                 # one Q4_0 matrix: nibbles + binary16 d
    bytes_q8 = K * 2 + K + (K // 32) * 4
    bytes_gemv = wbytes + K + (K // 32) * 4 + N * 4
    bytes_f2 = 2 * wbytes + K + (K // 32) * 4 + 2 * N * 4
    bytes_gemv_act = wbytes + K * 2 + N * 4
    bytes_f2_act = 2 * wbytes + K * 2 + 2 * N * 4
    bytes_step_split = bytes_q8 + bytes_gemv + bytes_f2
    bytes_step = bytes_gemv_act + bytes_f2_act

    def q8(i):
        B.q8_1_quantize_act(x, xq, xd)

    def gemv(i):
        (wq, wd), _, _ = rot[i % copies]
        B.q4_gemv(wq, wd, xq, xd, y)

    def fused2(i):
        _, (gq, gd), (uq, ud) = rot[i % copies]
        B.q4_gemv_fused2(gq, gd, uq, ud, xq, xd, y0, y1)

    def gemv_act(i):
        (wq, wd), _, _ = rot[i % copies]
        B.q4_gemv_act(wq, wd, x, ya)

    def fused2_act(i):
        _, (gq, gd), (uq, ud) = rot[i % copies]
        B.q4_gemv_fused2_act(gq, gd, uq, ud, x, ya0, ya1)

    def step_split(i):
        q8(i)
        gemv(i)
        fused2(i)

    def step(i):
        gemv_act(i)
        fused2_act(i)

    # eager results: the one-launch-per-matrix step must give the bits of the
    # quantise-then-GEMV step
    step_split(0)
    step(0)
    torch.cuda.synchronize()
    assert torch.equal(ya, y) and torch.equal(ya0, y0) and torch.equal(ya1, y1), \
        "q4_gemv_act / q4_gemv_fused2_act differ from q8_1_quantize_act + q4_gemv / q4_gemv_fused2"
    ref = (ya.clone(), ya0.clone(), ya1.clone())
    side = torch.cuda.Stream()

    def timed_steps(fn):
        g_all = graph_of([(lambda i=i: fn(i)) for i in range(copies)], side)
        rem = steps % copies
        g_rem = graph_of([(lambda i=i: fn(i)) for i in range(rem)], side) if rem else None
        for _ in range(max(1, -(-warmup // copies))):
            g_all.replay()
        torch.cuda.synchronize()
        # whole-job timing: exactly `steps` steps between synchronisations
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for _ in range(steps // copies):
            g_all.replay()
        if g_rem is not None:
            g_rem.replay()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall * 1e3 / steps, ev0.elapsed_time(ev1) / steps

    ms_split, gpu_ms_split = timed_steps(step_split)
    ms_per_step, gpu_ms_per_step = timed_steps(step)
    step(0)
    torch.cuda.synchronize()
    assert torch.equal(ya, ref[0]) and torch.equal(ya0, ref[1]) and torch.equal(ya1, ref[2]), \
        "graph replays changed the decode results"

    # per-kernel launch durations: back-to-back launches of one kernel,
    # (a) as a graph over the copies, (b) eagerly queued behind a hold
    reps = max(1, 200 // copies)
    per = {}
    for name, fn in (("q8_1_quantize_act", q8), ("q4_gemv", gemv), ("q4_gemv_fused2", fused2),
                     ("q4_gemv_act", gemv_act), ("q4_gemv_fused2_act", fused2_act)):
        g = graph_of([(lambda i=i: fn(i)) for i in range(copies)], side)
        per[name] = {"us_graph": graph_region_us(g, copies, reps),
                     "us_eager": region_us(fn, reps * copies)}
        del g
    log(f"[decode] step {ms_per_step * 1e3:.2f} us wall ({gpu_ms_per_step * 1e3:.2f} us GPU), "
        f"quantise-then-GEMV step {ms_split * 1e3:.2f} us; kernels "
        + ", ".join(f"{k} {v['us_graph']:.2f}/{v['us_eager']:.2f} us" for k, v in per.items())
        + " (graph/eager)")

    def kern(name, nbytes):
        us = per[name]["us_eager"]
        return {"us": us, "bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9, **per[name]}

    return {
        "ms_per_step": ms_per_step,
        "gpu_ms_per_step": gpu_ms_per_step,
        "bytes_step": bytes_step,
        "gbs_step": bytes_step / (ms_per_step * 1e-3) / 1e9,
        "launch": "HIP graph of %d steps, replayed" % copies,
        "gemv_act": kern("q4_gemv_act", bytes_gemv_act),
        "fused2_act": kern("q4_gemv_fused2_act", bytes_f2_act),
        "quantise_then_gemv_step": {
            "ms_per_step": ms_split, "gpu_ms_per_step": gpu_ms_split, "bytes_step": bytes_step_split,
            "gbs_step": bytes_step_split / (ms_split * 1e-3) / 1e9,
            "gemv": kern("q4_gemv", bytes_gemv),
            "fused2": kern("q4_gemv_fused2", bytes_f2),
            "q8_1_quantize_act": {"bytes": bytes_q8, **per["q8_1_quantize_act"]},
        },
        "copies": copies,
        "rotated_bytes": copies * 3 * wbytes,
    }


# ---------------------------------------------------------------------------
# prefill GEMM (Q4_0, M = 2048) and dequantise-then-GEMM
# ---------------------------------------------------------------------------

def gemm_section(iters: int):
    wl = synth.PREFILL
    M, N, K = wl.M, wl.N, wl.K
    log(f"[gemm] M={M} N={N} K={K}")
    W, X = synth.workload_inputs(wl)
    qs, d = B.q4_quantize(torch.from_numpy(W).cuda())
    x = bf16_dev(X)
    del W, X
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(B.q4_gemm_workspace_size(M, N, K), dtype=torch.uint8, device="cuda")
    flop = 2.0 * M * N * K
    fused_ms = steady_us(lambda i: B.q4_gemm(qs, d, x, y=y, workspace=ws), iters) * 1e-3
    # the same matrix-core GEMM on a weight image prepared once
    image = B.q4_pack_weight_image(qs, d)
    xws = torch.empty(B.lib().q4_gemm_image_workspace_size(M, K), dtype=torch.uint8, device="cuda")
    image_ms = steady_us(lambda i: B.q4_gemm_image(image, x, N, y=y, workspace=xws), iters) * 1e-3
    # dequantise-then-GEMM: our dequantiser, then (a) the library's dense MFMA
    # GEMM on fp16 W, (b) hipBLASLt through torch on bf16 W (the pages' "jit")
    w16 = torch.empty((N, K), dtype=torch.float16, device="cuda")
    wbf = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    deq16_ms = steady_us(lambda i: B.q4_dequantize(qs, d, out=w16), iters) * 1e-3
    deqbf_ms = steady_us(lambda i: B.q4_dequantize(qs, d, out_dtype=torch.bfloat16, out=wbf), iters) * 1e-3
    dense_ms = steady_us(lambda i: B.dense_gemm(x, w16, y=y), iters) * 1e-3
    blas_bf16_ms = steady_us(lambda i: torch.matmul(x, wbf.t(), out=y), iters) * 1e-3
    x16 = x.to(torch.float16)
    y16 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    blas_f16_ms = steady_us(lambda i: torch.matmul(x16, w16.t(), out=y16), iters) * 1e-3
    best_deq = deq16_ms + min(dense_ms, blas_f16_ms)
    # the integer-dot form on the int8 matrix cores: X quantised to Q8_1, then
    # q4_gemm_q8 (also what q4_gemm runs with the INT8 path forced)
    xq, xds = B.q8_1_quantize_act(x)
    q8_ms = steady_us(lambda i: B.q4_gemm_q8(qs, d, xq, xds, y=y), iters) * 1e-3
    q8_quant_ms = steady_us(lambda i: B.q8_1_quantize_act(x, xq, xds), iters) * 1e-3
    res = {
        "fused_us": fused_ms * 1e3,
        "fused_tflops": flop / (fused_ms * 1e-3) / 1e12,
        "image_us": image_ms * 1e3,
        "image_tflops": flop / (image_ms * 1e-3) / 1e12,
        "dequant_f16_us": deq16_ms * 1e3,
        "dequant_bf16_us": deqbf_ms * 1e3,
        "dense_gemm_f16_us": dense_ms * 1e3,
        "hipblaslt_bf16_us": blas_bf16_ms * 1e3,
        "hipblaslt_f16_us": blas_f16_ms * 1e3,
        "jit_bf16_us": (deqbf_ms + blas_bf16_ms) * 1e3,
        "dequant_then_gemm_best_us": best_deq * 1e3,
        "fused_vs_dequant_then_gemm": best_deq / fused_ms,
        "int8_gemm_q8_us": q8_ms * 1e3,
        "int8_gemm_q8_tops": flop / (q8_ms * 1e-3) / 1e12,
        "int8_q8_1_quantize_us": q8_quant_ms * 1e3,
        "flop": flop,
    }
    log(f"[gemm] fused {res['fused_us']:.1f} us = {res['fused_tflops']:.0f} TFLOP/s; "
        f"prepacked weights {res['image_us']:.1f} us = {res['image_tflops']:.0f} TFLOP/s; "
        f"dequant f16 {res['dequant_f16_us']:.1f} us; dense {res['dense_gemm_f16_us']:.1f} us; "
        f"hipBLASLt bf16 {res['hipblaslt_bf16_us']:.1f} us, f16 {res['hipblaslt_f16_us']:.1f} us; "
        f"int8 MFMA (Q8_1 X) {res['int8_gemm_q8_us']:.1f} us + quantise {res['int8_q8_1_quantize_us']:.1f} us")
    return res


# ---------------------------------------------------------------------------
# affine 4-bit sweep
# ---------------------------------------------------------------------------

def affine_section(iters: int):
    wl = synth.AFFINE
    N, K = wl.N, wl.K
    rng = np.random.default_rng(wl.seed)
    W = synth.weights(rng, N, K)
    q, s, b = B.affine4_quantize(bf16_dev(W))
    del W
    wbf = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    w16 = torch.empty((N, K), dtype=torch.float16, device="cuda")
    B.affine4_dequantize(q, s, b, out_dtype=torch.bfloat16, out=wbf)
    image = B.q4_pack_weight_image(q, s, b)        # weights prepared once
    out = []
    for M in synth.AFFINE_MS:
        W_, X = synth.workload_inputs(wl, M=M)
        del W_
        x = bf16_dev(X)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        wsn = B.q4_gemm_workspace_size(M, N, K, B.Q4_FMT_AFFINE4)
        ws = torch.empty(wsn, dtype=torch.uint8, device="cuda") if wsn else None
        it = max(5, min(iters, int(2000 / max(1, M // 32))))
        # compute-bound sizes are timed in steady state, the short calls behind a hold
        timer = steady_us if M >= 512 else region_us
        fused = timer(lambda i: B.affine4_gemm(q, s, b, x, y=y, workspace=ws), it) * 1e-3
        fused_img = None
        if M > 32:      # the matrix-core path (smaller M takes the skinny kernels, which need no image)
            wsi = torch.empty(max(B.q4_gemm_workspace_size(M, N, K, B.Q4_FMT_AFFINE4), 16), dtype=torch.uint8,
                              device="cuda")
            fused_img = timer(lambda i: B.q4_gemm_image(image, x, N, fmt=B.Q4_FMT_AFFINE4, y=y, workspace=wsi),
                                  it) * 1e-3
        deq16 = timer(lambda i: B.affine4_dequantize(q, s, b, out=w16), it) * 1e-3
        deqbf = timer(lambda i: B.affine4_dequantize(q, s, b, out_dtype=torch.bfloat16, out=wbf), it) * 1e-3
        ref = timer(lambda i: torch.matmul(x, wbf.t(), out=y), it) * 1e-3
        dense = timer(lambda i: B.dense_gemm(x, w16, y=y), it) * 1e-3
        flop = 2.0 * M * N * K
        byts = N * K // 2 + 2 * N * (K // 64) * 2 + M * K * 2 + M * N * 2
        t_roof = max(byts / (HBM_PEAK_GBS * 1e9), flop / (F16_MFMA_PEAK_TFLOPS * 1e12))
        rec = {
            "M": M,
            "fused_us": fused * 1e3,                   # affine4_gemm per call (repacks the weights at M > 32)
            "fused_prepared_image_us": fused_img * 1e3 if fused_img is not None else fused * 1e3,
            "jit_us": (deqbf + ref) * 1e3,            # dequantise to bf16 + hipBLASLt bf16
            "ref_us": ref * 1e3,                       # hipBLASLt on pre-dequantised bf16 W
            "dequant_dense_f16_us": (deq16 + dense) * 1e3,
            "tflops": flop / (fused * 1e-3) / 1e12,
            "gbs": byts / (fused * 1e-3) / 1e9,
            "roofline_frac": t_roof / (fused * 1e-3),
            "fused_beats_jit": fused < deqbf + ref,
            "fused_prepared_image_beats_jit": (fused_img if fused_img is not None else fused) < deqbf + ref,
        }
        out.append(rec)
        log(f"[affine] M={M}: fused {rec['fused_us']:.1f} us (prepared image {rec['fused_prepared_image_us']:.1f}), "
            f"jit {rec['jit_us']:.1f} us, "
            f"ref {rec['ref_us']:.1f} us, dequant + dense_gemm {rec['dequant_dense_f16_us']:.1f} us, "
            f"roofline {rec['roofline_frac']:.2f}")
    crossover = next((rec["M"] for rec in out if not rec["fused_beats_jit"]), None)
    crossover_img = next((rec["M"] for rec in out if not rec["fused_prepared_image_beats_jit"]), None)
    return {"sweep": out, "first_M_where_dequant_then_gemm_wins": crossover,
            "first_M_where_dequant_then_gemm_wins_over_prepared_images": crossover_img}


# ---------------------------------------------------------------------------
# affine 8-bit sweep: the same shapes at bits=8
# ---------------------------------------------------------------------------

def affine8_section(iters: int):
    """affine8_gemm (fused up to M = 32 on bf16 X, the matrix-core GEMM on images above; also
    forced dequantise-then-GEMM there) against the page's jit (dequantise to bf16 + hipBLASLt) and ref (hipBLASLt on bf16 W
    dequantised once), at the sweep's M values.  At M = 1 the weights rotate
    over ten copies (535 MB) so that they stream from HBM."""
    wl = synth.AFFINE
    N, K = wl.N, wl.K
    rng = np.random.default_rng(wl.seed)
    W = synth.weights(rng, N, K)
    q, s, b = B.affine8_quantize(bf16_dev(W))
    del W
    copies = 10
    qc = [(q.clone(), s.clone(), b.clone()) for _ in range(copies)]
    wbf = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    B.affine8_dequantize(q, s, b, out_dtype=torch.bfloat16, out=wbf)
    image = B.q4_pack_weight_image(q, s, b, fmt=B.Q4_FMT_AFFINE8)     # weights prepared once
    out = []
    for M in sorted(set(synth.AFFINE_MS) | {16}):
        X = synth.activations(rng, M, K)
        x = bf16_dev(X)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        wsn = B.lib().affine8_gemm_workspace_size(M, N, K)
        ws = torch.empty(wsn, dtype=torch.uint8, device="cuda") if wsn else None
        it = max(5, min(iters, int(2000 / max(1, M // 32))))
        timer = steady_us if M >= 512 else region_us
        fused = timer(lambda i: B.affine8_gemm(*qc[i % copies], x, y=y, workspace=ws), it) * 1e-3
        deq_path = None
        fused_img = None
        if M > 32:
            wsi = torch.empty(max(B.q4_gemm_workspace_size(M, N, K, B.Q4_FMT_AFFINE8), 16), dtype=torch.uint8,
                              device="cuda")
            fused_img = timer(lambda i: B.q4_gemm_image(image, x, N, fmt=B.Q4_FMT_AFFINE8, y=y, workspace=wsi),
                              it) * 1e-3
            del wsi
            wsd = torch.empty(N * K * 2, dtype=torch.uint8, device="cuda")
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_DEQUANT_GEMM)
            try:
                deq_path = timer(lambda i: B.affine8_gemm(*qc[i % copies], x, y=y, workspace=wsd), it) * 1e-3
            finally:
                B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
            del wsd
        deqbf = timer(lambda i: B.affine8_dequantize(*qc[i % copies], out_dtype=torch.bfloat16, out=wbf), it) * 1e-3
        ref = timer(lambda i: torch.matmul(x, wbf.t(), out=y), it) * 1e-3
        flop = 2.0 * M * N * K
        byts = N * K + 2 * N * (K // 64) * 2 + M * K * 2 + M * N * 2
        t_roof = max(byts / (HBM_PEAK_GBS * 1e9), flop / (F16_MFMA_PEAK_TFLOPS * 1e12))
        rec = {
            "M": M,
            "path": "fused vector" if M <= 4 else ("fused bf16 MFMA" if M <= 32 else
                                                   "matrix-core GEMM on X and weight images (both built per call)"),
            "affine8_gemm_us": fused * 1e3,
            "forced_dequant_gemm_us": deq_path * 1e3 if deq_path is not None else None,
            "prepared_image_us": fused_img * 1e3 if fused_img is not None else None,
            "prepared_image_beats_jit": (fused_img if fused_img is not None else fused) < deqbf + ref,
            "jit_us": (deqbf + ref) * 1e3,
            "ref_us": ref * 1e3,
            "gbs": byts / (fused * 1e-3) / 1e9,
            "tflops": flop / (fused * 1e-3) / 1e12,
            "roofline_frac": t_roof / (fused * 1e-3),
            "affine8_gemm_beats_jit": fused < deqbf + ref,
        }
        out.append(rec)
        dq = (f", prepared image {fused_img * 1e3:.1f} us, forced dequant + dense GEMM {deq_path * 1e3:.1f} us"
              if deq_path is not None else "")
        log(f"[affine8] M={M}: affine8_gemm {rec['affine8_gemm_us']:.1f} us ({rec['path']}){dq}, "
            f"jit {rec['jit_us']:.1f} us, ref {rec['ref_us']:.1f} us, roofline {rec['roofline_frac']:.2f}")
    return {"sweep": out}


# ---------------------------------------------------------------------------
# small M: q4_gemm / affine4_gemm on the skinny paths
# ---------------------------------------------------------------------------

SMALL_MS = (1, 2, 4, 8, 16, 32, 48, 64)


def small_section(iters: int):
    """q4_gemm and affine4_gemm at small M on the prefill weight shape (the
    skinny paths: the vector kernel at M = 1, the bf16-MFMA kernel above),
    against dequantise-to-bf16 + hipBLASLt.  Bound: HBM (weights + X + Y)."""
    wl = synth.PREFILL
    N, K = wl.N, wl.K
    rng = np.random.default_rng(wl.seed)
    W = synth.weights(rng, N, K)
    wd = bf16_dev(W)
    qs, d = B.q4_quantize(wd)
    aq, asc, abi = B.affine4_quantize(wd)
    del W, wd
    # ten copies of each (283 MB) rotate so that the weights stream from HBM,
    # not from the 256 MB last-level cache
    copies = 10
    q4c = [(qs.clone(), d.clone()) for _ in range(copies)]
    afc = [(aq.clone(), asc.clone(), abi.clone()) for _ in range(copies)]
    wbf = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    out = []
    for M in SMALL_MS:
        X = synth.activations(rng, M, K)
        x = bf16_dev(X)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        rec = {"M": M}
        for name, wbytes, run, deq in (
            ("q4_0", N * K // 2 + N * (K // 32) * 2,
             lambda i: B.q4_gemm(*q4c[i % copies], x, y=y, workspace=None),
             lambda i: B.q4_dequantize(*q4c[i % copies], out_dtype=torch.bfloat16, out=wbf)),
            ("affine4", N * K // 2 + 2 * N * (K // 64) * 2,
             lambda i: B.affine4_gemm(*afc[i % copies], x, y=y, workspace=None),
             lambda i: B.affine4_dequantize(*afc[i % copies], out_dtype=torch.bfloat16, out=wbf)),
        ):
            fused = min(region_us(run, iters) for _ in range(2))
            jit = region_us(deq, iters) + region_us(lambda i: torch.matmul(x, wbf.t(), out=y), iters)
            byts = wbytes + M * K * 2 + M * N * 2
            rec[name] = {"us": fused, "gbs": byts / (fused * 1e-6) / 1e9,
                         "roofline_frac": byts / (fused * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "dequant_bf16_hipblaslt_us": jit, "beats_dequant_then_gemm": fused < jit}
        out.append(rec)
        log(f"[small] M={M}: q4_0 {rec['q4_0']['us']:.2f} us ({rec['q4_0']['roofline_frac']:.2f}), "
            f"affine4 {rec['affine4']['us']:.2f} us ({rec['affine4']['roofline_frac']:.2f}); "
            f"dequant+hipBLASLt {rec['q4_0']['dequant_bf16_hipblaslt_us']:.1f} / "
            f"{rec['affine4']['dequant_bf16_hipblaslt_us']:.1f} us")
    return {"N": N, "K": K, "copies": copies, "sweep": out}


CROSS_MS = (16, 17, 24, 32, 33, 40, 48, 64, 65, 96, 128, 129)


def crossover_section(iters: int):
    """q4_gemm and affine4_gemm on N=12288, K=4096 around the skinny / matrix-core
    crossover: the automatic choice and each path forced, on bf16 and binary32
    X, with the workspace q4_gemm_workspace_size asks for and without one.
    These are the measurements the default thresholds rest on (not a default
    section: the bench line does not use them)."""
    wl = synth.PREFILL
    N, K = wl.N, wl.K
    rng = np.random.default_rng(wl.seed)
    wd = bf16_dev(synth.weights(rng, N, K))
    copies = 10
    fmts = {"q4_0": (B.Q4_FMT_Q4_0, B.q4_gemm, B.q4_quantize(wd)),
            "affine4": (B.Q4_FMT_AFFINE4, B.affine4_gemm, B.affine4_quantize(wd))}
    del wd
    out = []
    for M in CROSS_MS:
        X = synth.activations(rng, M, K)
        xs = {"bf16": bf16_dev(X), "f32": torch.from_numpy(X).cuda()}
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        for name, (f, gemm, planes) in fmts.items():
            rot = [tuple(t.clone() for t in planes) for _ in range(copies)]
            ws = torch.empty(max(16, B.q4_gemm_workspace_size(M, N, K, f)), dtype=torch.uint8, device="cuda")
            B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, B.Q4_PATH_MFMA)
            try:
                nm = B.q4_gemm_workspace_size(M, N, K, f)      # the matrix-core path's bytes
            finally:
                B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)
            wsm = torch.empty(max(16, nm), dtype=torch.uint8, device="cuda")
            for xn, x in xs.items():
                rec = {"M": M, "format": name, "x": xn}

                def t(force, w):
                    B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, force)
                    try:
                        return round(min(region_us(lambda i: gemm(*rot[i % copies], x, y=y, workspace=w), iters)
                                         for _ in range(2)), 2)
                    finally:
                        B.q4_set_dispatch(B.Q4_KEY_FORCE_PATH, -1)

                rec["auto_ws_us"] = t(-1, ws)
                rec["auto_no_ws_us"] = t(-1, None)
                rec["skinny_us"] = t(B.Q4_PATH_SKINNY, None) if M <= 64 else None
                rec["mfma_images_us"] = t(B.Q4_PATH_MFMA, wsm)
                rec["mfma_no_ws_us"] = t(B.Q4_PATH_MFMA, None)
                out.append(rec)
                log(f"[crossover] {name} {xn} M={M}: auto {rec['auto_ws_us']} (no workspace "
                    f"{rec['auto_no_ws_us']}), skinny {rec['skinny_us']}, matrix-core on images "
                    f"{rec['mfma_images_us']}, without {rec['mfma_no_ws_us']} us")
            del rot
    return {"N": N, "K": K, "copies": copies, "sweep": out}


# ---------------------------------------------------------------------------
# Llama-3.2-1B-shaped 16-layer stack
# ---------------------------------------------------------------------------

def llama_section(iters: int):
    rng = np.random.default_rng(0)
    L = synth.LLAMA1B_LAYERS
    layers = []
    total_bytes = 0
    flop512 = 0.0
    for _ in range(L):
        lw = {}
        for name, (n, k) in synth.LLAMA1B_SHAPES.items():
            qs, d = B.q4_quantize(torch.from_numpy(synth.weights(rng, n, k)).cuda())
            lw[name] = (qs, d)
            total_bytes += n * k // 2 + n * (k // 32) * 2
            flop512 += 2.0 * 512 * n * k
        layers.append(lw)
    torch.cuda.synchronize()
    H, F = 2048, 8192
    xs = {k: bf16_dev(synth.activations(rng, 1, k)) for k in (H, F)}
    yb = {n: torch.empty((1, n), dtype=torch.float32, device="cuda") for n in (512, 2048, 8192)}
    yb2 = {n: torch.empty((1, n), dtype=torch.float32, device="cuda") for n in (512, 8192)}

    # per layer: (q, k, v), o, (gate, up), down -- one launch per group of
    # matrices that share an activation; each GEMV quantises its bf16
    # activation on chip
    yqkv = [yb[2048], yb[512], yb2[512]]
    def decode_token(_i):
        for lw in layers:
            B.q4_gemv_multi_act([lw["q"], lw["k"], lw["v"]], xs[H], yqkv)
            B.q4_gemv_act(*lw["o"], xs[H], yb[2048])
            B.q4_gemv_fused2_act(*lw["gate"], *lw["up"], xs[H], yb[8192], yb2[8192])
            B.q4_gemv_act(*lw["down"], xs[F], yb[2048])

    side = torch.cuda.Stream()
    g_tok = graph_of([lambda: decode_token(0)], side)
    decode_ms = graph_region_us(g_tok, 1, iters) * 1e-3
    # prefill, M = 512
    Mp = 512
    xp = {k: bf16_dev(synth.activations(rng, Mp, k)) for k in (H, F)}
    yp = {n: torch.empty((Mp, n), dtype=torch.bfloat16, device="cuda") for n in (512, 2048, 8192)}

    wsn = max(B.q4_gemm_workspace_size(Mp, n, k) for (n, k) in synth.LLAMA1B_SHAPES.values())
    ws = torch.empty(max(wsn, 16), dtype=torch.uint8, device="cuda")

    names = ("q", "k", "v", "o", "gate", "up", "down")

    def prefill_per_call(_i):
        # q4_gemm on the raw planes: each call also repacks the weights
        for lw in layers:
            for name in names:
                qs, d = lw[name]
                B.q4_gemm(qs, d, xp[d.shape[1] * 32], y=yp[d.shape[0]], workspace=ws)

    # weights prepared once, as a model loader would (q4_pack_weight_image);
    # the workspace has room for the split-K partial results of the small
    # matrices
    images = [{name: B.q4_pack_weight_image(*lw[name]) for name in names} for lw in layers]

    def prefill_separate(_i):
        for lw, im in zip(layers, images):
            for name in names:
                n, kb = lw[name][1].shape
                B.q4_gemm_image(im[name], xp[kb * 32], n, y=yp[n], workspace=ws)

    # the loader's usual fusion for prefill: q|k|v and gate|up concatenated
    # along N into one weight each (the Q4_0 planes stacked by rows), so a
    # layer is four GEMMs: qkv [3072 x 2048], o, gate|up [16384 x 2048], down
    def stack(names_):
        return (torch.cat([lw_[n_][0] for n_ in names_]), torch.cat([lw_[n_][1] for n_ in names_]))
    fused = []
    for lw_ in layers:
        fused.append({"qkv": B.q4_pack_weight_image(*stack(("q", "k", "v"))),
                      "o": images[len(fused)]["o"],
                      "gateup": B.q4_pack_weight_image(*stack(("gate", "up"))),
                      "down": images[len(fused)]["down"]})
    yqkv_p = torch.empty((Mp, 3072), dtype=torch.bfloat16, device="cuda")
    ygu_p = torch.empty((Mp, 16384), dtype=torch.bfloat16, device="cuda")
    wsf = torch.empty(max(B.q4_gemm_workspace_size(Mp, n, k) for (n, k) in ((3072, H), (2048, H), (16384, H), (2048, F))),
                      dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def prefill(_i):
        for fm in fused:
            B.q4_gemm_image(fm["qkv"], xp[H], 3072, y=yqkv_p, workspace=wsf)
            B.q4_gemm_image(fm["o"], xp[H], 2048, y=yp[2048], workspace=wsf)
            B.q4_gemm_image(fm["gateup"], xp[H], 16384, y=ygu_p, workspace=wsf)
            B.q4_gemm_image(fm["down"], xp[F], 2048, y=yp[2048], workspace=wsf)

    prefill_call_ms = steady_us(prefill_per_call, max(3, iters // 4)) * 1e-3
    prefill_sep_ms = steady_us(prefill_separate, max(3, iters // 4)) * 1e-3
    prefill_ms = steady_us(prefill, max(3, iters // 4)) * 1e-3
    res = {
        "decode_tokens_per_s": 1e3 / decode_ms,
        "decode_us_per_token": decode_ms * 1e3,
        "decode_weight_gbs": total_bytes / (decode_ms * 1e-3) / 1e9,
        "prefill_tokens_per_s": Mp * 1e3 / prefill_ms,
        "prefill_tflops": flop512 / (prefill_ms * 1e-3) / 1e12,
        "prefill_separate_matrices_tokens_per_s": Mp * 1e3 / prefill_sep_ms,
        "prefill_separate_matrices_tflops": flop512 / (prefill_sep_ms * 1e-3) / 1e12,
        "prefill_repacking_per_call_tokens_per_s": Mp * 1e3 / prefill_call_ms,
        "prefill_repacking_per_call_tflops": flop512 / (prefill_call_ms * 1e-3) / 1e12,
        "weights_bytes": total_bytes,
        "launches": "decode: one HIP graph per token, 4 GEMV launches per layer (q4_gemv_multi_act on q/k/v, "
                    "q4_gemv_act, q4_gemv_fused2_act); prefill: eager q4_gemm_image launches on weight images "
                    "prepared once (q|k|v and gate|up stacked into one weight each: 4 GEMMs per layer), queued "
                    "back to back; also the 7 separate matrices on images, and q4_gemm repacking every call",
    }
    log(f"[llama] decode {res['decode_tokens_per_s']:.0f} tok/s ({res['decode_weight_gbs']:.0f} GB/s); "
        f"prefill {res['prefill_tokens_per_s']:.0f} tok/s ({res['prefill_tflops']:.0f} TFLOP/s), "
        f"separate matrices {res['prefill_separate_matrices_tokens_per_s']:.0f} tok/s "
        f"({res['prefill_separate_matrices_tflops']:.0f} TFLOP/s), "
        f"repacking per call {res['prefill_repacking_per_call_tokens_per_s']:.0f} tok/s "
        f"({res['prefill_repacking_per_call_tflops']:.0f} TFLOP/s)")
    return res


# ---------------------------------------------------------------------------
# counter calibration: a plain streaming kernel of known size
# ---------------------------------------------------------------------------

def calib_section():
    """torch.neg over 64 Mi float32 values: reads 256 MiB and writes 256 MiB,
    the reference for scaling the FETCH_SIZE / WRITE_SIZE counters of the
    same rocprofv3 run (the buffers are larger than the last-level cache)."""
    n = 64 << 20
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return {"kernel": "torch.neg float32, 64 Mi elements", "read_bytes": 4 * n, "write_bytes": 4 * n}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores, bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(budget_s: float):
    import oracle
    wl = synth.DECODE
    N, K = wl.N, wl.K
    W, X = synth.workload_inputs(wl)
    Xb = synth.bf16_bits_to_f32(synth.bf16_bits(X))
    wqs, wd = oracle.q4_0_quantize(W)
    bytes_gemv = N * K // 2 + N * (K // 32) * 2 + K + (K // 32) * 4 + N * 4
    reps = 0
    t0 = time.perf_counter()
    while True:
        xqs, xds = oracle.q8_1_quantize(Xb)
        oracle.q4q8_gemv(wqs, wd, xqs, xds)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {
        "value": bytes_gemv * reps / el / 1e9,
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"decode GEMV M=1 N={N} K={K} (Q8_1 quantise + int32 block dots + fp64 accumulate), "
                  f"{reps} repetitions in {el:.1f} s",
    }


def cpu_baseline_gemm(budget_s: float):
    """The oracle on the prefill GEMM (Q4_0 W [12288, 4096], bf16 X [2048, 4096]):
    dequantise W once, then the fp64 matmul on a sample of X rows, grown until
    it runs for about budget_s; the full call's time is the dequantisation plus
    the sample's matmul time scaled linearly to 2048 rows (every row costs the
    same N*K multiply-adds)."""
    import oracle
    wl = synth.PREFILL
    M, N, K = wl.M, wl.N, wl.K
    W, X = synth.workload_inputs(wl)
    Xf = synth.bf16_bits_to_f32(synth.bf16_bits(X)).astype(np.float64)
    qs, d = oracle.q4_0_quantize(W)
    del W
    t0 = time.perf_counter()
    What = oracle.q4_0_dequantize(qs, d)
    t_deq = time.perf_counter() - t0
    rows, t_mm = 2, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.matmul_f64(Xf[:rows], What)
        t_mm = time.perf_counter() - t0
        if t_mm >= budget_s / 4 or rows >= M:
            break
        rows = min(M, rows * max(2, int(budget_s / 4 / max(t_mm, 1e-3))))
    t_full = t_deq + t_mm * M / rows
    flop = 2.0 * M * N * K
    return {
        "value": flop / t_full / 1e9,
        "unit": "GFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"prefill GEMM M={M} N={N} K={K}: dequantise ({t_deq * 1e3:.1f} ms) + fp64 matmul on {rows} of "
                  f"{M} X rows ({t_mm:.2f} s), matmul scaled linearly to {M} rows: {t_full:.1f} s per call",
    }


def environment():
    """ROCm, HIP runtime/driver and torch versions, and a hash of the library
    sources (the GPU machine's copy of the tree carries no git metadata; the git
    commit is added when there is one)."""
    import ctypes
    import glob
    import subprocess
    env = {"torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipRuntimeGetVersion(ctypes.byref(v)) == 0:
            env["hip_runtime_version"] = v.value
        if hip.hipDriverGetVersion(ctypes.byref(v)) == 0:
            env["hip_driver_version"] = v.value
    except OSError:
        pass
    srcs = sorted(glob.glob(os.path.join(ROOT, "gemv_q4_affine_amd", "csrc", "*"))) + [os.path.join(ROOT, "include", "q4.h")]
    env["library_sources_sha256_16"] = sources_hash([os.path.relpath(p, ROOT) for p in srcs])
    try:
        env["git_commit"] = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                                           timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        env["git_commit"] = None
    if env["git_commit"] is None:
        # a copy of the tree without git metadata: the commit the library was built from
        try:
            with open(os.path.join(ROOT, "gemv_q4_affine_amd", "build_info.json")) as f:
                info = json.load(f)
            env["git_commit"] = info.get("git_commit")
            env["library_built_from_modified_tree"] = info.get("tree_modified")
        except (OSError, ValueError):
            pass
    env["device"] = torch.cuda.get_device_name(0)
    env["host_cpus_in_affinity"] = len(os.sched_getaffinity(0))
    return env


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=20,
                    help="distinct weight copies rotated through (>= 19 keeps the 256 MB cache out)")
    ap.add_argument("--sections", default="decode,gemm,affine,affine8,small,llama,cpu",
                    help="comma list of decode (always run), gemm, affine, small, llama, cpu, calib")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    sections = set(args.sections.split(","))
    torch.cuda.init()
    log(f"[bench] {torch.cuda.get_device_name(0)}; {B.version()}")

    dec = decode_section(args.steps, args.warmup, args.copies)
    extra = {"decode": dec}
    if "gemm" in sections:
        extra["gemm_m2048"] = gemm_section(20)
    if "affine" in sections:
        extra["affine4_sweep"] = affine_section(20)
    if "affine8" in sections:
        extra["affine8_sweep"] = affine8_section(20)
    if "small" in sections:
        extra["small_m"] = small_section(100)
    if "llama" in sections:
        extra["llama1b_stack"] = llama_section(20)
    if "crossover" in sections:
        extra["small_m_crossover"] = crossover_section(40)
    if "calib" in sections:
        extra["counter_calibration"] = calib_section()
    cpu = cpu_baseline(args.cpu_seconds) if "cpu" in sections else None
    if "cpu" in sections and "gemm_m2048" in extra:
        extra["gemm_cpu_baseline"] = cpu_baseline_gemm(args.cpu_seconds)
        log(f"[cpu] oracle GEMM {extra['gemm_cpu_baseline']['value']:.2f} GFLOP/s on "
            f"{extra['gemm_cpu_baseline']['cores']} threads")
    extra["environment"] = environment()

    g = dec["fused2_act"]
    line = {
        "metric": "Q4 GEMV GB/s (M=1) and Q4 GEMM TFLOP/s (M=2048), N=12288 K=4096",
        "value": round(dec["gbs_step"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0 x q8_1 (int32 block dots, f32 accumulate)",
        "data": "synthetic (seeded numpy PCG64: W ~ N(0, 0.02^2), x ~ N(0, 1) as bf16)",
        "config": {
            "workload": "decode GEMV Q4_0 N=12288 K=4096 M=1: q4_gemv_act + q4_gemv_fused2_act (gate, up) "
                        "per step, each quantising the bf16 activation to Q8_1 on chip; weights rotated over "
                        "%d copies, steps replayed as a HIP graph" % args.copies,
            "M": 1, "N": 12288, "K": 4096,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "q4_gemv_fused2_act (k_q4_gemv<1,2,4,2,2,bf16>), the step's longest kernel",
            "achieved": round(g["gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(g["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes_per_launch": g["bytes"],
            "avg_launch_us": round(g["us"], 3),
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    if "gemm_m2048" in extra:
        gm = extra["gemm_m2048"]
        line["extra"]["gemm_roofline"] = {
            "bound": "mfma", "achieved": round(gm["fused_tflops"], 1), "peak": F16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(gm["fused_tflops"] / F16_MFMA_PEAK_TFLOPS, 4),
            "what": "q4_gemm per call: X image + weight image + matrix-core GEMM",
            "achieved_prepacked_weights": round(gm["image_tflops"], 1),
            "frac_prepacked_weights": round(gm["image_tflops"] / F16_MFMA_PEAK_TFLOPS, 4),
            "cpu_baseline": extra.get("gemm_cpu_baseline"),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
