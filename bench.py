"""Benchmark of the QLoRA NF4 linear layer on one MI355X.

Headline workload: the seven linears of one 65B-shaped transformer block on
one GPU (q, k, v, o 8192 x 8192; gate, up 8192 x 22016; down 22016 x 8192;
809.5M weights), M = 2048 tokens, LoRA r = 64, alpha = 16.  One step =
nf4_quantize of all seven fp32 weights, then qlora_linear_fwd and
qlora_linear_bwd of every linear, one after another on one stream, inputs
resident in HBM.  `value` is the forward+backward algorithmic TFLOP/s of the
whole step (the quantize time is inside the step, its bytes are not counted).

Also reported (not part of `value`): the roofline of the dominant kernel (the
gate/up forward GEMM, timed live with HIP events on the launch stream, alone
and together with every launch that feeds it), the 7B attention projection
step, the memory-bound paths in GB/s against 8 TB/s and against the device's
own read ceiling at the same size (quantize, bf16 dequantize, small-M
dequant-GEMV at M = 1/8/16 on the 65B MLP shape), the 7B MLP set, and the CPU
oracle timed on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-components] [--copy-probe]
       python bench.py --memory-only | --attn7b-only [--copy-probe]   (profiler runs)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP64_PEAK_TFLOPS = 78.6      # MI355X fp64 vector (FMA counted as two flops)
METRIC = "QLoRA linear fwd+bwd TFLOP/s and NF4 dequant-GEMV GB/s, % of roofline"
HEADLINE = "block65b_m2048"
KERNEL_SOURCES = {"fwd_gemm": "gemm_big.hip", "bwd_dx": "gemm_big.hip", "fwd_gemv": "gemv.hip",
                  "quant_pass1": "quantize.hip", "dequant": "quantize.hip"}


def layer_flops(M, K, N, r):
    fwd = 2 * M * K * N + 2 * M * K * r + 2 * M * r * N
    bwd = 2 * M * N * K + 4 * M * N * r + 4 * M * K * r
    return fwd, bwd


def kernel_flops(name, M, K, N, r):
    if name == "fwd_gemm":
        return 2 * M * K * N + 2 * M * r * N       # X·Ŵ plus the Z·(cB) extension
    if name == "bwd_dx":
        return 2 * M * N * K + 2 * M * r * K       # G·Ŵᵀ plus the dZ·Aᵀ extension
    raise KeyError(name)


def src_hash(fname):
    with open(os.path.join(ROOT, "bit_nf4_quantized_10_amd", "csrc", fname), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(kernel, workload="attn7b_4096"):
    """HBM bytes per launch from the committed PMC summary of this kernel at
    this workload, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m_hash = re.search(r"source_sha256_16:\s*(\w+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash(KERNEL_SOURCES[kernel]):
        return None
    return float(m_bytes.group(1))


def build_workload(torch, qn, si, dev, name, keep_host=False):
    """Device buffers of every linear of a multi-matrix workload (inputs,
    states, outputs) and one workspace big enough for any of its calls."""
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    mats, ws_bytes, qws_bytes, host = [], 256, 256, []
    for j in range(len(si.WORKLOADS[name]["shapes"])):
        d = si.layer_inputs(name, matrix=j)
        M, K, N, r = d["M"], d["K"], d["N"], d["r"]
        m = {"M": M, "K": K, "N": N, "r": r, "c": d["c"], "W": torch.from_numpy(d["W"]).to(dev).reshape(-1),
             "X": bf(d["X_bits"]), "A": bf(d["A_bits"]), "B": bf(d["B_bits"]), "G": bf(d["G_bits"]),
             "state": qn.empty_state(K * N, dev),
             "Y": torch.empty(M, N, dtype=torch.bfloat16, device=dev),
             "Z": torch.empty(M, r, dtype=torch.bfloat16, device=dev),
             "dX": torch.empty(M, K, dtype=torch.bfloat16, device=dev),
             "dA": torch.empty(K, r, dtype=torch.float32, device=dev),
             "dB": torch.empty(r, N, dtype=torch.float32, device=dev)}
        if keep_host:
            host.append(d)
        del d
        ws_bytes = max(ws_bytes, *qn.qlora_workspace_bytes(M, K, N, r))
        qws_bytes = max(qws_bytes, qn.nf4_sizes(K * N)["quant_workspace_bytes"])
        mats.append(m)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    qws = torch.empty(qws_bytes, dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    return mats, ws, qws, status, host


def run_linear(qn, m, ws, timed=()):
    """Forward then backward of one linear; the kernels named in `timed`
    are timed (library timers) during this linear only."""
    for k in timed:
        qn.qlora_timer_enable(k, True)
    qn.qlora_linear_fwd(m["X"], m["state"], m["A"], m["B"], m["c"], m["K"], m["N"], m["Y"], m["Z"], ws)
    for k in timed:
        qn.qlora_timer_enable(k, False)
    qn.qlora_linear_bwd(m["G"], m["X"], m["Z"], m["state"], m["A"], m["B"], m["c"], m["K"], m["N"], True,
                        m["dX"], m["dA"], m["dB"], ws)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a step takes about 7.5 ms: 30 warm-up steps bring the clocks to their steady
    # state, 200 timed steps take about 1.5 s
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--attn7b-only", action="store_true",
                    help="run only the 7B attention step (M = K = N = 4096) for --steps steps after --warmup steps "
                         "(for profiler runs); prints its figures instead of the benchmark line")
    ap.add_argument("--memory-only", action="store_true",
                    help="run only the memory-bound paths on the 65B MLP weight (for profiler runs); prints "
                         "their figures instead of the benchmark line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the layer is measured on exactly one GPU; multi-GPU runs are not supported "
              "(a sharded layer splits N across GPUs and all-reduces dX and dZ in the backward)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_nf4_quantized_10_amd as qn
    import synth_inputs as si

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.attn7b_only:
        attn = attn7b_step(torch, qn, si, dev, steps=args.steps, warmup=args.warmup)[0]
        if args.copy_probe:
            a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
            torch.empty_like(a).copy_(a)
            torch.cuda.synchronize()
        print(json.dumps({"attn7b_4096": attn}))
        return
    if args.memory_only:
        flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        res = bench_memory65b(torch, qn, si, dev, flush, status)
        if args.copy_probe:
            a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
            torch.empty_like(a).copy_(a)
            torch.cuda.synchronize()
        print(json.dumps({"memory_paths_decode65b": res}))
        return
    wl = HEADLINE
    mats, ws, qws, status, host = build_workload(torch, qn, si, dev, wl, keep_host=not args.no_cpu)
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    dominant_ids = (4, 5)   # gate and up: the forward GEMMs with the most flops per launch
    print(f"bench: {wl} inputs resident", file=sys.stderr, flush=True)

    def step(i, timed=()):
        for m in mats:
            qn.nf4_quantize(m["W"], m["state"], qws, status)
        for j, m in enumerate(mats):
            run_linear(qn, m, ws, timed if j in dominant_ids else ())

    # warmup, with every kernel timed to give the per-kernel averages
    for k in qn.KERNEL_IDS:
        qn.qlora_timer_enable(k, True)
    for i in range(max(args.warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    per_kernel = {}
    for k in qn.KERNEL_IDS:
        ms, n = qn.qlora_timer_read(k)
        qn.qlora_timer_enable(k, False)
        if n:
            per_kernel[k] = {"avg_ms": round(ms / n, 4), "launches_per_step": round(n / max(args.warmup, 1), 2)}
    if qn.nf4_status_read(status) != 0:
        raise RuntimeError("quantize reported a bad status")

    # timed region: the dominant GEMM (and the launches that feed it) timed
    # live on the launch stream during the gate and up forwards
    feeders = ("dequant_bf16", "lora_down", "reduce")
    timed = ("fwd_gemm",) + feeders
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i, timed)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    dom_ms, dom_n = qn.qlora_timer_read("fwd_gemm")
    feed = {k: qn.qlora_timer_read(k) for k in feeders}
    dom_avg = dom_ms / max(dom_n, 1)
    feed_ms = sum(v[0] for v in feed.values()) / max(dom_n, 1)

    M, K, N, r = (mats[4][k] for k in ("M", "K", "N", "r"))
    flops = sum(sum(layer_flops(m["M"], m["K"], m["N"], m["r"])) for m in mats)
    fwd_f = sum(layer_flops(m["M"], m["K"], m["N"], m["r"])[0] for m in mats)
    value = flops / (ms_step * 1e-3) / 1e12
    dflops = kernel_flops("fwd_gemm", M, K, N, r)
    achieved = dflops / (dom_avg * 1e-3) / 1e12
    with_feed = dflops / ((dom_avg + feed_ms) * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": read_traffic("fwd_gemm", "block65b_gate"),
                "kernel": f"fwd_gemm (gate/up forward, M={M} K={K} N={N} r={r})",
                "avg_ms": round(dom_avg, 4), "launches": dom_n, "flops_per_launch": dflops,
                "feeders": {k: {"ms_per_launch_of_gemm": round(v[0] / max(dom_n, 1), 4), "launches": v[1]}
                            for k, v in feed.items()},
                "achieved_with_feeders": round(with_feed, 2),
                "frac_with_feeders": round(with_feed / MFMA_BF16_PEAK_TFLOPS, 4)}
    print(f"bench: {args.steps} timed steps, {ms_step:.4f} ms each", file=sys.stderr, flush=True)

    # the two halves of the step, each timed on its own
    def part(fn, n=20):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    q_ms = part(lambda i: [qn.nf4_quantize(m["W"], m["state"], qws, status) for m in mats])
    l_ms = part(lambda i: [run_linear(qn, m, ws) for m in mats])

    # every dense GEMM launch of the step (7 forwards and 7 dX), timed with
    # the library timers over 5 layer passes: the GEMM kernel's rate over the
    # whole step, beside the single dominant launch of `roofline`
    gemm_flops = sum(kernel_flops(k, m["M"], m["K"], m["N"], m["r"]) for m in mats for k in ("fwd_gemm", "bwd_dx"))
    for k in ("fwd_gemm", "bwd_dx"):
        qn.qlora_timer_enable(k, True)
    part(lambda i: [run_linear(qn, m, ws) for m in mats], n=5)
    g_ms = sum(qn.qlora_timer_read(k)[0] for k in ("fwd_gemm", "bwd_dx")) / 5
    for k in ("fwd_gemm", "bwd_dx"):
        qn.qlora_timer_enable(k, False)
    qbytes = 0
    for m in mats:
        sz = qn.nf4_sizes(m["K"] * m["N"])
        qbytes += 4 * m["K"] * m["N"] + (m["K"] * m["N"] + 1) // 2 + sz["n1"] + 4 * sz["n2"] + 4
    components = {"kernel_avg_ms_warmup": per_kernel,
                  "headline_parts": {"quantize_ms": round(q_ms, 4), "quantize_bytes": qbytes,
                                     "quantize_GBps": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
                                     "quantize_frac_hbm": round(qbytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                     "layers_ms": round(l_ms, 4),
                                     "layers_TFLOPs": round(flops / (l_ms * 1e-3) / 1e12, 1),
                                     "layers_frac_bf16_peak": round(flops / (l_ms * 1e-3) / 1e12
                                                                    / MFMA_BF16_PEAK_TFLOPS, 4),
                                     "how": "20 back-to-back passes of each half alone"},
                  "dense_gemms_of_step": {"ms_per_step": round(g_ms, 4), "flops_per_step": gemm_flops,
                                          "TFLOPs": round(gemm_flops / (g_ms * 1e-3) / 1e12, 1),
                                          "frac_bf16_peak": round(gemm_flops / (g_ms * 1e-3) / 1e12
                                                                  / MFMA_BF16_PEAK_TFLOPS, 4),
                                          "how": "the 14 dense GEMM launches of a layers pass (every forward and "
                                                 "dX, M >= 192 path), each timed on its dispatch packet, 5 passes"}}
    cpu = None if args.no_cpu else cpu_baseline(host, flops)
    del host
    if not args.no_components:
        del mats, ws, qws
        torch.cuda.empty_cache()
        components.update(bench_components(torch, qn, si, dev, args))
    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        components["copy_probe_bytes"] = {"read": a.numel() * 4, "write": a.numel() * 4}

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl, "linears": {n: list(kn) for n, kn in zip(names, mats_shapes())},
                   "M": M, "r": r, "alpha": 16.0,
                   "step": "nf4_quantize of all 7 weights, then qlora_linear_fwd + qlora_linear_bwd of each linear",
                   "weights": sum(k * n for k, n in mats_shapes()),
                   "flops_fwd": fwd_f, "flops_bwd": flops - fwd_f, "wall_s": round(wall, 3)},
        "roofline": roofline, "cpu_baseline": cpu, "components": components,
    }
    print(json.dumps(line))


def mats_shapes():
    import synth_inputs as si
    return list(si.WORKLOADS[HEADLINE]["shapes"])


def attn7b_step(torch, qn, si, dev, steps, warmup):
    """The 7B attention-shaped projection (M = K = N = 4096, r = 64):
    nf4_quantize + fwd + bwd, three input sets rotated so the Infinity Cache
    cannot carry a step's inputs over; the forward GEMM timed live."""
    stream = torch.cuda.current_stream()
    bf = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    sets = []
    for i in range(3):
        d = si.layer_inputs("attn7b_4096", matrix=0)   # same values, distinct buffers
        sets.append({"W": torch.from_numpy(d["W"]).to(dev).reshape(-1), "X": bf(d["X_bits"]),
                     "A": bf(d["A_bits"]), "B": bf(d["B_bits"]), "G": bf(d["G_bits"])})
    M, K, N, r, c = d["M"], d["K"], d["N"], d["r"], d["c"]
    P = K * N
    sizes = qn.nf4_sizes(P)
    fwd_ws, bwd_ws = qn.qlora_workspace_bytes(M, K, N, r)
    qws = torch.empty(sizes["quant_workspace_bytes"], dtype=torch.uint8, device=dev)
    ws = torch.empty(max(fwd_ws, bwd_ws, 256), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    outs = [{"state": qn.empty_state(P, dev), "Y": torch.empty(M, N, dtype=torch.bfloat16, device=dev),
             "Z": torch.empty(M, r, dtype=torch.bfloat16, device=dev),
             "dX": torch.empty(M, K, dtype=torch.bfloat16, device=dev),
             "dA": torch.empty(K, r, dtype=torch.float32, device=dev),
             "dB": torch.empty(r, N, dtype=torch.float32, device=dev)} for _ in sets]

    def step(i):
        s, o = sets[i % 3], outs[i % 3]
        qn.nf4_quantize(s["W"], o["state"], qws, status)
        qn.qlora_linear_fwd(s["X"], o["state"], s["A"], s["B"], c, K, N, o["Y"], o["Z"], ws)
        qn.qlora_linear_bwd(s["G"], s["X"], o["Z"], o["state"], s["A"], s["B"], c, K, N, True,
                            o["dX"], o["dA"], o["dB"], ws)

    for i in range(warmup):
        step(i)
    qn.qlora_timer_enable("fwd_gemm", True)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    gms, gn = qn.qlora_timer_read("fwd_gemm")
    qn.qlora_timer_enable("fwd_gemm", False)
    ms_step = ev0.elapsed_time(ev1) / steps
    fwd_f, bwd_f = layer_flops(M, K, N, r)
    gflops = kernel_flops("fwd_gemm", M, K, N, r)
    out = {"ms_per_step": round(ms_step, 4), "TFLOPs": round((fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12, 1),
           "steps": steps, "warmup": warmup,
           "fwd_gemm_ms": round(gms / max(gn, 1), 4),
           "fwd_gemm_frac_bf16_peak": round(gflops / (gms / max(gn, 1) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "fwd_gemm_traffic": read_traffic("fwd_gemm"),
           "how": "nf4_quantize + qlora_linear_fwd + qlora_linear_bwd, M = K = N = 4096, r = 64, three input "
                  "sets rotated"}
    return out, sets, outs, qws, status


def _flush_cache(flush):
    """Leave the 256 MB Infinity Cache cold and clean: overwrite it with a
    512 MB buffer, then read that buffer back, so that the timed call finds
    none of its inputs cached and has no dirty lines of the flush itself to
    write back (a write-only flush charges the next call with up to 256 MB
    of write-backs)."""
    flush.add_(1)
    flush.sum()


def _time_kernel(qn, torch, name, fn, reps, flush=None):
    """Average duration of kernel `name` over `reps` calls of fn, timed by the
    library's HIP events on the launch stream; with `flush`, the cache is
    flushed before every call (outside the timed kernel)."""
    qn.qlora_timer_enable(name, True)
    for i in range(reps):
        if flush is not None:
            _flush_cache(flush)
        fn(i)
    torch.cuda.synchronize()
    ms, n = qn.qlora_timer_read(name)
    qn.qlora_timer_enable(name, False)
    return ms / max(n, 1)


def _time_calls(torch, fn, reps, flush):
    """Average wall time of one call, each call bracketed by its own events
    after a cache flush."""
    total = 0.0
    for i in range(reps):
        _flush_cache(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(i)
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
    return total / reps


def read_ceiling(torch, dev, nbytes, flush, reps=7):
    """The device's own read ceiling at a given size: the plain streaming read
    of libqlora_probe.so over a buffer of that size, from a clean cache;
    best of several workgroup counts, median over reps."""
    from bit_nf4_quantized_10_amd import probe
    buf = torch.ones(nbytes // 16 * 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = None
    for grid in (2048, 4096, 8192):
        t = sorted(_time_calls(torch, lambda i: probe.read_probe(buf, sink, grid), 1, flush) for _ in range(reps))
        ms = t[len(t) // 2]
        if best is None or ms < best[0]:
            best = (ms, grid)
    del buf
    return {"bytes": nbytes // 16 * 16, "ms": round(best[0], 4),
            "GBps": round(nbytes / (best[0] * 1e-3) / 1e9, 1), "grid": best[1]}


def bench_memory65b(torch, qn, si, dev, flush, status):
    """The memory-bound paths on the 65B MLP weight (8192 x 22016): the whole
    nf4_quantize call, the bf16 dequantize, and the small-M dequant-GEMV
    forward at M = 1, 8, 16 (whole call and GEMV kernel), each call after a
    cache flush; plus the device's read ceiling at the GEMV's size."""
    res = {}
    # small-M dequant-GEMV on the 65B MLP shape
    d = si.layer_inputs("decode65b_8192x22016", M=16, with_grad=False)
    K, N, r, c = d["K"], d["N"], d["r"], d["c"]
    Pg = K * N
    states = []
    Wg = torch.from_numpy(d["W"]).to(dev).reshape(-1)
    for i in range(2):
        st, _ = qn.nf4_quantize(Wg)
        states.append(st)
    # quantize and bf16 dequantize at this size too (721 MB of fp32 in, 360 MB of bf16 out)
    sg = qn.nf4_sizes(Pg)
    qws_g = torch.empty(sg["quant_workspace_bytes"], dtype=torch.uint8, device=dev)
    st_g = qn.empty_state(Pg, dev)
    qfn_g = lambda i: qn.nf4_quantize(Wg, st_g, qws_g, status)
    qfn_g(0)
    qms_g = _time_calls(torch, qfn_g, 5, flush)
    qbytes_g = 4 * Pg + (Pg + 1) // 2 + sg["n1"] + 4 * sg["n2"] + 4
    res["quantize_decode65b"] = {"bytes": qbytes_g, "call_ms": round(qms_g, 4),
                                 "GBps_call": round(qbytes_g / (qms_g * 1e-3) / 1e9, 1),
                                 "frac_hbm_call": round(qbytes_g / (qms_g * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del Wg, qws_g, st_g
    out_g = torch.empty(Pg, dtype=torch.bfloat16, device=dev)
    dms_g = _time_kernel(qn, torch, "dequant",
                         lambda i: qn.nf4_dequantize(states[i % 2], "bf16", out=out_g), 8, flush)
    dbytes_g = (Pg + 1) // 2 + sg["n1"] + 4 * sg["n2"] + 4 + 2 * Pg
    res["dequant_bf16_decode65b"] = {"bytes": dbytes_g, "ms": round(dms_g, 4),
                                     "GBps": round(dbytes_g / (dms_g * 1e-3) / 1e9, 1),
                                     "frac_hbm": round(dbytes_g / (dms_g * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del out_g
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    A, B = bf(d["A_bits"]), bf(d["B_bits"])
    gemv = {}
    for M in (1, 8, 16):
        X = bf(d["X_bits"][:M])
        Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        Z = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(qn.qlora_workspace_bytes(M, K, N, r)[0], 256), dtype=torch.uint8, device=dev)
        gbytes = Pg // 2 + sg["n1"] + 4 * sg["n2"] + 4 + 2 * M * K + 2 * K * r + 2 * r * N + 2 * M * N + 2 * M * r
        fn = lambda i: qn.qlora_linear_fwd(X, states[i % 2], A, B, c, K, N, Y, Z, ws)
        for i in range(2):
            fn(i)
        call_ms = _time_calls(torch, fn, 12, flush)
        kms = _time_kernel(qn, torch, "fwd_gemv", fn, 12, flush)
        gemv[f"M{M}"] = {"bytes": gbytes, "call_ms": round(call_ms, 4), "gemv_kernel_ms": round(kms, 4),
                         "GBps_call": round(gbytes / (call_ms * 1e-3) / 1e9, 1),
                         "frac_hbm_call": round(gbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "GBps_kernel": round(gbytes / (kms * 1e-3) / 1e9, 1)}
    # the device's own read ceiling at the GEMV's size: the call is judged
    # against it as well as against the 8 TB/s specification (both are timed
    # as whole calls, launch included)
    ceil = read_ceiling(torch, dev, gemv["M16"]["bytes"], flush)
    for v in gemv.values():
        v["frac_read_ceiling_call"] = round(v["GBps_call"] / ceil["GBps"], 4)
    res["gemv_decode65b"] = gemv
    res["read_ceiling_gemv_size"] = ceil
    return res


def bench_components(torch, qn, si, dev, args):
    """The 7B attention step, then the memory-bound paths (each call preceded
    by a cache flush: a 512 MB buffer written, then read, so that no input or
    output is served from the Infinity Cache), then other workloads."""
    res = {}
    attn, sets, outs, qws, status = attn7b_step(torch, qn, si, dev, steps=1000, warmup=200)
    res["attn7b_4096"] = attn
    print("bench: attn7b_4096 measured", file=sys.stderr, flush=True)
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)
    P = sets[0]["W"].numel()
    n1, n2 = qn.nf4_sizes(P)["n1"], qn.nf4_sizes(P)["n2"]
    # quantize: fp32 read, codes + int8 codes + fp32 scales written
    qbytes = 4 * P + (P + 1) // 2 + n1 + 4 * n2 + 4
    qfn = lambda i: qn.nf4_quantize(sets[i % 3]["W"], outs[i % 3]["state"], qws, status)
    ms = _time_kernel(qn, torch, "quant_pass1", qfn, 10, flush)
    full_ms = _time_calls(torch, qfn, 10, flush)
    res["quantize_attn7b"] = {"bytes": qbytes, "pass1_ms": round(ms, 4), "call_ms": round(full_ms, 4),
                              "GBps_call": round(qbytes / (full_ms * 1e-3) / 1e9, 1),
                              "frac_hbm_call": round(qbytes / (full_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # bf16 dequantize
    dbytes = (P + 1) // 2 + n1 + 4 * n2 + 4 + 2 * P
    outs_bf = [torch.empty(P, dtype=torch.bfloat16, device=dev) for _ in range(3)]
    ms = _time_kernel(qn, torch, "dequant",
                      lambda i: qn.nf4_dequantize(outs[i % 3]["state"], "bf16", out=outs_bf[i % 3]), 16, flush)
    res["dequant_bf16_attn7b"] = {"bytes": dbytes, "ms": round(ms, 4),
                                  "GBps": round(dbytes / (ms * 1e-3) / 1e9, 1),
                                  "frac_hbm": round(dbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del outs_bf
    res.update(bench_memory65b(torch, qn, si, dev, flush, status))
    ceil = res["read_ceiling_gemv_size"]
    print("bench: memory-bound paths measured", file=sys.stderr, flush=True)
    out = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    wr = min(_time_calls(torch, lambda i: out.fill_(1.0), 3, flush) for _ in range(2))
    res["device_streaming_ceiling"] = {
        "read_at_gemv_size": ceil,
        "read_1GiB": read_ceiling(torch, dev, 1 << 30, flush, reps=3),
        "write_1GiB_GBps": round(out.numel() * 4 / (wr * 1e-3) / 1e9, 1),
        "how": "reads: the plain streaming read of libqlora_probe.so (16-byte loads, four in flight per lane), "
               "best of 2048/4096/8192 workgroups, median of 7 (3 at 1 GiB); write: torch fill of 1 GiB; "
               "cache flushed before each call"}
    del out
    # adapter merge for re-export at the bench workload's shape: fp64 FMA bound
    # (2 K N r flops), plus the re-quantize of the merged weight
    dm = si.layer_inputs("attn7b_4096", with_weight=False, with_grad=False)
    Km, Nm, rm, cm = dm["K"], dm["N"], dm["r"], dm["c"]
    stm = outs[0]["state"]
    Amd = torch.from_numpy(np.ascontiguousarray(dm["A_bits"]).view(np.int16)).view(torch.bfloat16).to(dev)
    Bmd = torch.from_numpy(np.ascontiguousarray(dm["B_bits"]).view(np.int16)).view(torch.bfloat16).to(dev)
    wm = qn.qlora_merge(stm, Amd, Bmd, cm, Km, Nm)
    mms = _time_kernel(qn, torch, "merge", lambda i: qn.qlora_merge(stm, Amd, Bmd, cm, Km, Nm, out=wm), 10, flush)
    mfl = 2 * Km * Nm * rm
    res["merge_attn7b"] = {"ms": round(mms, 4), "fp64_TFLOPs": round(mfl / (mms * 1e-3) / 1e12, 2),
                           "frac_fp64_peak": round(mfl / (mms * 1e-3) / 1e12 / FP64_PEAK_TFLOPS, 4),
                           "flops": mfl}
    del wm, Amd, Bmd
    # grouped q, k, v of the 7B block (3 x 4096 columns sharing X, r = 64 each)
    # against three separate linears, fwd + bwd each way
    Kg, Ng, rg, cg, Mg = 4096, 4096, 64, 0.25, 4096
    gst = [outs[i]["state"] for i in range(3)]
    Xg = sets[0]["X"]
    Ag = torch.cat([sets[i]["A"] for i in range(3)], dim=1).contiguous()
    Bg = torch.cat([sets[i]["B"] for i in range(3)], dim=1).contiguous()
    Gg = torch.cat([sets[i]["G"] for i in range(3)], dim=1).contiguous()
    Ns = [Ng] * 3
    fgw, bgw = qn.qlora_grouped_workspace_bytes(Mg, Kg, Ns, rg)
    gws = torch.empty(max(fgw, bgw), dtype=torch.uint8, device=dev)
    Yg = torch.empty(Mg, 3 * Ng, dtype=torch.bfloat16, device=dev)
    Zg = torch.empty(Mg, 3 * rg, dtype=torch.bfloat16, device=dev)
    dXg = torch.empty(Mg, Kg, dtype=torch.bfloat16, device=dev)
    dAg = torch.empty(Kg, 3 * rg, dtype=torch.float32, device=dev)
    dBg = torch.empty(rg, 3 * Ng, dtype=torch.float32, device=dev)

    def grouped(i):
        qn.qlora_grouped_fwd(Xg, gst, Ag, Bg, cg, Kg, Ns, Yg, Zg, gws)
        qn.qlora_grouped_bwd(Gg, Xg, Zg, gst, Ag, Bg, cg, Kg, Ns, True, dXg, dAg, dBg, gws)

    fsw, bsw = qn.qlora_workspace_bytes(Mg, Kg, Ng, rg)
    sws = torch.empty(max(fsw, bsw), dtype=torch.uint8, device=dev)

    def separate(i):
        for j in range(3):
            o = outs[j]
            qn.qlora_linear_fwd(Xg, gst[j], sets[j]["A"], sets[j]["B"], cg, Kg, Ng, o["Y"], o["Z"], sws)
            qn.qlora_linear_bwd(sets[j]["G"], Xg, o["Z"], gst[j], sets[j]["A"], sets[j]["B"], cg, Kg, Ng, True,
                                o["dX"], o["dA"], o["dB"], sws)

    for fn in (grouped, separate):
        fn(0)
    gms = _time_calls(torch, grouped, 5, flush)
    sms = _time_calls(torch, separate, 5, flush)
    gfl = 3 * sum(layer_flops(Mg, Kg, Ng, rg))
    res["grouped_qkv_attn7b"] = {"grouped_ms": round(gms, 4), "separate_ms": round(sms, 4),
                                 "grouped_TFLOPs": round(gfl / (gms * 1e-3) / 1e12, 1),
                                 "separate_TFLOPs": round(gfl / (sms * 1e-3) / 1e12, 1),
                                 "how": "fwd + bwd of q, k, v (3 x 4096 x 4096, r = 64, M = 4096): one grouped "
                                        "call each way vs three single-linear calls each way, cache flushed"}
    del gws, sws, Yg, Zg, dXg, dAg, dBg, Ag, Bg, Gg
    # mid-size batches: M = 64 and 128 decode the weight inside the GEMM, 256
    # and 384 dequantize it first; both GEMMs split their reduction across
    # workgroups when the output has too few tiles for the device
    # (fwd_gemm_ms is the GEMM launch alone, without the fixed-order sum of
    # its partials)
    mid = {}
    for Mm in (64, 128, 256, 384):
        Xm, Gm = sets[0]["X"][:Mm].contiguous(), sets[0]["G"][:Mm].contiguous()
        fwm, bwm = qn.qlora_workspace_bytes(Mm, Kg, Ng, rg)
        wsm = torch.empty(max(fwm, bwm), dtype=torch.uint8, device=dev)
        Ym = torch.empty(Mm, Ng, dtype=torch.bfloat16, device=dev)
        Zm = torch.empty(Mm, rg, dtype=torch.bfloat16, device=dev)
        dXm = torch.empty(Mm, Kg, dtype=torch.bfloat16, device=dev)
        dAm = torch.empty(Kg, rg, dtype=torch.float32, device=dev)
        dBm = torch.empty(rg, Ng, dtype=torch.float32, device=dev)

        def stepm(i):
            qn.qlora_linear_fwd(Xm, gst[i % 3], sets[0]["A"], sets[0]["B"], cg, Kg, Ng, Ym, Zm, wsm)
            qn.qlora_linear_bwd(Gm, Xm, Zm, gst[i % 3], sets[0]["A"], sets[0]["B"], cg, Kg, Ng, True, dXm, dAm,
                                dBm, wsm)

        stepm(0)
        mms = _time_calls(torch, stepm, 6, flush)
        fwk = _time_kernel(qn, torch, "fwd_gemm", stepm, 6, flush)
        mfl = sum(layer_flops(Mm, Kg, Ng, rg))
        wbytes = (Kg * Ng) // 2 + (Kg * Ng) // 64   # packed codes + second-level codes, read by each GEMM
        mid[f"M{Mm}"] = {"ms": round(mms, 4), "TFLOPs": round(mfl / (mms * 1e-3) / 1e12, 1),
                         "fwd_gemm_ms": round(fwk, 4),
                         "fwd_gemm_TFLOPs": round((2 * Mm * Kg * Ng + 2 * Mm * rg * Ng) / (fwk * 1e-3) / 1e12, 1),
                         "fwd_gemm_weight_GBps": round(wbytes / (fwk * 1e-3) / 1e9, 1)}
        del wsm, Ym, Zm, dXm, dAm, dBm
    res["mid_m_attn7b"] = mid
    # the same layer step in the fp16 compute type (fp16 MFMA, fp16 Ŵ)
    Xh, Ah, Bh, Gh = (sets[0][k].to(torch.float16) for k in ("X", "A", "B", "G"))
    fws16, bws16 = qn.qlora_workspace_bytes(Mg, Kg, Ng, rg)
    ws16 = torch.empty(max(fws16, bws16), dtype=torch.uint8, device=dev)
    Yh = torch.empty(Mg, Ng, dtype=torch.float16, device=dev)
    Zh = torch.empty(Mg, rg, dtype=torch.float16, device=dev)
    dXh = torch.empty(Mg, Kg, dtype=torch.float16, device=dev)
    dAh = torch.empty(Kg, rg, dtype=torch.float32, device=dev)
    dBh = torch.empty(rg, Ng, dtype=torch.float32, device=dev)

    def step16(i):
        qn.qlora_linear_fwd(Xh, gst[0], Ah, Bh, cg, Kg, Ng, Yh, Zh, ws16)
        qn.qlora_linear_bwd(Gh, Xh, Zh, gst[0], Ah, Bh, cg, Kg, Ng, True, dXh, dAh, dBh, ws16)

    step16(0)
    hms = _time_calls(torch, step16, 5, flush)
    hfl = sum(layer_flops(Mg, Kg, Ng, rg))
    res["fp16_layer_attn7b"] = {"ms": round(hms, 4), "TFLOPs": round(hfl / (hms * 1e-3) / 1e12, 1),
                                "how": "qlora_linear_fwd + _bwd in the fp16 compute type, 4096 x 4096, r = 64, "
                                       "M = 4096, cache flushed"}
    del Xh, Ah, Bh, Gh, ws16, Yh, Zh, dXh, dAh, dBh
    # every linear of the 7B MLP set, one pass each
    del sets, outs
    torch.cuda.empty_cache()
    res["mlp7b_4096x11008"] = bench_workload_set(torch, qn, si, dev, "mlp7b_4096x11008", flush)
    print("bench: mlp7b_4096x11008 measured", file=sys.stderr, flush=True)
    # the vendor library's plain bf16 GEMM on this device (torch.matmul ->
    # hipBLASLt), as context for the MFMA fraction: the 4096^3 base shape and
    # the four distinct GEMM shapes of the 65B block, the weight operand stored
    # N x K as the forward's dequantized weight is (both operands contiguous
    # along the reduction)
    vendor = {}
    for (Mv, Kv, Nv) in ((4096, 4096, 4096), (2048, 8192, 8192), (2048, 8192, 22016), (2048, 22016, 8192)):
        xa = torch.randn(Mv, Kv, device=dev).to(torch.bfloat16)
        wb = torch.randn(Nv, Kv, device=dev).to(torch.bfloat16)
        yv = torch.empty(Mv, Nv, dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            torch.matmul(xa, wb.t(), out=yv)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            torch.matmul(xa, wb.t(), out=yv)
        e1.record()
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / 20
        vendor[f"{Mv}x{Kv}x{Nv}"] = {"ms": round(vms, 4),
                                     "TFLOPs": round(2 * Mv * Kv * Nv / (vms * 1e-3) / 1e12, 1)}
        del xa, wb, yv
    vendor["how"] = ("torch.matmul of M x K by (N x K)ᵀ bf16 (hipBLASLt), random normal operands, "
                     "20 back-to-back calls per shape, keyed MxKxN")
    res["vendor_gemm_bf16"] = vendor
    return res


def bench_workload_set(torch, qn, si, dev, name, flush, reps=3):
    """All linears of a multi-matrix workload, each with its own weight and
    inputs: nf4_quantize of every weight, then qlora_linear_fwd and _bwd of
    every linear, one after another on one stream (inputs resident in HBM,
    the Infinity Cache overwritten before each timed pass).  The layers'
    TFLOP/s count the fwd+bwd flops only; the quantize is timed on its own
    as well, against its algorithmic bytes."""
    mats, ws, qws, status, _ = build_workload(torch, qn, si, dev, name)

    def quant_all(i):
        for m in mats:
            qn.nf4_quantize(m["W"], m["state"], qws, status)

    def layers_all(i):
        for m in mats:
            qn.qlora_linear_fwd(m["X"], m["state"], m["A"], m["B"], m["c"], m["K"], m["N"], m["Y"], m["Z"], ws)
            qn.qlora_linear_bwd(m["G"], m["X"], m["Z"], m["state"], m["A"], m["B"], m["c"], m["K"], m["N"], True,
                                m["dX"], m["dA"], m["dB"], ws)

    def step(i):
        quant_all(i)
        layers_all(i)

    step(0)
    if qn.nf4_status_read(status) != 0:
        raise RuntimeError(f"quantize reported a bad status on {name}")
    sms = _time_calls(torch, step, reps, flush)
    qms = _time_calls(torch, quant_all, reps, flush)
    lms = _time_calls(torch, layers_all, reps, flush)
    flops = sum(sum(layer_flops(m["M"], m["K"], m["N"], m["r"])) for m in mats)
    qbytes = 0
    for m in mats:
        P = m["K"] * m["N"]
        sz = qn.nf4_sizes(P)
        qbytes += 4 * P + (P + 1) // 2 + sz["n1"] + 4 * sz["n2"] + 4
    out = {"matrices_KxN": [[m["K"], m["N"]] for m in mats], "M": mats[0]["M"], "r": mats[0]["r"],
           "step_ms": round(sms, 4), "step_TFLOPs": round(flops / (sms * 1e-3) / 1e12, 1),
           "layers_ms": round(lms, 4), "layers_TFLOPs": round(flops / (lms * 1e-3) / 1e12, 1),
           "layers_frac_bf16_peak": round(flops / (lms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "quantize_ms": round(qms, 4), "quantize_bytes": qbytes,
           "quantize_GBps": round(qbytes / (qms * 1e-3) / 1e9, 1),
           "quantize_frac_hbm": round(qbytes / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "flops_fwd_bwd": flops,
           "how": "nf4_quantize of every weight, then fwd + bwd of every linear, one stream, cache flushed; "
                  f"mean of {reps} passes"}
    del mats, ws, qws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(host, flops_total, rows=128, reps=3):
    """The oracle as it stands, on the host cores, on a bounded sample of the
    headline step, scaled to the whole step:
      - nf4_quantize's oracle on the q weight (8192 x 8192, 67.1M of the
        block's 809.5M weights), time scaled by the weight count;
      - the oracle's forward and backward of all seven linears on the first
        `rows` of the 2048 token rows, time scaled by 2048 / rows.  The
        layer products run on the bf16-rounded fp32 weights, which have the
        shape and dtype of Ŵ (the values do not change the oracle's time).
    Median of `reps` runs of each part."""
    from oracle import nf4_oracle as o
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    weights = sum(d["K"] * d["N"] for d in host)
    d0 = host[0]
    tq = []
    for _ in range(reps):
        t0 = time.perf_counter()
        o.quantize(d0["W"].ravel())
        tq.append(time.perf_counter() - t0)
    w_hat = [o.bf16_round(d["W"]) for d in host]
    tl = []
    for _ in range(reps):
        t0 = time.perf_counter()
        for d, wh in zip(host, w_hat):
            o.layer_forward(d["X"][:rows], wh, d["A"], d["B"], d["c"])
            o.layer_backward(d["G"][:rows], d["X"][:rows], wh, d["A"], d["B"], d["c"])
        tl.append(time.perf_counter() - t0)
    q_s = sorted(tq)[reps // 2] * weights / d0["W"].size
    l_s = sorted(tl)[reps // 2] * host[0]["M"] / rows
    step_s = q_s + l_s
    return {"value": round(flops_total / step_s / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "host_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"oracle quantize of the 8192x8192 q weight ({d0['W'].size / 1e6:.1f}M of {weights / 1e6:.1f}M "
                      f"weights, {sorted(tq)[reps // 2]:.2f} s) and fwd+bwd of all 7 linears on {rows} of "
                      f"{host[0]['M']} token rows ({sorted(tl)[reps // 2]:.2f} s), each the median of {reps} runs "
                      f"({sum(tq) + sum(tl):.1f} s of CPU work), scaled to the whole step: {step_s:.1f} s per step; "
                      f"cores = BLAS threads used, host_cores = CPUs the process may run on"}


if __name__ == "__main__":
    main()
