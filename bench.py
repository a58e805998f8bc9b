#!/usr/bin/env python3
"""Throughput of the SVDQuant W4A4 + low-rank linear on one MI355X.

One step = one full forward of the layer over one batch of tokens: the fused
smooth + quantize + lora_down kernel (k1), then the W4A4 GEMM with its scale
epilogue, lora_up and bias (k2).  Inputs, packed weights and outputs rotate
over more than 512 MB of buffers so that the 256 MB Infinity Cache cannot
serve a step from the previous one.

Prints one JSON line (rank 0).  Default workload: the DiT attention
projection, M=4096 tokens, K=N=3072, rank 32.  Other workloads (--workload)
are the small-K UNet widths and the DiT MLP linears.

Timing.  First the clocks settle: untimed steps for --settle-ms of wall time
(the host-side pack leaves the GPU idle, and a few warm-up steps are not
enough for the engine clock to ramp).  Then W eager warm-up steps, then K
eager steps with HIP events around every launch (per-kernel durations as the
stream sees them, dispatch gaps included).  Then, unless --no-graph, the same
K steps are captured into one HIP graph, replayed untimed for 150 ms (the
capture idles the GPU and the clock drops), and replayed once timed: `value`
and `ms_per_step` come from that replay (the launch path a serving loop would
use).  Per-kernel durations for the roofline come from graphs of K
back-to-back launches of that kernel alone over the same rotating buffers.
--workload dit_block times the four SVDQuant linears of a DiT block at width
3072 and 4608 tokens (fused QKV 3072 -> 9216, attention output 3072 -> 3072,
MLP up 3072 -> 12288 with GELU fused into its epilogue, MLP down
12288 -> 3072 reading the up projection's output), each branch widened by a
seeded rank-16 LoRA to r = 48; the attention itself is not part of it.
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

PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, TOP/s
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # HBM3E
PEAK_FP4_TFLOPS = 10100.0   # dense FP4 (and FP6) MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dit_proj")
    ap.add_argument("--rotate-mb", type=int, default=640, help="total bytes of rotated buffers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work of the oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--format", choices=["int4", "mxfp4"], default="int4",
                    help="int4: symmetric int4, one fp32 scale per 64 channels (int8 MFMA); "
                         "mxfp4: E2M1 with an E8M0 scale per 32 (block-scaled FP4 MFMA)")
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed steps for this much wall time before the warm-up, so that the "
                         "engine clock has ramped when timing starts")
    ap.add_argument("--tokens", type=int, default=0,
                    help="token rows M (default: the workload's own)")
    ap.add_argument("--path", choices=["auto", "two-kernel"], default="auto",
                    help="auto: the forward's own plan (one fused kernel for narrow layers); "
                         "two-kernel: the quantize kernel then the GEMM, always")
    ap.add_argument("--no-graph", action="store_true",
                    help="report the eager launch loop instead of the HIP graph replay")
    return ap.parse_args()


def kernel_source_hash(name: str, root: str = ROOT) -> str:
    """sha256 over a kernel source and every local header it includes (transitively)."""
    dirs = [os.path.join(root, "bit_diffusion_model_svdq_amd", "csrc"), os.path.join(root, "include")]
    h = hashlib.sha256()
    seen, todo = set(), [name]
    while todo:
        f = todo.pop(0)
        if f in seen:
            continue
        seen.add(f)
        path = next((os.path.join(d, f) for d in dirs if os.path.exists(os.path.join(d, f))), None)
        if path is None:
            raise FileNotFoundError(f)
        text = open(path, "rb").read()
        h.update(f.encode() + b"\0" + text)
        todo += re.findall(r'^\s*#\s*include\s+"([^"]+)"', text.decode(), flags=re.M)
    return h.hexdigest()[:16]


def load_traffic(kernel_file: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if taken on the current source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(workload, {}).get(kernel_file)
        if e and e.get("source_sha256_16") == kernel_source_hash(kernel_file):
            return e["bytes_per_launch"]
    except Exception:
        return None
    return None


def read_sclk_mhz():
    """The engine clock's current DPM level (MHz) from sysfs, or None where it is not readable."""
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(f):
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                    if m:
                        return int(m.group(1))
        except OSError:
            continue
    return None


def settle(torch, launch, ms):
    """Untimed launch(i) in chunks of 10 until `ms` of wall time has passed; returns
    (launches, wall ms)."""
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            launch(n)
            n += 1
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def host_cpu():
    """nproc (the CPUs this process may run on) and the CPU model, for the baseline's record."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"nproc": nproc, "cpu_model": model}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return 1


def copy_probe():
    import torch
    n = 256 << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe:
        copy_probe()
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import bit_diffusion_model_svdq_amd as S
    import synth

    if args.workload == "dit_block":
        return bench_block(args, S, synth, torch)
    w = synth.WORKLOADS[args.workload]
    M, K, N, r = (args.tokens or w.M), w.K, w.N, w.rank
    dev = torch.device("cuda:0")

    # ---- offline pack (host, untimed) through the library's packer
    t0 = time.time()
    X = synth.activations(w, M)
    W = synth.weight(w)
    b = synth.bias(w)
    A = np.zeros(K, np.float32)
    S.svdq_act_absmax_update(synth.calibration_activations(w), A)
    pk = S.svdq_pack_weights(W, A, w.alpha, r)
    mx = args.format == "mxfp4"
    if mx:   # same s, L1, L2; the residual quantized to MXFP4
        pk["Wq"], pk["w_scales"] = S.svdq_quantize_residual_mxfp4(W, pk["smooth"], pk["L1"], pk["L2"])
    pack_s = time.time() - t0
    print(f"# packed {args.workload} in {pack_s:.1f}s", file=sys.stderr, flush=True)

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    ws_bytes = (S.svdq_forward_workspace_bytes_mxfp4 if mx else S.svdq_forward_workspace_bytes)(M, K, N, r)
    per_set = (M * K * 2 + M * N * 2 + ws_bytes + N * K // 2 + pk["w_scales"].nbytes
               + r * (K + N) * 2 + K * 4 + N * 2)
    nsets = max(2, -(-args.rotate_mb * (1 << 20) // per_set))
    sets = []
    # the forward reads MXFP4 weight scales k-tiled; the oracle leg keeps them row-major
    base = dict(X=t(X), s=t(pk["smooth"]), L1=t(pk["L1"]), L2=t(pk["L2"]), Wq=t(pk["Wq"]),
                ws=t(S.svdq_mxfp4_tile_scales(pk["w_scales"]) if mx else pk["w_scales"]), b=t(b))
    for i in range(nsets):
        d = {k: v.clone() for k, v in base.items()}
        d["Y"] = torch.empty((M, N), dtype=torch.int16, device=dev)
        d["work"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        sets.append(d)
    torch.cuda.synchronize()

    quantize = S.svdq_forward_quantize_mxfp4 if mx else S.svdq_forward_quantize
    gemm = S.svdq_forward_gemm_mxfp4 if mx else S.svdq_forward_gemm

    # narrow layers run as one fused kernel: the step is then the forward call itself
    fused = args.path == "auto" and (S.svdq_forward_fused_mxfp4 if mx else S.svdq_forward_fused)(M, K, N, r)
    forward = S.svdq_linear_forward_mxfp4 if mx else S.svdq_linear_forward

    def step(d):
        if fused:
            forward(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], d["Y"], d["work"])
        else:
            quantize(d["X"], d["s"], d["L1"], d["work"])
            gemm(M, K, d["L2"], d["Wq"], d["ws"], d["b"], d["Y"], d["work"], r)

    settle_n, settle_ms = settle(torch, lambda i: step(sets[i % nsets]), args.settle_ms)
    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # ---- timed region: K steps, HIP events on the launch stream around each kernel
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        d = sets[i % nsets]
        e = ev[i]
        e[0].record()
        if fused:
            step(d)
            e[1].record()
            e[2].record()
        else:
            quantize(d["X"], d["s"], d["L1"], d["work"])
            e[1].record()
            gemm(M, K, d["L2"], d["Wq"], d["ws"], d["b"], d["Y"], d["work"], r)
            e[2].record()
    end.record()
    sclk_eager = read_sclk_mhz()   # sampled while the queued steps run
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    k1_ms = eager_k1_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    k2_ms = eager_k2_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_step = total_ms / args.steps
    eager_ms_step = ms_step

    graph_info = None
    if not args.no_graph:
        def k1_only(i):
            d = sets[i % nsets]
            quantize(d["X"], d["s"], d["L1"], d["work"])

        def k2_only(i):
            d = sets[i % nsets]
            gemm(M, K, d["L2"], d["Wq"], d["ws"], d["b"], d["Y"], d["work"], r)

        graph_clock = []
        ms_step = time_graph(torch, lambda i: step(sets[i % nsets]), args.steps, graph_clock)
        if fused:
            k1_ms = ms_step
        else:
            k1_ms = time_graph(torch, k1_only, args.steps)
            k2_ms = time_graph(torch, k2_only, args.steps)
        graph_info = {"steps_per_graph": args.steps, "ms_per_step": round(ms_step, 5),
                      "eager_ms_per_step": round(eager_ms_step, 5),
                      "eager_k1_us": round(eager_k1_ms * 1e3, 3), "eager_k2_us": round(eager_k2_ms * 1e3, 3),
                      "sclk_mhz": graph_clock[0]}

    if fused:   # the two-kernel figures below are placeholders, replaced by the fused kernel's
        k2_ms = k1_ms
    ops_main = 2.0 * M * N * K                 # the 4-bit product (int8 or FP4 MFMA)
    ops_low = 2.0 * M * r * (K + N)            # bf16 low-rank branch
    tops = (ops_main + ops_low) / (ms_step * 1e-3) / 1e12
    tokens_s = M / (ms_step * 1e-3)
    # scale bytes per row: one fp32 per 64 channels (int4) or one E8M0 byte per 32 (mxfp4)
    sb_row = K // 32 if mx else 4 * (K // 64)
    k1_bytes = M * (2 * K + K // 2 + sb_row + 4 * r) + r * K * 2 + K * 4
    k2_bytes = (M * (K // 2 + sb_row + 4 * r + 2 * N)
                + N * K // 2 + N * sb_row + 2 * r * (K + N) + 2 * N)
    k1_gbs = k1_bytes / (k1_ms * 1e-3) / 1e9
    peak_mfma = PEAK_FP4_TFLOPS if mx else PEAK_INT8_TOPS
    # k2's bound: whichever roofline floor is longer at this shape
    k2_bound = "mfma" if ops_main / (peak_mfma * 1e12) >= k2_bytes / (PEAK_HBM_GBS * 1e9) else "hbm"
    if k2_bound == "mfma":
        k2_achieved, k2_peak, k2_unit = ops_main / (k2_ms * 1e-3) / 1e12, peak_mfma, "TFLOP/s"
    else:
        k2_achieved, k2_peak, k2_unit = k2_bytes / (k2_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    k2_tops = ops_main / (k2_ms * 1e-3) / 1e12
    kind = "MXFP4" if mx else "W4A4"
    if args.workload == "dit_proj" and not mx:
        metric = "fused W4A4+low-rank linear TOPS and tokens/s at M=4096,K=N=3072,r=32 (% MFMA peak)"
    else:
        metric = f"fused {kind}+low-rank linear TOPS and tokens/s at M={M},K={K},N={N},r={r} (% MFMA peak)"
    # stored traffic is keyed by workload, format and (when overridden) token rows
    tkey = args.workload + (f"_m{M}" if M != w.M else "") + ("_mxfp4" if mx else "")
    k1_file, k2_file = ("k1_smooth_quant.hip", "k2_mxfp4_gemm.hip") if mx else \
        ("k1_smooth_quant.hip", "k2_w4a4_gemm.hip")

    out = {
        "metric": metric,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp4 e2m1 + e8m0 block scales on block-scaled FP4 MFMA (fp32 acc), bf16 low-rank + output"
                  if mx else "int4 codes on int8 MFMA (int32 acc), fp32 epilogue, bf16 low-rank + output"),
        "data": "synthetic",
        "config": {"workload": args.workload, "format": args.format, "M": M, "K": K, "N": N, "rank": r,
                   "path": "fused" if fused else "two-kernel",
                   "group": 32 if mx else 64, "rotated_sets": nsets, "hip_graph": not args.no_graph},
        "tokens_per_s": round(tokens_s, 1),
        "pct_mfma_peak": round(100.0 * tops / peak_mfma, 2),
        "roofline": {
            "kernel": "mxfp4_gemm (k2)" if mx else "w4a4_gemm (k2)",
            "bound": k2_bound,
            "achieved": round(k2_achieved, 2),
            "peak": k2_peak,
            "unit": k2_unit,
            "frac": round(k2_achieved / k2_peak, 4),
            "algorithmic": {"ops": ops_main, "bytes": k2_bytes},
            "traffic": load_traffic(k2_file, tkey),
            "avg_launch_us": round(k2_ms * 1e3, 3),
        },
        "kernels": {
            "k1_smooth_quant_lora_down": {"avg_launch_us": round(k1_ms * 1e3, 3), "bound": "hbm",
                                          "algorithmic_bytes": k1_bytes, "achieved_GBs": round(k1_gbs, 1),
                                          "peak_GBs": PEAK_HBM_GBS, "frac": round(k1_gbs / PEAK_HBM_GBS, 4),
                                          "traffic": load_traffic(k1_file, tkey)},
            "k2_gemm": {"avg_launch_us": round(k2_ms * 1e3, 3), "ops": ops_main,
                        "achieved_TOPS": round(k2_tops, 2),
                        "pct_mfma_peak": round(100.0 * k2_tops / peak_mfma, 2),
                        "algorithmic_bytes": k2_bytes,
                        "achieved_GBs": round(k2_bytes / (k2_ms * 1e-3) / 1e9, 1)},
        },
        "graph": graph_info,
        "clock": {"settle_steps": settle_n, "settle_ms": round(settle_ms, 1), "sclk_mhz_eager": sclk_eager,
                  "source": "pp_dpm_sclk (current DPM level)"},
        "wall_s_timed": round(wall, 4),
        "pack_s": round(pack_s, 2),
    }

    if fused:   # one kernel: it is the dominant one, and k1/k2 do not run
        fb = (M * K * 2 + N * K // 2 + N * sb_row + r * K * 2 + N * r * 2 + K * 4 + 2 * N
              + M * N * 2)
        fkern = "mxfp4_fused_smallk" if mx else "w4a4_fused_smallk"
        f_bound = "mfma" if ops_main / (peak_mfma * 1e12) >= fb / (PEAK_HBM_GBS * 1e9) else "hbm"
        f_gbs = fb / (k1_ms * 1e-3) / 1e9
        f_tops = ops_main / (k1_ms * 1e-3) / 1e12
        f_ach, f_peak, f_unit = (f_tops, peak_mfma, "TFLOP/s") if f_bound == "mfma" else \
            (f_gbs, PEAK_HBM_GBS, "GB/s")
        out["roofline"] = {
            "kernel": f"{fkern} (quantize + lora_down + GEMM + lora_up in one kernel)",
            "bound": f_bound, "achieved": round(f_ach, 2), "peak": f_peak, "unit": f_unit,
            "frac": round(f_ach / f_peak, 4), "algorithmic": {"ops": ops_main, "bytes": fb},
            "traffic": load_traffic("k12_fused_smallk.hip", tkey),
            "avg_launch_us": round(k1_ms * 1e3, 3)}
        out["kernels"] = {fkern: {
            "avg_launch_us": round(k1_ms * 1e3, 3), "algorithmic_bytes": fb, "achieved_GBs": round(f_gbs, 1),
            "peak_GBs": PEAK_HBM_GBS, "frac_hbm": round(f_gbs / PEAK_HBM_GBS, 4), "ops": ops_main,
            "achieved_TOPS": round(f_tops, 2), "pct_mfma_peak": round(100.0 * f_tops / peak_mfma, 2)}}
        if graph_info:
            graph_info.pop("eager_k2_us", None)
            graph_info["eager_fused_us"] = graph_info.pop("eager_k1_us")

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, X, pk, b, args.cpu_seconds, mx)
    print(json.dumps(out), flush=True)


GRAPH_SETTLE_MS = 150.0


def time_graph(torch, launch, n, clock=None):
    """Capture launch(0..n-1) into one HIP graph, replay it untimed for
    GRAPH_SETTLE_MS of wall time (at least once: the capture leaves the GPU idle
    and the engine clock drops meanwhile), then once between HIP events on the
    current stream; returns ms per launch(i).  If `clock` is a list, the engine
    clock read while the timed replay runs is appended."""
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):       # warm the launch path outside the capture
        launch(0)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            launch(i)
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < GRAPH_SETTLE_MS:
        g.replay()
        torch.cuda.synchronize()
    gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gs.record()
    g.replay()
    ge.record()
    if clock is not None:
        clock.append(read_sclk_mhz())
    torch.cuda.synchronize()
    ms = gs.elapsed_time(ge) / n
    del g
    return ms


# The DiT block: (name, workload, activation, input); "H" is the up projection's output.
BLOCK = (("qkv", "dit_qkv", "none", "X"), ("out", "dit_out", "none", "X"),
         ("up", "mlp_up", "gelu_tanh", "X"), ("down", "mlp_down", "none", "H"))


def bench_block(args, S, synth, torch):
    mx = args.format == "mxfp4"
    dev = torch.device("cuda:0")

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    # ---- offline pack of the four layers (host, untimed): library packer, LoRA appended
    t0 = time.time()
    layers = []
    for name, wname, act, src in BLOCK:
        w = synth.WORKLOADS[wname]
        W = synth.weight(w)
        A = np.zeros(w.K, np.float32)
        S.svdq_act_absmax_update(synth.calibration_activations(w), A)
        pk = S.svdq_pack_weights(W, A, w.alpha, w.rank)
        if mx:
            pk["Wq"], pk["w_scales"] = S.svdq_quantize_residual_mxfp4(W, pk["smooth"], pk["L1"], pk["L2"])
        la, lb = synth.lora_factors(w)
        L1, L2 = S.svdq_append_lora(pk["smooth"], pk["L1"], pk["L2"], la, lb)
        X = synth.activations(w) if src == "X" else None
        layers.append(dict(name=name, w=w, act=act, src=src, M=w.M, K=w.K, N=w.N, r=L1.shape[0], X=X,
                           pk=dict(pk, L1=L1, L2=L2), b=synth.bias(w)))
    pack_s = time.time() - t0
    print(f"# packed dit_block in {pack_s:.1f}s", file=sys.stderr, flush=True)
    M = layers[0]["M"]
    assert all(L["M"] == M for L in layers)

    wsb = S.svdq_forward_workspace_bytes_mxfp4 if mx else S.svdq_forward_workspace_bytes
    quantize = S.svdq_forward_quantize_mxfp4 if mx else S.svdq_forward_quantize
    gemm = S.svdq_forward_gemm_act_mxfp4 if mx else S.svdq_forward_gemm_act
    acts = {"none": S.SVDQ_ACT_NONE, "gelu_tanh": S.SVDQ_ACT_GELU_TANH}
    per_set = 0
    for L in layers:
        L["ws_bytes"] = wsb(L["M"], L["K"], L["N"], L["r"])
        per_set += (L["M"] * L["K"] * 2 if L["X"] is not None else 0) + L["M"] * L["N"] * 2 + L["ws_bytes"] \
            + L["N"] * L["K"] // 2 + L["pk"]["w_scales"].nbytes + L["r"] * (L["K"] + L["N"]) * 2
    nsets = max(2, -(-args.rotate_mb * (1 << 20) // per_set))
    sets = []
    for i in range(nsets):
        d = []
        for L in layers:
            wsc = L["pk"]["w_scales"]
            e = dict(s=t(L["pk"]["smooth"]), L1=t(L["pk"]["L1"]), L2=t(L["pk"]["L2"]), Wq=t(L["pk"]["Wq"]),
                     ws=t(S.svdq_mxfp4_tile_scales(wsc) if mx else wsc), b=t(L["b"]),
                     Y=torch.empty((L["M"], L["N"]), dtype=torch.int16, device=dev),
                     work=torch.empty(L["ws_bytes"], dtype=torch.uint8, device=dev))
            e["X"] = t(L["X"]) if L["X"] is not None else None
            d.append(e)
        d[3]["X"] = d[2]["Y"]          # the down projection reads H = GELU(up) in place
        sets.append(d)
    torch.cuda.synchronize()

    def run(d, ev=None):
        for j, (L, e) in enumerate(zip(layers, d)):
            if ev is not None:
                ev[2 * j].record()
            quantize(e["X"], e["s"], e["L1"], e["work"])
            if ev is not None:
                ev[2 * j + 1].record()
            gemm(L["M"], L["K"], e["L2"], e["Wq"], e["ws"], e["b"], acts[L["act"]], e["Y"], e["work"], L["r"])
        if ev is not None:
            ev[2 * len(layers)].record()

    settle_n, settle_ms = settle(torch, lambda i: run(sets[i % nsets]), args.settle_ms)
    for i in range(args.warmup):
        run(sets[i % nsets])
    torch.cuda.synchronize()
    nev = 2 * len(layers) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        run(sets[i % nsets], evs[i])
    end.record()
    sclk_eager = read_sclk_mhz()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = eager_ms_step = start.elapsed_time(end) / args.steps
    dur = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(nev - 1)] for e in evs]).mean(axis=0)
    if not args.no_graph:
        ms_step = time_graph(torch, lambda i: run(sets[i % nsets]), args.steps)

    peak_mfma = PEAK_FP4_TFLOPS if mx else PEAK_INT8_TOPS
    sb_row = lambda K: K // 32 if mx else 4 * (K // 64)
    kern = {}
    ops_total = 0.0
    for j, L in enumerate(layers):
        M_, K, N, r = L["M"], L["K"], L["N"], L["r"]
        ops_main, ops_low = 2.0 * M_ * N * K, 2.0 * M_ * r * (K + N)
        ops_total += ops_main + ops_low
        k1_ms, k2_ms = float(dur[2 * j]), float(dur[2 * j + 1])
        k1_bytes = M_ * (2 * K + K // 2 + sb_row(K) + 4 * r) + r * K * 2 + K * 4
        k2_bytes = (M_ * (K // 2 + sb_row(K) + 4 * r + 2 * N) + N * K // 2 + N * sb_row(K)
                    + 2 * r * (K + N) + 2 * N)
        kern[L["name"]] = {
            "M": M_, "K": K, "N": N, "r": r, "activation": L["act"],
            "k1_us": round(k1_ms * 1e3, 3), "k1_GBs": round(k1_bytes / (k1_ms * 1e-3) / 1e9, 1),
            "k2_us": round(k2_ms * 1e3, 3), "k2_ops": ops_main, "k2_bytes": k2_bytes,
            "k2_TOPS": round(ops_main / (k2_ms * 1e-3) / 1e12, 2),
            "k2_pct_mfma_peak": round(100.0 * ops_main / (k2_ms * 1e-3) / 1e12 / peak_mfma, 2)}
    dom = max(kern, key=lambda k: kern[k]["k2_us"])
    dk = kern[dom]
    dom_us = dk["k2_us"]
    if not args.no_graph:    # the dominant GEMM alone, K back-to-back launches from a graph
        j = [L["name"] for L in layers].index(dom)
        L = layers[j]

        def k2_only(i):
            e = sets[i % nsets][j]
            gemm(L["M"], L["K"], e["L2"], e["Wq"], e["ws"], e["b"], acts[L["act"]], e["Y"], e["work"], L["r"])
        dom_us = round(time_graph(torch, k2_only, args.steps) * 1e3, 3)
    achieved = dk["k2_ops"] / (dom_us * 1e-6) / 1e12
    tops = ops_total / (ms_step * 1e-3) / 1e12
    kind = "MXFP4" if mx else "W4A4"
    out = {
        "metric": (f"fused {kind}+low-rank DiT block (QKV 3072->9216, out 3072->3072, MLP 3072->12288 +GELU "
                   f"->3072; r=32+16 LoRA) TOPS and tokens/s at M={M} (% MFMA peak)"),
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp4 e2m1 + e8m0 block scales on block-scaled FP4 MFMA (fp32 acc), bf16 low-rank + output"
                  if mx else "int4 codes on int8 MFMA (int32 acc), fp32 epilogue, bf16 low-rank + output"),
        "data": "synthetic",
        "config": {"workload": "dit_block", "format": args.format, "M": M, "layers": [L["name"] for L in layers],
                   "rank": layers[0]["r"], "rotated_sets": nsets, "hip_graph": not args.no_graph},
        "eager_ms_per_step": round(eager_ms_step, 5),
        "tokens_per_s": round(M / (ms_step * 1e-3), 1),
        "pct_mfma_peak": round(100.0 * tops / peak_mfma, 2),
        "roofline": {"kernel": f"{'mxfp4' if mx else 'w4a4'}_gemm (k2) of the {dom} projection", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": peak_mfma, "unit": "TFLOP/s",
                     "frac": round(achieved / peak_mfma, 4),
                     "algorithmic": {"ops": dk["k2_ops"], "bytes": dk["k2_bytes"]}, "traffic": None,
                     "avg_launch_us": dom_us},
        "kernels": kern,
        "wall_s_timed": round(wall, 4),
        "clock": {"settle_steps": settle_n, "settle_ms": round(settle_ms, 1), "sclk_mhz_eager": sclk_eager,
                  "source": "pp_dpm_sclk (current DPM level)"},
        "pack_s": round(pack_s, 2),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_block(layers, args.cpu_seconds, mx)
    print(json.dumps(out), flush=True)


def cpu_baseline_block(layers, seconds, mx):
    """The CPU oracle on the same few token rows through the four layers (its own chain)."""
    from oracle import svdq_oracle as O
    cores = blas_threads()
    fwd = O.forward_mx if mx else O.forward
    rows, dt = 4, 0.0
    for _ in range(5):
        t0 = time.perf_counter()
        H = None
        for L in layers:
            X = L["X"][:rows] if L["src"] == "X" else O.bf16_from_f64(H)
            Y = fwd(X, L["pk"]["smooth"], L["pk"]["L1"], L["pk"]["L2"], L["pk"]["Wq"], L["pk"]["w_scales"],
                    L["b"], activation=None if L["act"] == "none" else L["act"])
            if L["name"] == "up":
                H = Y
        dt = time.perf_counter() - t0
        if dt >= 0.5 * seconds or rows >= 256:
            break
        rows = int(min(256, max(rows + 1, rows * min(8.0, 1.2 * seconds / max(dt, 1e-3)))))
    ops = sum(2.0 * rows * L["N"] * L["K"] + 2.0 * rows * L["r"] * (L["K"] + L["N"]) for L in layers)
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "tokens_per_s": round(rows / dt, 2),
            "cores": cores, **host_cpu(), "kind": "oracle", "seconds": round(dt, 2),
            "sample": (f"{rows} token rows through the four block linears (full K and N, r=48), float64 numpy "
                       f"oracle chain on host cores")}


def cpu_baseline(w, X, pk, b, seconds, mx=False):
    """The CPU oracle (as it stands) on a bounded sample of rows of the same workload."""
    from oracle import svdq_oracle as O
    cores = blas_threads()
    fwd = O.forward_mx if mx else O.forward
    # grow the sample until it takes about `seconds` (whole workload, repeated, if it is smaller)
    rows, passes, dt = 16, 1, 0.0
    for _ in range(6):
        t0 = time.perf_counter()
        for _ in range(passes):
            fwd(X[:rows], pk["smooth"], pk["L1"], pk["L2"], pk["Wq"], pk["w_scales"], b)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * seconds or passes >= 8:
            break
        grow = min(8.0, 1.2 * seconds / max(dt, 1e-3))
        if rows < X.shape[0]:
            rows = int(min(X.shape[0], max(rows + 1, rows * grow)))
        else:
            passes = int(min(8, max(passes + 1, passes * grow)))
    done = rows * passes
    ops = 2.0 * done * w.N * w.K + 2.0 * done * w.rank * (w.K + w.N)
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "tokens_per_s": round(done / dt, 2),
            "cores": cores, **host_cpu(), "kind": "oracle", "seconds": round(dt, 2),
            "sample": (f"{rows} of {X.shape[0]} token rows of {w.name} x {passes} pass(es) (full K={w.K}, N={w.N}, "
                       f"r={w.rank}), float64 numpy oracle forward on host cores")}


if __name__ == "__main__":
    main()
