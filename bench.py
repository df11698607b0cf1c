#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config hy3]

One step = one moe_layer_forward call (router logits, gate top-k, routing,
grouped GEMM1 + SwiGLU, grouped GEMM2, shared expert if any, combine) over
one batch of synthetic tokens already resident in HBM.  W untimed warm-up
steps, then exactly K timed steps bracketed by torch.cuda.synchronize().
The grouped GEMM1 kernel (the largest weight stream) is timed with HIP events
recorded by the library around its launch in every timed step; its roofline
fraction is reported against MI355X's 8 TB/s HBM (decode) or its dense MFMA
peak (prefill, with the HBM fraction and max(t_flop, t_byte) / t beside it).
The default workload is the largest one, the Hy3-style layer (T = 4096,
E = 192, shared expert).  The CPU oracle is timed on
a bounded sample of the same workload on the host's cores.  Prints one JSON
line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill) vs peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0     # dense fp8 MFMA (the scaled FP8 x FP4 instruction runs at this rate)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="hy3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the second timing of the layer replayed from a captured HIP graph")
    ap.add_argument("--cold-steps", type=int, default=0,
                    help="also time this many steps with a 512 MiB read before each one (L2 and "
                         "Infinity Cache evicted), by HIP events around each step")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0,
                    help="wall-clock budget of the oracle sample")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 times) and "
                         "exit: the reference for scaling HBM byte counters")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="print the HBM-counter summary (markdown) of a rocprofv3 --pmc FETCH_SIZE / "
                         "WRITE_SIZE pair of runs of this bench and of --calibrate-copy-mib 1024, and exit")
    return ap.parse_args()


# The kernel each bench config grades (layers: GEMM1, w13 + SwiGLU; the norm
# configs: their one kernel): the sources it is built from and the
# kernel-name prefix rocprofv3 reports.  A counter summary
# (profiles/hbm_counters_<config>.md) records the hash of those sources; its
# byte counts are reported as roofline.traffic only while the hash matches.
_CSRC = "expert_routing_grouped_gate_amd/csrc/"
GEMM1 = {
    "bf16_stream": ((_CSRC + "ffn_bf16.hip", _CSRC + "common.hpp"), "ffn_skinny<true"),
    "bf16_tiled": ((_CSRC + "tiled_bf16.hip", _CSRC + "common.hpp", _CSRC + "mxfmt.hpp"), "ffn_tiled4<true"),
    "w4a8_stream": ((_CSRC + "mx.hip", _CSRC + "common.hpp", _CSRC + "mxfmt.hpp"), "ffn_mx_stream<true"),
    "w4a8_tiled": ((_CSRC + "mx_tiled.hip", _CSRC + "common.hpp", _CSRC + "mxfmt.hpp"), "ffn_mx_tiled<true"),
}
_NORM_SRC = (_CSRC + "norm.hip", _CSRC + "rowops.hpp", _CSRC + "common.hpp", _CSRC + "mxfmt.hpp")
NORM_KERNELS = {
    "add_rmsnorm": (_NORM_SRC, "add_rmsnorm_kernel"),
    "add_rmsnorm_mx": (_NORM_SRC, "add_rmsnorm_kernel"),
    "combine_add_rmsnorm": (_NORM_SRC, "combine_add_rmsnorm_kernel"),
}


def gemm1_streams(cfg) -> bool:
    """The library's kernel choice for this layer (the model shapes, where
    the tiled kernels fit): the weight-streaming GEMMs with at most 16
    tokens, or with at most 3 (bf16) / 8 (W4A8) rows per expert on average
    and no bf16 shared expert with shared_I == I; else the LDS-tiled ones."""
    if cfg.T <= 16:
        return True
    R = cfg.T * cfg.k
    if cfg.fmt == "w4a8":
        return R <= 8 * cfg.E
    return not (cfg.shared_I > 0 and cfg.shared_I == cfg.I) and R <= 3 * cfg.E


def gemm1_family(cfg) -> str:
    return ("w4a8_" if cfg.fmt == "w4a8" else "bf16_") + ("stream" if gemm1_streams(cfg) else "tiled")


def counters_md(config: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_counters_{config}.md")


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it does not write back and invalidate the caches, so it does
    not put a bubble into the stream it times (a default event costs ~3 us
    per record here).  The library records it on the layer's stream around
    the GEMM1 launch; elapsed times are read after a device synchronise."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")   # the runtime torch already loaded
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            TimingEvent._hip = hip
        self._lib = TimingEvent._hip   # (held by the instance: module globals may be gone in __del__)
        h = ctypes.c_void_p()
        rc = self._lib.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value   # the handle MoeLayer.time_ffn_up passes to the library

    def record(self, stream_handle) -> None:
        """Record on a stream (a hipStream_t handle, e.g. torch's
        current_stream().cuda_stream)."""
        rc = self._lib.hipEventRecord(self.cuda_event, stream_handle)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, end: "TimingEvent") -> float:
        import ctypes
        f = ctypes.c_float()
        rc = self._lib.hipEventElapsedTime(ctypes.byref(f), self.cuda_event, end.cuda_event)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(f.value)

    def __del__(self):
        lib, ev = getattr(self, "_lib", None), getattr(self, "cuda_event", None)
        if lib is not None and ev:
            try:
                lib.hipEventDestroy(ev)
            except Exception:   # interpreter shutdown: nothing left to release to
                pass


def graded_kernel(config: str):
    """(sources, rocprofv3 kernel-name prefix) of the kernel a bench config grades."""
    if config in NORM_KERNELS:
        return NORM_KERNELS[config]
    return GEMM1[gemm1_family(_layer_configs()[config])]


def source_hash(sources) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gemm1_source_hash(family: str) -> str:
    return source_hash(GEMM1[family][0])


def _counter_means(path):
    import collections
    import csv
    d = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        d[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in d.items()}


COUNTER_TITLES = {
    "qwen3_decode": "Qwen3-style decode layer (T=16, H=4096, E=128, top-8, I=1536, bf16)",
    "qwen3_prefill": "Qwen3-style prefill layer (T=4096, H=4096, E=128, top-8, I=1536, bf16)",
    "qwen3_decode_w4a8": "Qwen3-style decode layer with W4A8 experts (T=16, H=4096, E=128, top-8, I=1536, "
                         "MXFP4 weights, MXFP8 activations, Zipf router bias)",
    "qwen3_prefill_w4a8": "Qwen3-style prefill layer with W4A8 experts (T=4096, H=4096, E=128, top-8, I=1536, "
                          "MXFP4 weights, MXFP8 activations)",
    "hy3": "Hy3-style layer (T=4096, H=4096, E=192, top-8 sigmoid x2.826, I=1536, shared expert I=1536, bf16)",
    "add_rmsnorm": "residual add + RMSNorm before the layer (T=4096, H=4096, fp32 + bf16 outputs, bf16 residual)",
}


def summarize_counters(config, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Markdown summary of HBM byte counters per kernel, scaled by what the
    same counters read for a plain 1 GiB device copy."""
    fetch, write = _counter_means(fetch_csv), _counter_means(write_csv)
    cf = max(v for k, v in _counter_means(copy_fetch_csv).items() if "copyBuffer" in k)
    cw = max(v for k, v in _counter_means(copy_write_csv).items() if "copyBuffer" in k)
    kib = 1024 * 1024  # the copy moves 1 GiB = 1,048,576 KiB each way
    sf, sw = kib / cf, kib / cw
    run = f"python $R/bench.py --config {config} --steps 5 --warmup 2 --no-cpu-baseline --no-graph"
    lines = [f"# HBM byte counters, {COUNTER_TITLES.get(config, config)}", "",
             "Each counter in its own pass (run from /tmp on one MI355X, repo at $R, output under $OUT):", "", "```",
             f"rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_FETCH_SIZE_{config} -o run --output-format csv -- {run}",
             f"rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_WRITE_SIZE_{config} -o run --output-format csv -- {run}",
             "rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_FETCH_SIZE_copy -o run --output-format csv -- python $R/bench.py --calibrate-copy-mib 1024",
             "rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_WRITE_SIZE_copy -o run --output-format csv -- python $R/bench.py --calibrate-copy-mib 1024",
             f"python $R/bench.py --config {config} --summarize-counters <the four run_counter_collection.csv files>",
             "```", "",
             f"Calibration (1 GiB device copy): FETCH_SIZE {cf:,.1f} KiB -> scale x{sf:.3f}; "
             f"WRITE_SIZE {cw:,.1f} KiB -> scale x{sw:.3f}.", "",
             "| kernel | FETCH_SIZE KiB | read bytes (scaled) | WRITE_SIZE KiB | written bytes (scaled) |",
             "|---|---|---|---|---|"]
    g1 = None
    graded = graded_kernel(config) if (config in NORM_KERNELS or config in _layer_configs()) else None
    for k in sorted(fetch, key=lambda k: -fetch[k]):
        if not k.startswith(("void moe::", "moe::")):
            continue
        rb, wb = fetch[k] * sf * 1024, write.get(k, 0.0) * sw * 1024
        lines.append(f"| `{k[:80]}` | {fetch[k]:,.1f} | {rb / 1e9:.4f} GB | {write.get(k, 0.0):,.1f} | {wb / 1e6:.3f} MB |")
        if graded is not None and graded[1] in k.split("(")[0] and g1 is None:
            g1 = (rb, wb)
    if graded is not None:
        lines += ["", "Machine-readable (bench.py reports `roofline.traffic` from these only while the graded "
                  "kernel's sources still hash to the value below):", "",
                  f"kernel: {graded[1]}",
                  f"kernel_source_sha256_16: {source_hash(graded[0])}",
                  f"kernel_read_bytes: {int(g1[0]) if g1 else 0}",
                  f"kernel_write_bytes: {int(g1[1]) if g1 else 0}"]
    lines.append("")
    print("\n".join(lines))


def _layer_configs():
    from expert_routing_grouped_gate_amd import workloads as W
    return W.CONFIGS


def measured_traffic(config: str):
    """HBM bytes per launch of the graded kernel from the committed counter
    summary of this config, or None when it is missing or was taken on other
    sources of that kernel."""
    try:
        kv = {}
        for line in open(counters_md(config)):
            if ":" in line and line.split(":")[0].strip() in ("kernel_source_sha256_16", "kernel_read_bytes",
                                                              "kernel_write_bytes"):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
        if kv.get("kernel_source_sha256_16") != source_hash(graded_kernel(config)[0]):
            return None
        return int(kv["kernel_read_bytes"]) + int(kv["kernel_write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def measured_gemm1_traffic(cfg):
    return measured_traffic(cfg.name)


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def calibrate_copy(mib: int):
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {mib} MiB 5 times")


def workload_bytes_flops(cfg, counts):
    """Algorithmic work of one layer call: weights of the experts the routing
    touched (+ shared expert), router weight and bias, x in, out out; flops
    of the routed and shared expert GEMMs."""
    n_touched = int((counts > 0).sum())
    R = cfg.T * cfg.k
    if cfg.fmt == "w4a8":
        w13_e = 2 * cfg.I * cfg.H // 2 + 2 * cfg.I * cfg.H // 32
        w2_e = cfg.H * cfg.I // 2 + cfg.H * cfg.I // 32
    else:
        w13_e = 2 * cfg.I * cfg.H * 2
        w2_e = cfg.H * cfg.I * 2
    shared = 0
    if cfg.shared_I:
        shared = 3 * cfg.shared_I * cfg.H * 2
    layer_bytes = (n_touched * (w13_e + w2_e) + shared + cfg.E * cfg.H * 4
                   + (cfg.E * 4 if cfg.bias != "none" else 0) + 2 * cfg.T * cfg.H * 2)
    flops = 2 * R * 3 * cfg.I * cfg.H + 2 * cfg.T * 3 * cfg.shared_I * cfg.H
    # GEMM1 (w13 + SwiGLU) alone: touched w13 slices, x read, act written
    act_b = R * cfg.I * (1 + 1 / 32 if cfg.fmt == "w4a8" else 2)
    g1_bytes = n_touched * w13_e + cfg.T * cfg.H * 2 + act_b
    g1_flops = 2 * R * 2 * cfg.I * cfg.H
    # bf16 with shared_I == I on the tiled GEMMs: the library runs the shared
    # expert as one more group of the GEMM1 launch (its w13, its activations
    # written, its flops)
    g1_shared = (cfg.fmt == "bf16" and cfg.shared_I > 0 and cfg.shared_I == cfg.I
                 and not gemm1_streams(cfg))
    if g1_shared:
        g1_bytes += 2 * cfg.shared_I * cfg.H * 2 + cfg.T * cfg.shared_I * 2
        g1_flops += 2 * cfg.T * 2 * cfg.shared_I * cfg.H
    return dict(n_touched=n_touched, layer_bytes=layer_bytes, flops=flops,
                g1_bytes=int(g1_bytes), g1_flops=g1_flops, g1_shared=g1_shared)


def cpu_baseline(cfg, cpu, budget_s):
    """The oracle as it stands, token by token on the host, until the budget
    is spent or every token is done."""
    import numpy as np
    import threadpoolctl
    import torch

    from oracle import moe, mx

    x = cpu["x"].to(torch.float64).numpy()
    wr = cpu["wr"].numpy()
    bias = None if cpu["bias"] is None else cpu["bias"].numpy()

    def expert(e):
        if cfg.fmt == "w4a8":
            return (mx.mxfp4_dequant(cpu["w13"][e].numpy(), cpu["w13_scales"][e].numpy(), cfg.H),
                    mx.mxfp4_dequant(cpu["w2"][e].numpy(), cpu["w2_scales"][e].numpy(), cfg.I))
        return cpu["w13"][e].to(torch.float64).numpy(), cpu["w2"][e].to(torch.float64).numpy()

    shared = None
    if cfg.shared_I:
        shared = (cpu["shared_w13"].to(torch.float64).numpy(), cpu["shared_w2"].to(torch.float64).numpy())
    done = 0
    t0 = time.perf_counter()
    while done < cfg.T and time.perf_counter() - t0 < budget_s:
        moe.layer_forward(x, wr, cfg.k, cfg.gate, expert, cfg.E, bias=bias, routed_scale=cfg.routed_scale,
                          eps=cfg.eps, shared_weights=shared, fmt=cfg.fmt, tokens=[done])
        done += 1
    dt = time.perf_counter() - t0
    blas = [i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    cores = max([torch.get_num_threads()] + blas)
    return {"value": done / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {done} of {cfg.T} tokens of the same layer, one oracle call per token "
                      f"(fp64 numpy; routing over all tokens each call), {dt:.1f} s",
            "cpu_model": host_cpu_model(), "host_cpus": os.cpu_count()}


NORM_CONFIGS = {
    # the norm before the MoE layer at the prefill shape: "RMSNorm + Cast"
    # (fp32 for the gate, bf16 for the experts, the residual) and "RMSNorm +
    # MX quant" (MXFP8 codes and scales, the residual)
    "add_rmsnorm": dict(T=4096, H=4096, mx=False),
    "add_rmsnorm_mx": dict(T=4096, H=4096, mx=True),
}


def bench_combine_norm(args):
    """The layer's combine fused with the next step's residual add + RMSNorm
    (moe_combine_add_rmsnorm) at the prefill layer's shape: one step = one
    call over T tokens with the fp32 + bf16 + residual outputs; fence-free
    HIP events around each call; the separate moe_combine + moe_add_rmsnorm
    calls are timed the same way in the same run for comparison."""
    import torch

    from expert_routing_grouped_gate_amd import binding as B
    from expert_routing_grouped_gate_amd import workloads as W

    T, k, H = 4096, 8, 4096
    eps = 1e-6
    y, pp, w = (t.cuda() for t in W.draw_combine_inputs(T, k, H, seed=4097))
    _, r, g = (t.cuda() for t in W.draw_norm_inputs(T, H, seed=4098))
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def fused():
        B.combine_add_rmsnorm(y, pp, w, None, g, eps, r)

    def separate():
        B.combine(y, pp, w, None, out)
        B.add_rmsnorm(out, g, eps, r)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
        t0 = time.perf_counter()
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, sum(a.elapsed_ms(b) for a, b in ev) / args.steps

    ms, k_ms = timed(fused)
    sep_ms, sep_k_ms = timed(separate)
    alg = int(T * k * H * 2 + T * H * 2 + T * k * 8 + H * 2 + T * H * (4 + 2 + 2))
    gbs = alg / (k_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"combine_add_rmsnorm: the layer's combine (T={T}, top-{k}, H={H}) fused with "
                               "the next residual add + RMSNorm (fp32 + bf16 outputs, bf16 residual)",
                   "T": T, "k": k, "H": H, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config),
                     "kernel": "combine_add_rmsnorm_kernel", "kernel_ms": round(k_ms, 5), "algorithmic_bytes": alg},
        "separate": {"ms_per_step": round(sep_ms, 5), "events_ms": round(sep_k_ms, 5),
                     "calls": "moe_combine + moe_add_rmsnorm"},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def bench_norm(args):
    """The residual add + RMSNorm step (moe_add_rmsnorm) alone: one step =
    one call over T tokens, inputs resident in HBM; fence-free HIP events on
    the stream the binding launches on (torch's current stream) around every
    timed call."""
    import numpy as np
    import torch

    from expert_routing_grouped_gate_amd import binding as B
    from expert_routing_grouped_gate_amd import workloads as W

    c = NORM_CONFIGS[args.config]
    T, H, use_mx = c["T"], c["H"], c["mx"]
    eps = 1e-6
    x, r, w = W.draw_norm_inputs(T, H, seed=4096)
    xd, rd, wd = x.cuda(), r.cuda(), w.cuda()
    kw = dict(f32=not use_mx, bf16=not use_mx, residual_out=True, mx=use_mx)
    for _ in range(args.warmup):
        B.add_rmsnorm(xd, wd, eps, rd, **kw)
    torch.cuda.synchronize()
    K = args.steps
    ev = [(TimingEvent(), TimingEvent()) for _ in range(K)]
    stream = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        B.add_rmsnorm(xd, wd, eps, rd, **kw)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    k_ms = sum(a.elapsed_ms(b) for a, b in ev) / K
    out_b = (1 + 1 / 32 + 2) if use_mx else (4 + 2 + 2)
    alg = int(2 * T * H * 2 + H * 2 + out_b * T * H)
    gbs = alg / (k_ms * 1e-3) / 1e9
    cpu_b = None
    if not args.no_cpu_baseline:
        from oracle import norm
        import threadpoolctl
        xs, rs, ws = x.double().numpy(), r.double().numpy(), w.double().numpy()
        n, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < min(args.cpu_budget_s, 5.0):
            norm.add_rmsnorm(xs, rs, ws, eps)
            n += 1
        dt = time.perf_counter() - t1
        blas = [i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        cpu_b = {"value": round(n * T / dt, 1), "unit": "tokens/s", "cores": max([1] + blas), "kind": "oracle",
                 "sample": f"{n} oracle calls over all {T} tokens (fp64 numpy), {dt:.1f} s",
                 "cpu_model": host_cpu_model(), "host_cpus": os.cpu_count()}
    form = "MXFP8 codes + scales and bf16 residual" if use_mx else "fp32 + bf16 outputs and bf16 residual"
    res = {
        "metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.config}: residual add + RMSNorm before the MoE layer, T={T} H={H}, {form}",
                   "T": T, "H": H, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config), "kernel": "add_rmsnorm_kernel",
                     "kernel_ms": round(k_ms, 5), "algorithmic_bytes": alg},
        "cpu_baseline": cpu_b,
    }
    print(json.dumps(res), flush=True)


def time_graph_replay(layer, x, out, K, Wm):
    """The layer step captured once into a HIP graph (the library reads no
    device value on the host, so one capture serves every step) and replayed:
    W untimed replays, then K replays bracketed by device synchronisations.
    Every replay must reproduce the eager output bit for bit."""
    import torch
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(x, out)  # a first call on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, out)
    for _ in range(Wm):
        g.replay()
    torch.cuda.synchronize()
    log(f"[bench] timing {K} graph replays")
    t0 = time.perf_counter()
    for _ in range(K):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    if not torch.equal(out, eager):
        raise RuntimeError("graph replay output differs from the eager step")
    del g
    return {"ms_per_step": round(ms, 5), "matches_eager": True}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.config, *args.summarize_counters)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from expert_routing_grouped_gate_amd import binding as B
    from expert_routing_grouped_gate_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    B.load()
    if args.config in NORM_CONFIGS:
        bench_norm(args)
        return
    if args.config == "combine_add_rmsnorm":
        bench_combine_norm(args)
        return
    cfg = W.CONFIGS[args.config]
    log(f"[bench] drawing {cfg.name}")
    cpu = W.draw_layer(cfg, progress=log)
    dev = {k: (v.to("cuda") if v is not None else None) for k, v in cpu.items()}
    fmt = B.FMT_W4A8 if cfg.fmt == "w4a8" else B.FMT_BF16
    w = B.ExpertWeights(H=cfg.H, I=cfg.I, E=cfg.E, fmt=fmt, w13=dev["w13"], w2=dev["w2"],
                        w13_scales=dev.get("w13_scales"), w2_scales=dev.get("w2_scales"),
                        shared_I=cfg.shared_I, shared_w13=dev.get("shared_w13"),
                        shared_w2=dev.get("shared_w2"))
    mode = B.GATE_SIGMOID if cfg.gate == "sigmoid" else B.GATE_SOFTMAX
    layer = B.MoeLayer(w, dev["wr"], cfg.k, mode, dev["bias"], cfg.routed_scale, cfg.eps)
    x = dev["x"]
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    layer.alloc(cfg.T, x.device)

    K, Wm = args.steps, args.warmup
    ev = [(TimingEvent(), TimingEvent()) for _ in range(K)]
    ev_step = [(TimingEvent(), TimingEvent()) for _ in range(K)]
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    log(f"[bench] warm-up {Wm} steps")
    for _ in range(Wm):
        layer.forward(x, out)
    torch.cuda.synchronize()
    log(f"[bench] timing {K} steps")
    t0 = time.perf_counter()
    for i in range(K):
        layer.time_ffn_up(*ev[i])
        layer.forward(x, out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    layer.time_ffn_up(None, None)
    g1_ms = sum(a.elapsed_ms(b) for a, b in ev) / K
    ms = elapsed * 1e3 / K

    # a second pass of K steps, each between two events, for the median and
    # min (their records cost launch time, so the timed pass has none)
    for a, b in ev_step:
        a.record(stream)
        layer.forward(x, out)
        b.record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_ms(b) for a, b in ev_step)

    cold = None
    if args.cold_steps > 0:
        # each step after a read of 512 MiB (outside its events): the touched
        # weights come from HBM, not from a cache the previous step filled.
        # A read, not a write: a written buffer leaves the Infinity Cache
        # full of dirty lines whose write-back the timed step would pay for.
        flush = torch.ones(64 << 20, dtype=torch.int64, device="cuda")
        sink = torch.empty(1, dtype=torch.int64, device="cuda")
        for _ in range(3):
            torch.sum(flush, dim=0, keepdim=True, out=sink)
        torch.cuda.synchronize()
        ev_cold = [(TimingEvent(), TimingEvent()) for _ in range(args.cold_steps)]
        for a, b in ev_cold:
            torch.sum(flush, dim=0, keepdim=True, out=sink)
            a.record(stream)
            layer.forward(x, out)
            b.record(stream)
        torch.cuda.synchronize()
        c = sorted(a.elapsed_ms(b) for a, b in ev_cold)
        cold = {"steps": args.cold_steps, "median_ms": round(c[len(c) // 2], 5), "min_ms": round(c[0], 5),
                "flush_read_bytes": 512 << 20}
        del flush

    graph = None if args.no_graph else time_graph_replay(layer, x, out, K, Wm)

    counts = layer.buf["counts"].cpu().numpy()
    wl = workload_bytes_flops(cfg, counts)
    g1_gbs = wl["g1_bytes"] / (g1_ms * 1e-3) / 1e9
    layer_gbs = wl["layer_bytes"] / (ms * 1e-3) / 1e9
    layer_tflops = wl["flops"] / (ms * 1e-3) / 1e12
    # the contraction's own dense peak: bf16, or fp8 for the scaled FP8 x FP4 MFMA
    mfma_peak = FP8_PEAK_TFLOPS if cfg.fmt == "w4a8" else BF16_PEAK_TFLOPS
    traffic = measured_gemm1_traffic(cfg)
    g1_t_byte = wl["g1_bytes"] / (HBM_PEAK_GBS * 1e9)
    g1_t_flop = wl["g1_flops"] / (mfma_peak * 1e12)
    # graded on HBM while the GEMM's flops at the dense MFMA peak take less
    # than half the time of its bytes at the HBM peak (decode and mid-size
    # layers), else on MFMA (the prefill layers: 0.7-1.5x)
    if 2 * g1_t_flop < g1_t_byte:
        roof = {"bound": "hbm", "achieved": round(g1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(g1_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        g1_tf = wl["g1_flops"] / (g1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(g1_tf, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(g1_tf / mfma_peak, 4), "traffic": traffic,
                "hbm_gbs": round(g1_gbs, 1), "hbm_frac": round(g1_gbs / HBM_PEAK_GBS, 4)}
    roof.update({"kernel": f"grouped GEMM1 (w13 + SwiGLU{' + shared expert' if wl['g1_shared'] else ''})",
                 "kernel_ms": round(g1_ms, 4),
                 "roof_frac": round(max(g1_t_byte, g1_t_flop) / (g1_ms * 1e-3), 4),
                 "algorithmic_bytes": wl["g1_bytes"], "algorithmic_flops": wl["g1_flops"]})
    layer_t_byte = wl["layer_bytes"] / (HBM_PEAK_GBS * 1e9)
    layer_t_flop = wl["flops"] / (mfma_peak * 1e12)

    cpu_b = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        cpu_b = cpu_baseline(cfg, cpu, args.cpu_budget_s)

    desc = (f"{cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} top-{cfg.k} {cfg.gate}"
            f"{' x%.3f' % cfg.routed_scale if cfg.gate == 'sigmoid' else ''} I={cfg.I}"
            f"{' shared I=%d' % cfg.shared_I if cfg.shared_I else ''} {cfg.fmt}")
    res = {
        "metric": METRIC, "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wm, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4xmxfp8" if cfg.fmt == "w4a8" else "bf16", "data": "synthetic",
        "config": {"workload": desc, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                   "experts_touched": wl["n_touched"], "parallelism": "single GPU"},
        "layer": {"hbm_gbs": round(layer_gbs, 1), "hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
                  "tflops": round(layer_tflops, 2), "mfma_frac": round(layer_tflops / mfma_peak, 4),
                  "roof_frac": round(max(layer_t_byte, layer_t_flop) / (ms * 1e-3), 4),
                  "roof_bound": "hbm" if layer_t_byte >= layer_t_flop else "mfma",
                  "algorithmic_bytes": wl["layer_bytes"], "flops": wl["flops"]},
        "roofline": roof,
        "cpu_baseline": cpu_b,
    }
    res["step_ms"] = {"median": round(step_ms[K // 2], 5), "min": round(step_ms[0], 5),
                      "source": "HIP events around each step of a second pass of K steps"}
    if cold is not None:
        res["cold"] = cold
    if graph is not None:
        res["graph"] = dict(graph, tokens_per_s=round(cfg.T / (graph["ms_per_step"] * 1e-3), 1))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
