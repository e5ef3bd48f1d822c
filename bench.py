#!/usr/bin/env python3
"""Benchmark of the W4A8 MoE routed-expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]

A step is one pass of the whole layer (quant_act, route, permute, gate/up
grouped GEMM, SwiGLU, down grouped GEMM, combine) over one batch of
synthetic tokens, inputs already resident in HBM.  The default workload is
decode at 128 tokens (H=6144, I=2048, 256 experts, top-8), the shape the
headline value is quoted on; the same run then times the 8K-token prefill
(the metric's other half) into a "prefill" block of the line and the skewed
16K-token prefill into a "skewed_prefill" block (--no-prefill skips both;
--config 3 or 4 makes either the headline workload), and decode at 256 tokens
with Zipf(1.1)-skewed routing into a "skewed_decode" block (--no-skewed skips
it; --config 5 makes it the headline workload).  Each workload also reports
the median, p10 and p90 of single graph replays, timed after its timed region.

Prints ONE JSON line: layer tokens/s, the roofline of the dominant kernel
(the gate/up grouped GEMM, timed with events on its own stream: HBM bytes
where its FLOPs per algorithmic byte are below the chip's ridge point, as at
decode, FP8 MFMA FLOPs above it, as at prefill), and the CPU oracle timed on
a bounded sample of the decode workload on every host core and on one.

The step is timed twice over K steps: launched kernel by kernel with events
around each kernel (the per-kernel times and the roofline's launch duration),
and replayed from a HIP graph of the same step (one launch per step: the
headline value; --no-graph reports the eager rate instead).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + % HBM peak (decode T=128) and % FP8 MFMA peak (prefill T=8192)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published (no sparsity)
FP64_PEAK_TFLOPS = 78.6        # MI355X fp64 vector, published
# fp64 operations of the clip-ratio search per weight: for each of the 11
# ratios the residual w - q s (2), its square and its sum (2)
FP64_OPS_PER_WEIGHT = 44


KERNEL_SOURCES = {"gg_stream": "gemm_stream.hip", "gg_tiled": "gemm_tiled.hip"}


def kernel_sources_hash(kernel: str) -> str:
    """Hash of one grouped-GEMM kernel's sources: counter files taken on other code are ignored."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_grouped_gemm_token_amd", "csrc")
    for name in ("common.hpp", "gemm_common.hpp", KERNEL_SOURCES[kernel]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(path: str, kernel_hash: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary (text,
    one "key: value" per line), if it was taken on the current kernel sources."""
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            key, sep, val = line.partition(":")
            if sep and not line.startswith(("#", " ", "|", "`")):
                fields[key.strip()] = val.strip()
    if fields.get("kernel_sources_hash") != kernel_hash:
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def roofline_bound(flops: float, algorithmic_bytes: float) -> str:
    """The roofline that bounds a kernel: "hbm" while its FLOPs per algorithmic byte are below the
    ridge point of the two published peaks (625 FLOP/B), else "mfma"."""
    return "hbm" if flops / algorithmic_bytes < FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"


def workload_tag(shape) -> str:
    """File-name tag of a workload, e.g. decode_T128."""
    return shape.name.split()[0] + f"_T{shape.T}"


def _oracle_layer(wl, sel, scheme: str) -> dict:
    """The oracle's whole layer on the tokens sel of the workload (the plain oracle, as it stands)."""
    import oracle
    from quantized_grouped_gemm_token_amd import workloads
    if scheme == "channel":
        s13c, s2c = workloads.channel_scales(wl)
        return oracle.moe_layer_i8(wl.x_bf16[sel], wl.logits[sel], wl.w13, s13c, wl.w2, s2c, k=wl.shape.k)
    if scheme == "mxfp4":
        w13m, s13m, w2m, s2m = workloads.mxfp4_weights(wl)
        return oracle.moe_layer_mxfp4(wl.x_bf16[sel], wl.logits[sel], w13m, s13m, w2m, s2m, k=wl.shape.k)
    return oracle.moe_layer(wl.x_bf16[sel], wl.logits[sel], wl.w13, wl.s13, wl.w2, wl.s2, k=wl.shape.k)


def cpu_baseline(wl, n_tokens: int, scheme: str = "g128") -> dict:
    """The oracle layer on the first n_tokens tokens of the workload, timed on this host: with every
    core for BLAS (the value), then with one thread."""
    from threadpoolctl import threadpool_limits
    sel = np.arange(n_tokens)
    cores = os.cpu_count() or 1
    runs = {}
    for threads in (cores, 1):
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            res = _oracle_layer(wl, sel, scheme)
            runs[threads] = time.perf_counter() - t0
    touched = int((np.diff(res["offsets"]) > 0).sum())
    sample = (f"the oracle's whole layer (numpy, fp64 sums; BLAS on {cores} threads, its per-expert "
              f"dequantization single-threaded numpy) on {n_tokens} of the {wl.shape.T} tokens of "
              f"'{wl.shape.name}', touching {touched} experts; {runs[cores]:.1f} s wall")
    return {"value": round(n_tokens / runs[cores], 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": sample,
            "single_thread": {"value": round(n_tokens / runs[1], 4), "unit": "tokens/s", "cores": 1,
                              "sample": f"the same {n_tokens} tokens with BLAS on 1 thread; {runs[1]:.1f} s wall"}}


def oracle_configs(indices, log) -> int:
    """The oracle's whole layer on every token of each listed workload, timed on this host's cores (BLAS
    on all of them; for the decode-sized workloads also on one thread): one JSON line per workload."""
    from threadpoolctl import threadpool_limits

    from quantized_grouped_gemm_token_amd import workloads
    cores = os.cpu_count() or 1
    for index in indices:
        t0 = time.perf_counter()
        wl = workloads.make_skewed_decode() if index == 5 else workloads.make_config(index)
        gen_s = time.perf_counter() - t0
        sh = wl.shape
        sel = np.arange(sh.T)
        log(f"oracle on {sh.name} (generated in {gen_s:.1f} s)")
        line = {"oracle_workload": sh.name, "tokens": sh.T, "cores": cores}
        for threads in ((cores, 1) if sh.T <= 256 and index != 5 else (cores,)):
            with threadpool_limits(limits=threads):
                t0 = time.perf_counter()
                res = _oracle_layer(wl, sel, "g128")
                sec = time.perf_counter() - t0
            key = "all_cores" if threads == cores else "one_thread"
            line[key] = {"seconds": round(sec, 2), "tokens_per_s": round(sh.T / sec, 3)}
            log(f"  {key}: {sec:.1f} s")
        line["touched_experts"] = int((np.diff(res["offsets"]) > 0).sum())
        print(json.dumps(line), flush=True)
        del wl, res
    return 0


def bench_wquant_mxfp4(args, log) -> int:
    """The MXFP4 quantizer on the gate/up weights of 16 experts (fp32 [16, 4096, 6144]): HBM-bound."""
    import torch

    from quantized_grouped_gemm_token_amd import ops

    E, N, K = 16, 4096, 6144
    gen = torch.Generator(device="cuda:0").manual_seed(1234)
    w = torch.randn((E, N, K), generator=gen, device="cuda:0", dtype=torch.float32) * 0.02
    packed = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device="cuda:0")
    for _ in range(max(args.warmup, 1)):
        ops.w4a8_moe_quantize_weights_mxfp4(w, packed, scales)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        ops.w4a8_moe_quantize_weights_mxfp4(w, packed, scales)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    in_bytes = w.numel() * 4
    moved = in_bytes + packed.numel() + scales.numel()          # 4 + 1/2 + 1/32 bytes per weight
    log(f"quantize mxfp4 {E}x{N}x{K}: {ms:.3f} ms")
    cpu = None
    if args.cpu_tokens > 0:
        from oracle import mxfp4_oracle
        try:
            from threadpoolctl import threadpool_limits
            limit = threadpool_limits(limits=1)
        except Exception:   # pragma: no cover
            limit = None
        n_rows = 1024
        sample = w[0, :n_rows].cpu().numpy()
        t0 = time.perf_counter()
        mxfp4_oracle.quantize_mxfp4(sample)
        dt = time.perf_counter() - t0
        if limit is not None:
            limit.restore_original_limits()
        cpu = {"value": round(n_rows * K * 4 / dt / 1e9, 4), "unit": "GB/s of fp32 weights", "cores": 1,
               "kind": "oracle", "sample": f"oracle MXFP4 quantizer on {n_rows} rows x {K} of the same weights; "
                                           f"{dt:.1f} s wall"}
    achieved = moved / ms / 1e6
    line = {"metric": "MXFP4 g32 weight quantizer GB/s of fp32 weights", "value": round(in_bytes / ms / 1e6, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32 in, e2m1 + e8m0 out", "data": "synthetic (seeded N(0, 0.02))",
            "config": {"workload": f"gate/up weights of {E} experts [{E}, {N}, {K}]"},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                         "note": "algorithmic bytes: 4 read + 0.5 + 1/32 written per weight"},
            "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)
    return 0


def bench_wquant(args, log) -> int:
    """The weight quantizer on the gate/up weights of 16 experts (fp32 [16, 4096, 6144])."""
    import torch

    from quantized_grouped_gemm_token_amd import ops

    E, N, K = 16, 4096, 6144
    gen = torch.Generator(device="cuda:0").manual_seed(1234)
    w = torch.randn((E, N, K), generator=gen, device="cuda:0", dtype=torch.float32) * 0.02
    packed = torch.empty((E, N, K // 8), dtype=torch.int32, device="cuda:0")
    scales = torch.empty((E, N, K // 128), dtype=torch.float32, device="cuda:0")
    for _ in range(max(args.warmup, 1)):
        ops.w4a8_moe_quantize_weights(w, True, packed, scales)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        ops.w4a8_moe_quantize_weights(w, True, packed, scales)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    in_bytes = w.numel() * 4
    moved = in_bytes + packed.numel() * 4 + scales.numel() * 4
    log(f"quantize {E}x{N}x{K}: {ms:.3f} ms")
    cpu = None
    if args.cpu_tokens > 0:
        import oracle
        try:
            from threadpoolctl import threadpool_limits
            limit = threadpool_limits(limits=1)
        except Exception:   # pragma: no cover
            limit = None
        n_rows = 256
        sample = w[0, :n_rows].cpu().numpy()
        t0 = time.perf_counter()
        oracle.quantize_int4_g128(sample)
        dt = time.perf_counter() - t0
        if limit is not None:
            limit.restore_original_limits()
        cpu = {"value": round(n_rows * K * 4 / dt / 1e9, 4), "unit": "GB/s of fp32 weights", "cores": 1,
               "kind": "oracle", "sample": f"oracle quantizer on {n_rows} rows x {K} of the same weights; "
                                           f"{dt:.1f} s wall"}
    fp64_ops = FP64_OPS_PER_WEIGHT * w.numel()
    line = {"metric": "INT4 g128 weight quantizer (11-ratio MSE clip) GB/s of fp32 weights", "value":
            round(in_bytes / ms / 1e6, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32 in, int4 + f32 scales out (fp64 decisions)", "data": "synthetic (seeded N(0, 0.02))",
            "config": {"workload": f"gate/up weights of {E} experts [{E}, {N}, {K}]"},
            "roofline": {"bound": "alu", "achieved": round(fp64_ops / ms / 1e9, 2), "peak": FP64_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(fp64_ops / ms / 1e9 / FP64_PEAK_TFLOPS, 4), "traffic": None,
                         "note": f"fp64 vector arithmetic: {FP64_OPS_PER_WEIGHT} ops per weight (11 clip ratios x "
                                 f"(residual w - q s, its square and sum)); HBM at {moved / ms / 1e6:.0f} GB/s"},
            "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload index: 1 decode T=128 (default), "
                                                          "2 decode T=256, 3 prefill T=8192, 4 skewed T=16384, "
                                                          "5 skewed decode T=256")
    ap.add_argument("--cpu-tokens", type=int, default=32, help="tokens in the CPU oracle sample (0: skip)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="with the default decode workload, skip the prefill T=8192 and skewed prefill "
                         "T=16384 blocks of the line")
    ap.add_argument("--no-skewed", action="store_true",
                    help="with the default decode workload, skip the skewed decode T=256 block of the line")
    ap.add_argument("--tokens", type=int, default=0, help="run the config's shape with this many tokens")
    ap.add_argument("--zipf", action="store_true", help="skew the routing of the config's shape by Zipf(1.1)")
    ap.add_argument("--algo", choices=("auto", "stream", "tiled"), default="auto",
                    help="grouped-GEMM kernel of both GEMMs (default: the library's automatic choice)")
    ap.add_argument("--scatter", choices=("auto", "on", "off"), default="auto",
                    help="step 7: on = routing weights applied in the down GEMM's epilogue, token-major rows, "
                         "then a contiguous combine; off = the gather combine; auto = the layer's choice")
    ap.add_argument("--oracle-configs", default="",
                    help="instead of the GPU benchmark, time the CPU oracle's whole layer on every token of "
                         "these workloads (comma-separated indices, e.g. 0,1,2,3,4,5): one JSON line each")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--scheme", choices=("g128", "channel", "mxfp4"), default="g128",
                    help="g128: INT4 group-128 x FP8 per token (default); channel: per-channel INT4 x INT8 per "
                         "token; mxfp4: MXFP4 group-32 x FP8 per token")
    ap.add_argument("--op", choices=("layer", "wquant"), default="layer",
                    help="layer: the MoE layer (default); wquant: the offline weight quantizer (INT4 group 128, "
                         "or MXFP4 with --scheme mxfp4)")
    ap.add_argument("--no-graph", action="store_true",
                    help="report the eager (kernel-by-kernel) step rate as the value instead of the graph replay")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the layer, run a plain device copy of this many bytes (5 times): the "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the layer holds all experts on one device and has no multi-GPU path)", file=sys.stderr)
        return 2

    log = (lambda *a: None) if args.quiet else (lambda *a: print("[bench]", *a, file=sys.stderr, flush=True))
    if args.oracle_configs:
        return oracle_configs([int(c) for c in args.oracle_configs.split(",")], log)

    import torch

    from quantized_grouped_gemm_token_amd import ops

    log = (lambda *a: None) if args.quiet else (lambda *a: print("[bench]", *a, file=sys.stderr, flush=True))
    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(5):
            dst.copy_(src)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / 5
        print(json.dumps({"copy_bytes_each_way": n * 4, "ms_per_copy": round(ms, 5),
                          "GBps_read_plus_write": round(2 * n * 4 / ms / 1e6, 1)}), flush=True)
        return 0
    if not ops.w4a8_moe_device_supported():
        print("bench.py: cuda:0 is not a gfx950: " + ops.last_error(), file=sys.stderr)
        return 1
    if args.op == "wquant":
        return bench_wquant_mxfp4(args, log) if args.scheme == "mxfp4" else bench_wquant(args, log)
    m = measure_layer(args.config, args, log)
    line = {
        "metric": METRIC, "value": round(m["shape"].T / (m["ms_step"] * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(m["ms_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"channel": "int8 x int4 (int32 accumulate)", "mxfp4": "fp8e4m3 x mxfp4 e2m1 (fp32 accumulate)",
                  "g128": "fp8e4m3 x int4 (fp32 accumulate)"}[args.scheme],
        "data": "synthetic (seeded; uniform 4-bit codes, lognormal scales, N(0,1) bf16 activations)",
        "config": m["config"], "roofline": m["roofline"], "cpu_baseline": None, "gemms": m["gemms"],
        "step_ms": m["step_ms"], "launch": "eager" if args.no_graph else "hip graph replay",
        "eager_ms_per_step": m["eager_ms"], "graph_ms_per_step": m["graph_ms"],
        "replay_ms_single_steps": m["replay_stats"], "device": m["device"], "kernel_sources_hash": m["roofline"]["kernel_sources_hash"],
    }
    wl = m.pop("wl")
    del m
    # the other workloads of the metric, in the same run: the prefill half (the 8K-token prompt), the
    # skewed prefill (reported against the same bar) and decode with skewed routing
    blocks = []
    if args.config == 1 and not args.no_prefill:
        blocks += [("prefill", 3), ("skewed_prefill", 4)]
    if args.config == 1 and not args.no_skewed:
        blocks += [("skewed_decode", 5)]
    for key, index in blocks:
        q = measure_layer(index, args, log)
        line[key] = {
            "workload": q["shape"].name, "tokens_per_s": round(q["shape"].T / (q["ms_step"] * 1e-3), 1),
            "ms_per_step": round(q["ms_step"], 5), "launch": line["launch"], "roofline": q["roofline"],
            "gemms": q["gemms"], "step_ms": q["step_ms"], "eager_ms_per_step": q["eager_ms"],
            "graph_ms_per_step": q["graph_ms"], "replay_ms_single_steps": q["replay_stats"]}
        del q
    if args.cpu_tokens > 0:
        n = min(args.cpu_tokens, wl.shape.T)
        log(f"CPU oracle on {n} tokens ({os.cpu_count()} BLAS threads, then 1) ...")
        line["cpu_baseline"] = cpu_baseline(wl, n, args.scheme)
    print(json.dumps(line), flush=True)
    return 0


def measure_layer(index: int, args, log) -> dict:
    """Time the layer on workload `index` (per-step kernel events, then graph replay) and price its
    gate/up GEMM against its roofline."""
    import torch

    from quantized_grouped_gemm_token_amd import ops, workloads
    from quantized_grouped_gemm_token_amd.layer import W4A8MoE, W4A8MoEChannel, W4A8MoEMxfp4

    dev = "cuda:0"
    t0 = time.time()
    if args.tokens or args.zipf:
        # the config's shape with another token count and / or Zipf(1.1)-skewed routing
        import dataclasses
        base = workloads.SKEWED_DECODE if index == 5 else workloads.WORKLOADS[index]
        T = args.tokens or base.T
        shape = dataclasses.replace(base, T=T, zipf_s=1.1 if args.zipf else base.zipf_s,
                                    name=base.name.split(" T=")[0] + f" T={T}" + base.name[base.name.index(" H="):]
                                    + (" zipf1.1" if args.zipf and base.zipf_s is None else ""))
        wl = workloads.make_workload(shape, 1000 + index)
    else:
        wl = workloads.make_skewed_decode() if index == 5 else workloads.make_config(index)
    sh = wl.shape
    log(f"generated {sh.name} in {time.time() - t0:.1f} s")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    channel = args.scheme == "channel"
    mxfp4 = args.scheme == "mxfp4"
    scatter = {"auto": None, "on": True, "off": False}[args.scatter]
    if channel:
        s13c, s2c = workloads.channel_scales(wl)
        moe = W4A8MoEChannel(to(wl.w13), to(s13c), to(wl.w2), to(s2c), k=sh.k, scatter=scatter)
    elif mxfp4:
        w13m, s13m, w2m, s2m = workloads.mxfp4_weights(wl)
        moe = W4A8MoEMxfp4(to(w13m), to(s13m), to(w2m), to(s2m), k=sh.k, scatter=scatter)
    else:
        moe = W4A8MoE(to(wl.w13), to(wl.s13), to(wl.w2), to(wl.s2), k=sh.k, scatter=scatter)
    x = torch.from_numpy(wl.x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = to(wl.logits)
    algo = {"auto": ops.W4A8_GG_AUTO, "stream": ops.W4A8_GG_STREAM, "tiled": ops.W4A8_GG_TILED}[args.algo]
    y = torch.empty((sh.T, sh.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        moe(x, logits, y, algo=algo)
    torch.cuda.synchronize()
    log(f"{sh.name}: warmup {args.warmup} done")

    steps = moe.steps
    evs = [{s: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for s in steps}
           for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        moe(x, logits, y, events=evs[i], algo=algo)
    stop.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(stop) / args.steps
    per_step = {s: float(np.mean([e[s][0].elapsed_time(e[s][1]) for e in evs])) for s in steps}
    log(f"{sh.name}: per step ms: " + ", ".join(f"{k}={v:.4f}" for k, v in per_step.items()))

    # the same step replayed from a HIP graph: W untimed replays, then exactly K timed ones
    graph = moe.capture(x, logits, y, algo=algo)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        graph.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(stop) / args.steps
    log(f"{sh.name}: step: eager {eager_ms:.4f} ms, graph replay {graph_ms:.4f} ms")
    ms_step = eager_ms if args.no_graph else graph_ms
    # the spread of single steps: K more replays, each between its own pair of events (after the timed
    # region, so that its events add nothing to it)
    rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in rev:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    one = np.array([a.elapsed_time(b) for a, b in rev])
    replay_stats = {"median": round(float(np.median(one)), 5), "p10": round(float(np.percentile(one, 10)), 5),
                    "p90": round(float(np.percentile(one, 90)), 5), "steps": int(one.size)}

    # algorithmic work of the routed experts actually touched
    offsets = moe.buffers(sh.T)["offsets"].cpu().numpy()
    counts = np.diff(offsets)
    touched = int((counts > 0).sum())
    R = sh.T * sh.k

    # packed 4-bit weights plus scales: fp32 per row (channel), fp32 per 128 (g128), one E8M0 byte per 32 (mxfp4)
    def scale_bytes(n_rows, k):
        return n_rows * (4 if channel else (k // 32 if mxfp4 else k // 128 * 4))
    w13_bytes = 2 * sh.I * sh.H // 2 + scale_bytes(2 * sh.I, sh.H)
    w2_bytes = sh.H * sh.I // 2 + scale_bytes(sh.H, sh.I)
    # the layer's gate/up GEMM has SwiGLU fused into its epilogue: it writes act [R][I] and
    # the partial row maxima [R][I/64] (fp32) instead of the [R][2I] gate/up output
    out_bytes = R * sh.I * 4 + R * (sh.I // 64) * 4 if moe.fused else R * 2 * sh.I * 4
    gate_up_bytes = (touched * w13_bytes + sh.T * sh.H + sh.T * 4 * (2 if channel else 1) + R * 4 + (sh.E + 1) * 4
                     + out_bytes)
    gate_up_flops = 2.0 * R * 2 * sh.I * sh.H
    down_flops = 2.0 * R * sh.H * sh.I
    t_gu = per_step["gemm_gate_up"] * 1e-3
    t_dn = per_step["gemm_down"] * 1e-3
    # the kernel that ran: the library's automatic choice takes the streaming one while no expert has more
    # than 20 rows and the average at most 10, else the tiled one
    decode = args.algo == "stream" or (args.algo == "auto" and R <= 10 * sh.E and int(counts.max()) <= 20)
    kernel = "gg_stream" if decode else "gg_tiled"
    khash = kernel_sources_hash(kernel)
    tag = workload_tag(sh) + ("" if args.scheme == "g128" else "_" + args.scheme)
    traffic = load_traffic(os.path.join(ROOT, "profiles", f"{kernel}_{tag}_pmc.txt"), khash)
    if roofline_bound(gate_up_flops, gate_up_bytes) == "hbm":
        achieved = gate_up_bytes / t_gu / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        achieved = gate_up_flops / t_gu / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TOP/s" if channel else "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                "traffic": traffic}
    roof["kernel"] = f"{kernel} (gate/up grouped GEMM)"
    roof["algorithmic_bytes"] = int(gate_up_bytes)
    roof["algorithmic_flops"] = gate_up_flops
    roof["avg_launch_ms"] = round(per_step["gemm_gate_up"], 5)
    roof["kernel_sources_hash"] = khash

    both_weight_bytes = touched * (w13_bytes + w2_bytes)
    gemms = {"weight_GBps": round(both_weight_bytes / (t_gu + t_dn) / 1e9, 1),
             "tflops": round((gate_up_flops + down_flops) / (t_gu + t_dn) / 1e12, 2),
             "hbm_frac_weights": round(both_weight_bytes / (t_gu + t_dn) / 1e9 / HBM_PEAK_GBS, 4),
             "mfma_frac": round((gate_up_flops + down_flops) / (t_gu + t_dn) / 1e12 / FP8_PEAK_TFLOPS, 4),
             "down_mfma_frac": round(down_flops / t_dn / 1e12 / FP8_PEAK_TFLOPS, 4),
             "down_weight_GBps": round(touched * w2_bytes / t_dn / 1e9, 1),
             "touched_experts": touched, "max_rows_per_expert": int(counts.max()),
             "empty_experts": int((counts == 0).sum())}
    config = {"workload": sh.name, "tokens": sh.T, "hidden": sh.H, "intermediate": sh.I, "experts": sh.E,
              "top_k": sh.k, "scheme": {"channel": "per-channel int4 x per-token int8",
                                        "mxfp4": "mxfp4 g32 x fp8", "g128": "int4 g128 x fp8"}[args.scheme],
              "combine": "scatter in the down GEMM + contiguous sum" if moe.uses_scatter(sh.T) else "gather"}
    device = torch.cuda.get_device_name(0)
    del graph, moe, x, logits, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return dict(wl=wl, shape=sh, ms_step=ms_step, eager_ms=round(eager_ms, 5), graph_ms=round(graph_ms, 5),
                step_ms={k: round(v, 5) for k, v in per_step.items()}, roofline=roof, gemms=gemms, config=config,
                device=device, replay_stats=replay_stats)


if __name__ == "__main__":
    sys.exit(main())
