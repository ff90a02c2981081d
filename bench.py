#!/usr/bin/env python3
"""Benchmark of the sparse MLA prefill forward on one MI355X.

One step = one call of the forward over one synthetic batch (the whole path:
top-k compaction, KV gather, both contractions, softmax, store). Inputs are
resident in HBM before the timed region. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wide|large|tp4|small|tiny]
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

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
D = 512


def algorithmic(inp: dict) -> dict:
    """Work the operation must do (valid slots only)."""
    T, H, k = inp["T"], inp["H"], inp["topk_n"]
    nvalid = int(((inp["topk"] >= 0) & (inp["topk"] < inp["num_kv"])).sum())
    flops = 4.0 * H * D * nvalid  # S = QK^T and O = PV, 2 flop per MAC each
    row = 512.0 if inp.get("kv_scale") is not None else 1024.0  # fp8 or bf16 pool row
    gathered = row * nvalid  # one pool row per valid slot (K == V)
    io = T * H * 1024.0 * 2 + T * H * 4.0 + T * k * 4.0  # q + o + lse + indices
    return {"valid_slots": nvalid, "flops": flops, "gathered_bytes": gathered, "bytes": gathered + io}


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in ("sparse_attention_top_amd/csrc/smla_common.h", "sparse_attention_top_amd/csrc/sparse_mla.hip",
                "include/sparse_mla.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE, scaled
    by the copy-kernel calibration), if recorded for the current kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    digest = source_digest()
    for line in open(path):
        m = re.match(r"\|\s*%s\s*\|\s*([0-9a-f]+)\s*\|\s*([0-9.eE+]+)\s*\|" % re.escape(workload), line)
        if m and m.group(1) == digest:
            return float(m.group(2))
    return None


def time_gpu(run, steps, warmup, stream, flush=None):
    """Warm (back-to-back) timing, or cold when `flush` is given: it runs before every
    launch, outside the bracketing events. Returns wall seconds and per-launch stats (ms)."""
    import torch

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush()
        starts[i].record(stream)
        run()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, {"mean": float(np.mean(per_launch)), "median": float(np.median(per_launch)),
                  "min": float(np.min(per_launch))}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp: dict, target_s: float = 15.0):
    """The oracle, untuned, on the host cores over an evenly spaced token sample."""
    import oracle

    T = inp["T"]
    n = max(1, min(T, 128))
    tokens = np.linspace(0, T - 1, n).round().astype(np.int64)
    t0 = time.perf_counter()
    oracle.forward(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"], tokens=tokens,
                   want_exact=False, want_bf16=True, kv_scale=inp.get("kv_scale"))
    dt = time.perf_counter() - t0
    if dt < target_s / 4 and n < T:  # grow the sample toward the target wall time
        n = int(min(T, n * max(1.0, target_s / max(dt, 1e-3))))
        tokens = np.linspace(0, T - 1, n).round().astype(np.int64)
        t0 = time.perf_counter()
        oracle.forward(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"], tokens=tokens,
                       want_exact=False, want_bf16=True, kv_scale=inp.get("kv_scale"))
        dt = time.perf_counter() - t0
    nv = int(((inp["topk"][tokens] >= 0) & (inp["topk"][tokens] < inp["num_kv"])).sum())
    flops = 4.0 * inp["H"] * D * nv
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "%d of %d tokens (evenly spaced), %d valid slots, %.2f s wall" % (len(tokens), T, nv, dt),
            "ms_per_call_extrapolated": dt * 1e3 * inp["T"] / len(tokens), "cpu_model": cpu_model()}


def measure(name: str, steps: int, warmup: int, cold_steps: int = 0, idx64: bool = False):
    import torch

    from sparse_attention_top_amd import kernel_name, sparse_mla_prefill, synth

    inp = synth.make_inputs(name)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp["q"].view(np.int16)).view(torch.bfloat16).to(dev)
    kv_scale = inp.get("kv_scale")
    if kv_scale is not None:  # OCP FP8 E4M3 codes
        kv = torch.from_numpy(inp["kv"]).to(dev).view(torch.float8_e4m3fn)
    else:
        kv = torch.from_numpy(inp["kv"].view(np.int16)).view(torch.bfloat16).to(dev)
    topk = torch.from_numpy(inp["topk"].astype(np.int64) if idx64 else inp["topk"]).to(dev)
    sink = torch.from_numpy(inp["sink"]).to(dev) if inp["sink"] is not None else None
    out = torch.empty_like(q)
    lse = torch.empty((inp["T"], inp["H"]), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run():
        sparse_mla_prefill(q, kv, topk, sink, inp["scale"], out=out, lse=lse, kv_scale=kv_scale)

    wall, st = time_gpu(run, steps, warmup, stream)
    alg = algorithmic(inp)
    t = {"wall_s": wall, "ms_per_call": wall * 1e3 / steps, "kernel_ms_mean": st["mean"],
         "kernel_ms_median": st["median"], "kernel_ms_min": st["min"],
         "kernel": kernel_name(inp["H"], inp["topk_n"], kv_scale is not None)}
    # few (token, head group) units: the library splits each top-k row and merges (the split path's kernels)
    H, fp8 = inp["H"], kv_scale is not None
    nw = 1 if H <= 16 else 2 if H <= 32 else (8 if fp8 and H > 64 else 4)
    units = inp["T"] * -(-H // (16 * nw))
    if units < torch.cuda.get_device_properties(dev).multi_processor_count and inp["topk_n"] >= 128:
        t["kernel"] = "smla_fwd%s_split_kernel<%d, %d> + smla_merge_kernel" % ("_fp8" if fp8 else "", nw,
                                                                              4 if fp8 and nw >= 4 else 2)
    if cold_steps:
        # cold caches: overwrite 512 MiB (more than the 256 MB MALL plus 8 x 4 MB of L2) before each launch
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        _, cst = time_gpu(run, cold_steps, 1, stream, flush=lambda: scratch.fill_(1))
        t["cold"] = {"kernel_ms_mean": cst["mean"], "kernel_ms_median": cst["median"], "kernel_ms_min": cst["min"],
                     "launches": cold_steps, "flush_bytes": 512 << 20}
        del scratch
    return inp, alg, t


def measure_bwd(name: str, steps: int, warmup: int):
    """The backward on a workload: dO ~ N(0, 1) from a seeded device generator,
    o and lse from one forward call, then `steps` timed backward calls."""
    import torch

    from sparse_attention_top_amd import sparse_mla_backward, sparse_mla_prefill, synth

    inp = synth.make_inputs(name)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp["q"].view(np.int16)).view(torch.bfloat16).to(dev)
    kv = torch.from_numpy(inp["kv"].view(np.int16)).view(torch.bfloat16).to(dev)
    topk = torch.from_numpy(inp["topk"]).to(dev)
    sink = torch.from_numpy(inp["sink"]).to(dev) if inp["sink"] is not None else None
    gen = torch.Generator(device=dev)
    gen.manual_seed(inp["config"].seed + 1000)
    dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    o, lse = sparse_mla_prefill(q, kv, topk, sink, inp["scale"])
    stream = torch.cuda.current_stream(dev)

    def run():
        sparse_mla_backward(q, kv, dout, o, lse, topk, sink, inp["scale"])

    wall, st = time_gpu(run, steps, warmup, stream)
    nvalid = int(((inp["topk"] >= 0) & (inp["topk"] < inp["num_kv"])).sum())
    ms = st["mean"]
    flops_valid = 10.0 * inp["H"] * D * nvalid  # S, dP, dQ and the two dkv terms per valid (slot, head)
    flops_pages = 10.0 * inp["T"] * inp["H"] * inp["topk_n"] * D  # the backward page's TFLOPS convention
    return {"workload": "bwd:" + name, "ms_per_call": wall * 1e3 / steps, "kernel_ms_mean": ms,
            "kernel_ms_median": st["median"], "kernel_ms_min": st["min"],
            "tflops_pages_formula": flops_pages / (ms * 1e-3) / 1e12,
            "tflops_valid": flops_valid / (ms * 1e-3) / 1e12, "valid_slots": nvalid,
            "roofline": {"bound": "mfma", "achieved": flops_valid / (ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops_valid / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "traffic": None, "kernel": "backward (five phases)"},
            "note": "per-call time of the whole backward (dq, dkv, d_sink: five kernels and the sort); "
                    "TFLOPS as the backward page counts them, 10 T H topk 512 / t, and on valid slots"}


def roofline(alg, t, kernel, workload, bound):
    if bound == "mfma":
        achieved = alg["flops"] / (t["kernel_ms_mean"] * 1e-3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = alg["bytes"] / (t["kernel_ms_mean"] * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": traffic_from_profiles(kernel, workload), "kernel": kernel}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wide", choices=["tiny", "small", "tp4", "wide", "large", "glm", "decode",
                                                          "tp4_fp8", "wide_fp8", "glm_fp8", "wide_k1024", "long"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timing of the main workload")
    ap.add_argument("--bwd", action="store_true",
                    help="only time the backward on --workload and print its line (for profiling)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": max(1, args.steps)}))
        return

    from sparse_attention_top_amd import synth

    if args.bwd:
        print("bench: backward on %s, %d warmup + %d timed steps" % (args.workload, args.warmup, args.steps),
              file=sys.stderr, flush=True)
        print(json.dumps(measure_bwd(args.workload, args.steps, args.warmup)))
        return

    print("bench: workload %s, %d warmup + %d timed steps" % (args.workload, args.warmup, args.steps),
          file=sys.stderr, flush=True)
    inp, alg, t = measure(args.workload, args.steps, args.warmup, cold_steps=0 if args.no_cold else min(args.steps, 20))
    bound = "mfma" if inp["H"] > 16 else "hbm"
    tflops = alg["flops"] / (t["ms_per_call"] * 1e-3) / 1e12
    gbs = alg["gathered_bytes"] / (t["ms_per_call"] * 1e-3) / 1e9
    if bound == "mfma":
        metric, value, unit = "sparse MLA prefill fwd TFLOPS (valid slots, H=%d)" % inp["H"], tflops, "TFLOP/s"
    else:
        metric, value, unit = "sparse MLA prefill fwd gathered-KV GB/s (H=%d)" % inp["H"], gbs, "GB/s"
    cfg = inp["config"]
    if inp.get("kv_scale") is not None:
        metric = metric + " [fp8 pool]"
    line = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "topk": cfg.topk, "num_kv": cfg.num_kv,
                   "head_dim": D, "valid_slots": alg["valid_slots"], "seed": cfg.seed,
                   "inputs_sha256": synth.fingerprint(inp)[:16], "parallelism": "none"},
        "tflops": tflops,
        "gathered_gbs": gbs,
        "kernel_ms_mean": t["kernel_ms_mean"],
        "kernel_ms_median": t["kernel_ms_median"],
        "kernel_ms_min": t["kernel_ms_min"],
        "cold": t.get("cold"),
        "roofline": roofline(alg, t, t["kernel"], cfg.name, bound),
    }
    print("bench: %s %.4f ms/call, %.1f TFLOP/s, %.1f GB/s gathered" % (cfg.name, t["ms_per_call"], tflops, gbs),
          file=sys.stderr, flush=True)
    if not args.no_secondary:
        sec = []
        for other in ("tp4", "large", "small", "glm", "decode", "tp4:int64", "tp4_fp8", "glm_fp8", "wide_fp8"):
            if other == args.workload:
                continue
            name2, _, kind = other.partition(":")
            i2, a2, t2 = measure(name2, max(10, args.steps // 2), args.warmup, idx64=kind == "int64")
            b2 = "mfma" if i2["H"] > 16 else "hbm"
            sec.append({"workload": other, "ms_per_call": t2["ms_per_call"], "kernel_ms_mean": t2["kernel_ms_mean"],
                        "kernel_ms_median": t2["kernel_ms_median"], "kernel_ms_min": t2["kernel_ms_min"],
                        "tflops": a2["flops"] / (t2["ms_per_call"] * 1e-3) / 1e12,
                        "gathered_gbs": a2["gathered_bytes"] / (t2["ms_per_call"] * 1e-3) / 1e9,
                        "valid_slots": a2["valid_slots"],
                        "roofline": roofline(a2, t2, t2["kernel"], other, b2)})
            if kind == "int64":
                sec[-1]["note"] = "int64 top-k rows: index conversion kernel + the int32 path"
            if i2["T"] * -(-i2["H"] // 128) < 256:
                sec[-1]["note"] = ("few-token call: split-KV kernel + merge kernel; per-launch events include the "
                                   "host launch gap, rocprofv3 kernel time is the GPU figure")
            print("bench: %s %.4f ms/call" % (other, t2["ms_per_call"]), file=sys.stderr, flush=True)
        for name in ("wide", "wide_k1024", "long", "tp4"):
            b = measure_bwd(name, max(10, args.steps // 2), args.warmup)
            sec.append(b)
            print("bench: bwd:%s %.4f ms/call, %.1f TFLOPS (page formula)" % (name, b["kernel_ms_mean"],
                                                                             b["tflops_pages_formula"]),
                  file=sys.stderr, flush=True)
        line["secondary"] = sec
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
