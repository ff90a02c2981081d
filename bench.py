#!/usr/bin/env python3
"""Benchmark of the sparse MLA prefill forward on one MI355X.

One step = one call of the forward over one synthetic batch (the whole path:
top-k compaction, KV gather, both contractions, softmax, store). Inputs are
resident in HBM before the timed region. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large|wide|tp4|small|tiny|...]

The headline is the largest 128-head workload (large: T=8192, topk 1024);
every other workload is a secondary entry with its own seed, input digest,
warm and cold timings, roofline and CPU-oracle baseline.
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
    """Work the operation must do (valid slots only).

    gathered_bytes is logical: one pool row per valid slot, most of them served
    by L2 / MALL (window rows are shared by consecutive tokens). compulsory_bytes
    is what must cross HBM at least once: q, o, lse, the indices, and every
    referenced pool row once."""
    T, H, k = inp["T"], inp["H"], inp["topk_n"]
    valid = (inp["topk"] >= 0) & (inp["topk"] < inp["num_kv"])
    nvalid = int(valid.sum())
    flops = 4.0 * H * D * nvalid  # S = QK^T and O = PV, 2 flop per MAC each
    row = 512.0 if inp.get("kv_scale") is not None else 1024.0  # fp8 or bf16 pool row
    gathered = row * nvalid  # one pool row per valid slot (K == V)
    io = T * H * 1024.0 * 2 + T * H * 4.0 + T * k * 4.0  # q + o + lse + indices
    rows = np.unique(inp["topk"][valid]).size
    return {"valid_slots": nvalid, "flops": flops, "gathered_bytes": gathered, "bytes": gathered + io,
            "compulsory_bytes": io + row * rows, "referenced_rows": int(rows)}


def gpu_clock_sampler():
    """Returns a function that samples the GPU's graphics clock (MHz) and socket
    power (W) through amdsmi as a pair (either may be None), or None where amdsmi
    is not available. sample.power_cap_w holds the board's power limit."""
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None

    def num(v, hi):
        return float(v) if isinstance(v, (int, float)) and 0 < v < hi else None

    def sample():
        mhz = watts = None
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            mhz, watts = num(m.get("current_gfxclk"), 10000), num(m.get("current_socket_power"), 5000)
        except Exception:
            pass
        if mhz is None:
            try:
                mhz = num(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX).get("clk"), 10000)
            except Exception:
                pass
        return mhz, watts

    try:
        sample.power_cap_w = amdsmi.amdsmi_get_power_cap_info(h).get("power_cap") / 1e6
    except Exception:
        sample.power_cap_w = None
    return sample


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in ("sparse_attention_top_amd/csrc/smla_common.h", "sparse_attention_top_amd/csrc/smla_acc128.h",
                "sparse_attention_top_amd/csrc/sparse_mla.hip", "include/sparse_mla.h"):
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


def time_gpu(run, steps, warmup, stream, flush=None, clock=None):
    """Warm (back-to-back) timing, or cold when `flush` is given: it runs before every
    launch, outside the bracketing events. Returns wall seconds and per-launch stats (ms);
    with a clock sampler, also the graphics clock under the same workload."""
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
    st = {"mean": float(np.mean(per_launch)), "median": float(np.median(per_launch)),
          "min": float(np.min(per_launch))}
    if clock is not None:
        st["gfx_clock_mhz"] = loaded_clock(run, clock)
    return wall, st


def loaded_clock(run, clock, seconds: float = 1.5, settle: float = 0.8):
    """The graphics clock and socket power while the workload runs back to back
    (after the timed region, so the sampling costs it nothing): amdsmi's
    current_gfxclk and current_socket_power, which the SMU refreshes every few
    tens of ms, sampled after `settle` seconds (the power manager needs most of
    a second to settle at the board limit)."""
    import torch

    mhz, watts, t0 = [], [], time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        ev = torch.cuda.Event()
        for _ in range(8):
            run()
        ev.record()
        if time.perf_counter() - t0 >= settle and len(mhz) < 400:
            c, w = clock()
            if c is not None:
                mhz.append(c)
            if w is not None:
                watts.append(w)
        while not ev.query():
            time.sleep(0.001)
    torch.cuda.synchronize()
    if not mhz:
        return None
    out = {"median": float(np.median(mhz)), "min": float(np.min(mhz)), "max": float(np.max(mhz)),
           "samples": len(mhz), "source": "amdsmi current_gfxclk, workload running back to back"}
    if watts:
        out["socket_power_w"] = float(np.median(watts))
        out["board_power_cap_w"] = getattr(clock, "power_cap_w", None)
    return out


def gemm_at_power_limit(clock, n: int = 8192, seconds: float = 2.5):
    """A library bf16 GEMM (torch.matmul, n x n x n) run back to back for a few
    seconds: the dense MFMA rate a tuned vendor kernel sustains at this board's
    power limit, the practical ceiling next to the nominal peak."""
    import torch

    a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16).contiguous()
    c = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)
    torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    rates, mhz, watts, t0 = [], [], [], time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.matmul(a, b, out=c)
        e1.record()
        e1.synchronize()
        if time.perf_counter() - t0 > seconds / 2:
            rates.append(10 * 2.0 * n ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12)
            if clock is not None:
                cv, wv = clock()
                if cv is not None:
                    mhz.append(cv)
                if wv is not None:
                    watts.append(wv)
    out = {"tflops": float(np.median(rates)), "shape": "bf16 %d x %d x %d, torch.matmul" % (n, n, n),
           "seconds": seconds}
    if mhz:
        out["gfx_clock_mhz"] = float(np.median(mhz))
    if watts:
        out["socket_power_w"] = float(np.median(watts))
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


_ORACLE_THREADS = None


def cpu_baseline(inp: dict, target_s: float = 15.0, threads: int = 0):
    """The oracle, untuned, on the host cores (all of them, or `threads`) over an
    evenly spaced token sample grown toward target_s of wall time; the whole call
    when it fits. Reported in the workload's own unit (TFLOP/s for H > 16,
    gathered GB/s for H <= 16) and as ms per call extrapolated to every token."""
    import oracle

    global _ORACLE_THREADS
    if _ORACLE_THREADS is None:
        _ORACLE_THREADS = oracle.threads()  # before any single-thread run changes the default
    nthr = threads if threads > 0 else _ORACLE_THREADS
    T = inp["T"]

    def run(tokens):
        t0 = time.perf_counter()
        oracle.forward(inp["q"], inp["kv"], inp["topk"], inp["sink"], inp["scale"], tokens=tokens,
                       want_exact=False, want_bf16=True, kv_scale=inp.get("kv_scale"), threads=nthr)
        return time.perf_counter() - t0

    n = max(1, min(T, 32 if nthr == 1 else 128))
    tokens = np.linspace(0, T - 1, n).round().astype(np.int64)
    dt = run(tokens)
    if dt < target_s / 4 and n < T:  # grow the sample toward the target wall time
        n = int(min(T, n * max(1.0, target_s / max(dt, 1e-3))))
        tokens = np.linspace(0, T - 1, n).round().astype(np.int64)
        dt = run(tokens)
    valid = (inp["topk"][tokens] >= 0) & (inp["topk"][tokens] < inp["num_kv"])
    nv = int(valid.sum())
    row = 512.0 if inp.get("kv_scale") is not None else 1024.0
    if inp["H"] > 16:
        value, unit = 4.0 * inp["H"] * D * nv / dt / 1e12, "TFLOP/s"
    else:
        value, unit = row * nv / dt / 1e9, "GB/s"
    return {"value": value, "unit": unit, "cores": nthr, "kind": "oracle",
            "sample": "%d of %d tokens (evenly spaced), %d valid slots, %.2f s wall" % (len(tokens), T, nv, dt),
            "ms_per_call_extrapolated": dt * 1e3 * T / len(tokens), "cpu_model": cpu_model()}


def measure(name: str, steps: int, warmup: int, cold_steps: int = 0, idx64: bool = False, clock=None):
    import torch

    from sparse_attention_top_amd import fp8_pool_decoded, kernel_name, sparse_mla_prefill, synth

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

    wall, st = time_gpu(run, steps, warmup, stream, clock=clock)
    alg = algorithmic(inp)
    # an fp8 pool is either read by the fp8 kernels or decoded once per call into a bf16 copy for the bf16 ones
    decoded = kv_scale is not None and fp8_pool_decoded(inp["T"], inp["topk_n"], inp["num_kv"])
    H, fp8 = inp["H"], kv_scale is not None and not decoded
    t = {"wall_s": wall, "ms_per_call": wall * 1e3 / steps, "kernel_ms_mean": st["mean"],
         "kernel_ms_median": st["median"], "kernel_ms_min": st["min"], "kernel": kernel_name(H, inp["topk_n"], fp8)}
    if decoded:
        t["pool_decode"] = "smla_fp8_pool_decode_kernel (the pool to bf16 code values, each call, inside the events)"
    if "gfx_clock_mhz" in st:
        t["gfx_clock_mhz"] = st["gfx_clock_mhz"]
    # few (token, head group) units: the library splits each top-k row and merges (the split path's kernels)
    nw = 1 if H <= 16 else 2 if H <= 32 else (8 if fp8 and H > 64 else 4)
    units = inp["T"] * -(-H // (16 * nw))  # as the library counts them to choose the split path
    if units < torch.cuda.get_device_properties(dev).multi_processor_count and inp["topk_n"] >= 128:
        t["kernel"] = "smla_fwd%s_split_kernel<%d, %d> + smla_merge_kernel" % ("_fp8" if fp8 else "", nw,
                                                                              4 if fp8 and nw >= 4 else 2)
    elif idx64 and H <= 16 and not fp8:  # the 16-row kernel reads int64 rows itself
        t["kernel"] = t["kernel"].replace("smla_fwd16_kernel<1, ", "smla_fwd16_i64_kernel<")
        t["idx64_native"] = True
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
    """The dominant kernel against its bound. MFMA-bound (H > 16): valid-slot flops
    over the bf16 dense peak. Otherwise HBM: the compulsory bytes (q, o, lse,
    indices, each referenced pool row once) over the HBM peak; the logical
    gathered bytes, mostly L2/MALL hits, are reported apart as gathered_gbs."""
    if bound == "mfma":
        achieved = alg["flops"] / (t["kernel_ms_mean"] * 1e-3) / 1e12
        peak, unit, what = PEAK_BF16_TFLOPS, "TFLOP/s", "4 H 512 flop per valid slot"
    else:
        achieved = alg["compulsory_bytes"] / (t["kernel_ms_mean"] * 1e-3) / 1e9
        peak, unit, what = PEAK_HBM_GBS, "GB/s", "compulsory HBM bytes: q + o + lse + indices + referenced rows once"
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": traffic_from_profiles(kernel, workload), "kernel": kernel, "work": what}


def entry(name: str, steps: int, warmup: int, cold_steps: int, clock, cpu: bool, idx64: bool = False) -> dict:
    """One workload: warm and cold timings, roofline, seed and input digest, CPU baseline."""
    from sparse_attention_top_amd import synth

    inp, alg, t = measure(name, steps, warmup, cold_steps=cold_steps, idx64=idx64, clock=clock)
    cfg = inp["config"]
    bound = "mfma" if inp["H"] > 16 else "hbm"
    e = {"workload": name + (":int64" if idx64 else ""), "T": cfg.T, "H": cfg.H, "topk": cfg.topk,
         "num_kv": cfg.num_kv, "seed": cfg.seed, "inputs_sha256": synth.fingerprint(inp)[:16],
         "valid_slots": alg["valid_slots"], "steps": steps, "ms_per_call": t["ms_per_call"],
         "kernel_ms_mean": t["kernel_ms_mean"], "kernel_ms_median": t["kernel_ms_median"],
         "kernel_ms_min": t["kernel_ms_min"], "kernel": t["kernel"],
         "tflops": alg["flops"] / (t["kernel_ms_mean"] * 1e-3) / 1e12,
         "gathered_gbs": alg["gathered_bytes"] / (t["kernel_ms_mean"] * 1e-3) / 1e9,
         "compulsory_gbs": alg["compulsory_bytes"] / (t["kernel_ms_mean"] * 1e-3) / 1e9,
         "cold": t.get("cold"), "gfx_clock_mhz": t.get("gfx_clock_mhz"),
         "roofline": roofline(alg, t, t["kernel"], name, bound)}
    if inp.get("kv_scale") is not None:
        e["pool"] = "fp8 e4m3 codes, per-tensor scale"
        if t.get("pool_decode"):
            e["pool_decode"] = t["pool_decode"]
    if idx64:
        e["note"] = ("int64 top-k rows, read by the 16-row kernel itself" if t.get("idx64_native") else
                     "int64 top-k rows: index conversion kernel + the int32 path")
    if "split" in t["kernel"]:
        e["note"] = ("few-token call: split-KV kernel + merge kernel; per-launch events include the "
                     "host launch gap, rocprofv3 kernel time is the GPU figure")
    if cpu and not idx64:
        e["cpu_baseline"] = cpu_baseline(inp, target_s=2.0)
        if name in ("tiny", "small"):
            e["cpu_baseline_1thread"] = cpu_baseline(inp, target_s=2.0, threads=1)
    return inp, alg, t, e


# Secondary workloads: every other configuration of the benchmark, timed warm
# (>= 50 launches, >= 200 for the sub-0.1 ms ones) and cold (each launch after
# a 512 MiB overwrite), each with its own CPU-oracle baseline.
SECONDARY = ("wide", "tp4", "small", "tiny", "glm", "decode", "tp4:int64", "tp4_fp8", "glm_fp8", "wide_fp8",
             "wide_k1024")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large", choices=["tiny", "small", "tp4", "wide", "large", "glm", "decode",
                                                           "tp4_fp8", "wide_fp8", "glm_fp8", "wide_k1024", "long"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timings")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock sampling window (keeps the launch count fixed for profiling)")
    ap.add_argument("--bwd", action="store_true",
                    help="only time the backward on --workload and print its line (for profiling)")
    ap.add_argument("--fp8-pool-decode", default="auto", choices=["never", "auto", "always"],
                    help="how fp8 pools are read: by the fp8 kernels (never), decoded once per call into a bf16 "
                         "copy for the bf16 kernels (always), or as the library chooses (auto, the default)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.fp8_pool_decode != "auto":
        from sparse_attention_top_amd import set_fp8_pool_decode

        set_fp8_pool_decode(args.fp8_pool_decode)

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

    if args.bwd:
        print("bench: backward on %s, %d warmup + %d timed steps" % (args.workload, args.warmup, args.steps),
              file=sys.stderr, flush=True)
        print(json.dumps(measure_bwd(args.workload, args.steps, args.warmup)))
        return

    clock = None if args.no_clock else gpu_clock_sampler()
    print("bench: workload %s, %d warmup + %d timed steps" % (args.workload, args.warmup, args.steps),
          file=sys.stderr, flush=True)
    inp, alg, t = measure(args.workload, args.steps, args.warmup, cold_steps=0 if args.no_cold else min(args.steps, 20),
                          clock=clock)
    bound = "mfma" if inp["H"] > 16 else "hbm"
    tflops = alg["flops"] / (t["ms_per_call"] * 1e-3) / 1e12
    gbs = alg["gathered_bytes"] / (t["ms_per_call"] * 1e-3) / 1e9
    metric = "sparse MLA prefill fwd TFLOPS (H=128) & gathered-KV GB/s (H=16), ms/call"
    value, unit = (tflops, "TFLOP/s") if bound == "mfma" else (gbs, "GB/s")
    cfg = inp["config"]
    from sparse_attention_top_amd import synth

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
        "gfx_clock_mhz": t.get("gfx_clock_mhz"),
        "roofline": roofline(alg, t, t["kernel"], cfg.name, bound),
    }
    if t.get("pool_decode"):
        line["pool_decode"] = t["pool_decode"]
    print("bench: %s %.4f ms/call, %.1f TFLOP/s, %.1f GB/s gathered" % (cfg.name, t["ms_per_call"], tflops, gbs),
          file=sys.stderr, flush=True)
    if clock is not None and bound == "mfma":
        g = gemm_at_power_limit(clock)
        line["gemm_at_power_limit"] = g
        line["roofline"]["frac_of_power_limited_gemm"] = line["roofline"]["achieved"] / g["tflops"]
        print("bench: library bf16 GEMM at the power limit %.0f TFLOP/s" % g["tflops"], file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inp)
    if not args.no_secondary:
        sec = []
        for other in SECONDARY:
            name2, _, kind = other.partition(":")
            if name2 == args.workload and not kind:
                continue
            small = name2 in ("tiny", "small", "decode")
            steps2 = max(200 if small else 50, args.steps)
            _, _, _, e = entry(name2, steps2, args.warmup, 0 if args.no_cold else 10, clock,
                               cpu=not args.no_cpu_baseline, idx64=kind == "int64")
            sec.append(e)
            print("bench: %s %.4f ms/call" % (other, e["kernel_ms_mean"]), file=sys.stderr, flush=True)
        for name in ("wide", "wide_k1024", "long", "tp4"):
            b = measure_bwd(name, max(10, args.steps // 2), args.warmup)
            sec.append(b)
            print("bench: bwd:%s %.4f ms/call, %.1f TFLOPS (page formula)" % (name, b["kernel_ms_mean"],
                                                                             b["tflops_pages_formula"]),
                  file=sys.stderr, flush=True)
        line["secondary"] = sec
    print(json.dumps(line))


if __name__ == "__main__":
    main()
