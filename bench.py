"""Benchmark: batched Gram Newton–Schulz on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --calibrate-copy ...          (under rocprofv3 --pmc)
    python bench.py --ingest-pmc FETCH.csv WRITE.csv [--workload NAME]

One step = one ns_orthogonalize call over the whole bucket (normalize, every
GEMM of Algorithm 3 or 1, output), inputs resident in HBM.  Prints one JSON
line: matrices/s (whole job), effective TFLOP/s from the pages' FLOP formula
and its fraction of the fp16 dense MFMA peak, a roofline object for the
dominant kernel (per-launch durations from HIP events recorded by the library
on the stream its kernels run on, over K more calls timed right after the K
throughput calls, which carry no per-launch events), the fp64 CPU oracle
timed on a bounded
sample of the same workload, a parity object comparing the GPU output with
those oracle outputs, and (default workload only) the same figures for the
other four buckets under "other_configs", each against the roofline that
bounds it (MFMA for the 4096-wide buckets, HBM for the GPT-2-small and MoE
buckets, whose algorithmic intensity is below the ridge point).
Progress lines go to stderr; stdout carries the one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "matrices/s and effective TFLOP/s (% fp16 MFMA peak), Gram NS, 7B bucket"
# metric label and the roofline that bounds each bucket (the HBM-bound ones
# sit below the ridge point, 2516.6 TFLOP/s / 8 TB/s = 315 FLOP/B)
WORKLOAD_INFO = {
    "llama7b_mlp_32x11008x4096_bf16": (METRIC, "mfma"),
    "square_32x4096x4096_f16": ("matrices/s and effective TFLOP/s (% fp16 MFMA peak), standard NS "
                                "(square fallback), 32x4096x4096 fp16 bucket", "mfma"),
    "gpt2s_mlp_42x768x3072_f16": ("matrices/s and effective TFLOP/s (% of HBM roofline), Gram NS, "
                                  "GPT-2-small MLP bucket 42x768x3072 fp16", "hbm"),
    "moe_512x2048x512_f16": ("matrices/s and effective TFLOP/s (% of HBM roofline), Gram NS, "
                             "MoE expert bucket 512x2048x512 fp16", "hbm"),
    "single_1x128x512_f32": ("calls/s, Gram NS, single fp32 128x512 matrix (launch-latency bound)", "latency"),
}
OTHER_CONFIGS = ("gpt2s_mlp_42x768x3072_f16", "square_32x4096x4096_f16", "moe_512x2048x512_f16",
                 "single_1x128x512_f32")
# matrices of each bucket the parity sample compares with the oracle (a
# bounded set: the oracle is fp64 numpy on the host)
PARITY_SAMPLE = {"gpt2s_mlp_42x768x3072_f16": list(range(0, 42, 3)), "square_32x4096x4096_f16": [0],
                 "moe_512x2048x512_f16": list(range(0, 512, 32)), "single_1x128x512_f32": [0]}
PEAK_FP16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk/CU x 2.4 GHz (dense)
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "llama7b_mlp_32x11008x4096_bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """Hash of the kernels and the launch plan with comments and blank space
    removed, so that only a change of the code voids stored counter data."""
    import re

    h = hashlib.sha256()
    for f in ("nsg_kernels.hip", "nsg_internal.h", "nsg_api.cpp"):  # kernels and the launch plan
        with open(os.path.join(ROOT, "newton_schulz_gram_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_flops(entry, G):
    """Pages' count for one launch over the bucket: 2 M N K for a general
    product, M N K for a symmetric one (half the product is computed)."""
    if entry["kernel"] == "gemm_nt":
        return 2.0 * entry["M"] * entry["N"] * entry["K"] * G
    if entry["kernel"] == "gemm_nt_sym":
        return 1.0 * entry["M"] * entry["N"] * entry["K"] * G
    return 0.0


# Device kernel symbol -> the library's launch kind (the timing label).
def kernel_kind(symbol: str):
    if "copy_kernel" in symbol:
        return "copy"
    if "gemm256" in symbol or "gemm_nt_kernel" in symbol:
        # the symmetric flag: second template argument of gemm256h_kernel<DT, SYM, CIN> and
        # gemm256_kernel<DT, SYM, NW>, last of gemm_nt_kernel<DT, BM, BN, WGM, WGN, SYM>
        targs = [t.strip() for t in symbol[symbol.index("<") + 1:symbol.index(">")].split(",")]
        sym = targs[-1] if "gemm_nt_kernel" in symbol else targs[1]
        return "gemm_nt_sym" if sym in ("true", "1") else "gemm_nt"
    if "norm_reduce_kernel" in symbol:
        return "norm_reduce"
    if "scale_cast_transpose" in symbol:
        return "scale_cast_transpose"
    return None


COPY_BYTES = 1 << 30   # the calibration copy: 1 GiB read, 1 GiB written


def read_counter_csv(path, counter):
    """{kind: [value per dispatch]} for one counter of a rocprofv3 --pmc run."""
    import csv

    out = {}
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            k = kernel_kind(row["Kernel_Name"])
            if k is not None:
                out.setdefault(k, []).append(float(row["Counter_Value"]))
    return out


def ingest_pmc(fetch_csv, write_csv, workload):
    """HBM bytes per launch of each GEMM kind from FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch), each scaled so that the calibration copy of COPY_BYTES reads
    and writes exactly COPY_BYTES; stored with the kernel-source hash so that a
    later change of the kernels voids it."""
    fetch = read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = read_counter_csv(write_csv, "WRITE_SIZE")
    f_scale = COPY_BYTES / (1024.0 * sum(fetch["copy"]) / len(fetch["copy"]))
    w_scale = COPY_BYTES / (1024.0 * sum(write["copy"]) / len(write["copy"]))
    ent = {}
    for k in ("gemm_nt", "gemm_nt_sym", "norm_reduce", "scale_cast_transpose"):
        if k not in fetch or k not in write:
            continue
        rd = 1024.0 * f_scale * sum(fetch[k]) / len(fetch[k])
        wr = 1024.0 * w_scale * sum(write[k]) / len(write[k])
        ent[k] = {"bytes_per_launch": rd + wr, "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
                  "dispatches": len(fetch[k]), "kernel_src": kernel_source_hash()}
    tr = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    tr[workload] = dict(ent, calibration={"copy_bytes": COPY_BYTES, "fetch_scale": f_scale,
                                          "write_scale": w_scale})
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(tr, fh, indent=1, sort_keys=True)
    print(json.dumps(tr[workload]))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def host_info():
    threads, blas = None, None
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"] or threadpool_info()
        threads = max((d.get("num_threads") or 0) for d in info) or None
        blas = ", ".join(sorted({f"{d.get('internal_api')} {d.get('version') or ''}".strip() for d in info}))
    except Exception:
        pass
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:
        pass
    return threads, blas, cpu_model


def oracle_outputs(w, x_cpu, idx):
    """The oracle on matrices idx of the bucket (fp64 numpy, as it stands)."""
    import oracle

    return oracle.orthogonalize(x_cpu[idx].double().numpy(), w.steps, w.coeffs, w.mode, w.restart_after,
                                w.safety)


def cpu_baseline(w, x_cpu, budget_s: float = 30.0):
    """The oracle as it stands, on a bounded sample: whole matrices of the bucket,
    stopping once half the time budget is spent (at least one matrix).
    Returns (baseline object, sample indices, oracle outputs)."""
    import numpy as np

    threads, blas, cpu_model = host_info()
    outs, done, t0 = [], 0, time.perf_counter()
    while done < w.G:
        outs.append(oracle_outputs(w, x_cpu, [done])[0])
        done += 1
        if time.perf_counter() - t0 > budget_s / 2:
            break
    dt = time.perf_counter() - t0
    base = {"value": done / dt, "unit": "matrices/s", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": f"{done} of {w.G} matrices ({w.R}x{w.C}), full NS in fp64 numpy, {dt:.1f} s",
            "seconds_per_matrix": dt / done, "blas": blas, "cpu_model": cpu_model,
            "host_cpu_count": os.cpu_count()}
    return base, list(range(done)), np.stack(outs)


def parity_object(out_gpu, idx, ref, classes=None):
    """GPU output of matrices idx against the oracle's: worst relative
    Frobenius error, cosine, 256 x 256 block error and element error (the
    measures of the GPU parity tests), plus whether the pages' bars hold;
    with `classes` (matrix index -> conditioning class) also the worst
    relative error per class."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity_metrics import bucket_errors, summary

    o = out_gpu[idx].float().cpu()
    errs = bucket_errors(o, ref)
    sm = summary(errs)
    res = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in sm.items()}
    res["matrices"] = idx if len(idx) <= 8 else f"{len(idx)} of the bucket: {idx[0]}..{idx[-1]}"
    res["within_bars"] = bool(sm["rel_max"] <= 3e-2 and sm["cos_min"] >= 0.97)
    if classes is not None:
        per = {}
        for g, e in zip(idx, errs):
            c = classes(g)
            per[c] = round(max(per.get(c, 0.0), e["rel"]), 6)
        res["rel_max_per_class"] = per
    return res


def bench_select(args, w, dev):
    """Selection front-end + Gram NS on the selected lines (Dion3 paper,
    Algorithm 4, steps 3-4); effective FLOPs from the k x m problem."""
    import torch

    import newton_schulz_gram_amd as nsg
    import synth

    torch.cuda.set_device(dev)
    x = synth.make(w).to(dev)
    G, R, C = x.shape
    dim, k = nsg.select_plan(R, C, args.select_fraction)
    kw = dict(steps=w.steps, coeffs=w.coeffs, mode=w.mode, restart_after=w.restart_after, safety=w.safety,
              compute_dtype=w.compute, sym_updates=not args.general_updates)
    out = torch.empty_like(x)
    for _ in range(args.warmup):
        nsg.orthogonalize_selected(x, args.select_fraction, dim=dim, out=out, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        nsg.orthogonalize_selected(x, args.select_fraction, dim=dim, out=out, **kw)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sub = (k, R) if dim == 1 else (k, C)   # the submatrix, short side first
    credited, _ = nsg.flops(sub[0], sub[1], **kw) if sub[0] <= sub[1] else nsg.flops(sub[1], sub[0], **kw)
    # the front-end alone: norms + top-k, timed on their own
    for _ in range(2):
        keys = nsg.l1_norms(x, dim)
        nsg.topk(keys, k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        keys = nsg.l1_norms(x, dim)
    torch.cuda.synchronize()
    t_norm = (time.perf_counter() - t1) / args.steps
    t1 = time.perf_counter()
    for _ in range(args.steps):
        nsg.topk(keys, k)
    torch.cuda.synchronize()
    t_topk = (time.perf_counter() - t1) / args.steps
    in_bytes = x.numel() * x.element_size()
    res = {
        "metric": f"matrices/s, Dion3 selection (f={args.select_fraction}) + Gram NS",
        "value": round(G * args.steps / wall, 3), "unit": "matrices/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(1e3 * wall / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16" if w.compute == "f16" else w.compute,
        "data": "synthetic",
        "config": {"workload": w.name, "G": G, "R": R, "C": C, "select_dim": "columns" if dim else "rows",
                   "fraction": args.select_fraction, "k": k, "submatrix": [int(v) for v in sub]},
        "effective_tflops": round(credited * G * args.steps / wall / 1e12, 2),
        "l1_norms": {"ms": round(1e3 * t_norm, 3), "gbs": round(in_bytes / t_norm / 1e9, 1)},
        "topk_ms": round(1e3 * t_topk, 3),
    }
    print(json.dumps(res), flush=True)


def bench_muon(args, w, dev):
    """One Muon step per timed step (Dion3 paper, Eq. (1) with decoupled weight
    decay; bf16 W written back with stochastic rounding, fp32 momentum)."""
    import torch

    import newton_schulz_gram_amd as nsg
    import synth

    torch.cuda.set_device(dev)
    grad = synth.make(w).to(dev)
    G, R, C = grad.shape
    W = torch.randn(G, R, C, device=dev).to(torch.bfloat16)
    M = torch.zeros(G, R, C, device=dev, dtype=torch.float32)
    kw = dict(steps=w.steps, coeffs=w.coeffs, mode=w.mode, restart_after=w.restart_after, safety=w.safety,
              compute_dtype=w.compute, sym_updates=not args.general_updates)
    for i in range(args.warmup):
        nsg.muon_step(W, M, grad, 0.95, 0.02, 0.01, 1.0, seed=1, step=i, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        nsg.muon_step(W, M, grad, 0.95, 0.02, 0.01, 1.0, seed=1, step=args.warmup + i, **kw)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the elementwise kernels on their own
    O = torch.empty(G, R, C, device=dev, dtype=torch.float32)
    n = W.numel()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        nsg.muon_momentum(M, grad, 0.95)
    torch.cuda.synchronize()
    tm = (time.perf_counter() - t1) / args.steps
    t1 = time.perf_counter()
    for i in range(args.steps):
        nsg.muon_update(W, O, 0.0, 0.0, 1.0, seed=1, step=i)
    torch.cuda.synchronize()
    tu = (time.perf_counter() - t1) / args.steps
    credited, _ = nsg.flops(R, C, **kw)
    res = {
        "metric": "matrices/s, Muon step (momentum + Gram NS + update, bf16 stochastic rounding)",
        "value": round(G * args.steps / wall, 3), "unit": "matrices/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(1e3 * wall / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16" if w.compute == "f16" else w.compute,
        "data": "synthetic", "config": {"workload": w.name, "G": G, "R": R, "C": C, "W": "bf16", "M": "f32"},
        "effective_tflops": round(credited * G * args.steps / wall / 1e12, 2),
        "momentum": {"ms": round(1e3 * tm, 3), "gbs": round(n * 10 / tm / 1e9, 1)},
        "update": {"ms": round(1e3 * tu, 3), "gbs": round(n * 8 / tu / 1e9, 1)},
    }
    print(json.dumps(res), flush=True)


def bench_blas(args, w, dev):
    """Calibration only: the vendor BLAS (torch.matmul) on the bucket's product shapes, fp16 operands,
    full products (it has no symmetric or fused forms). Not part of the library's path."""
    import torch
    torch.manual_seed(0)
    G, n, m = w.G, min(w.R, w.C), max(w.R, w.C)
    rnd = lambda *s: (torch.randn(*s, device=dev) * 0.5).half()

    def timed(f, reps):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    Q, X = rnd(G, n, n), rnd(G, n, m)
    Xt = X.transpose(1, 2).contiguous()
    cases = [("Q X (n x n times n x m)", lambda: torch.matmul(Q, X), 2.0 * G * n * n * m),
             ("X X^T (n x m times m x n)", lambda: torch.matmul(X, Xt), 2.0 * G * n * n * m),
             ("Q Q (n x n times n x n)", lambda: torch.matmul(Q, Q), 2.0 * G * n ** 3)]
    res = {}
    for name, f, fl in cases:
        ms = timed(f, max(args.steps, 1))
        res[name] = {"ms": round(ms, 3), "tflops": round(fl / ms / 1e9, 1),
                     "pct_fp16_peak": round(100.0 * fl / ms / 1e9 / PEAK_FP16_TFLOPS, 1)}
    print(json.dumps({"vendor_blas_fp16": res, "workload": w.name, "G": G, "n": n, "m": m}), flush=True)


def time_workload(w, dev, steps, warmup, sym_updates=True, calibrate_copy=False, min_seconds=0.0):
    """Warm up, then time `steps` whole calls with per-launch HIP events from the
    library; returns (result dict, input on the host, GPU output).  With
    min_seconds > 0, `steps` grows (up to 1000) until the timed calls take
    about that long at the warm-up calls' pace, so that one slow call cannot
    dominate a short bucket's rate."""
    import torch

    import newton_schulz_gram_amd as nsg
    import synth

    t_gen = time.perf_counter()
    x_cpu = synth.make(w)
    t_gen = time.perf_counter() - t_gen
    x = x_cpu.to(dev)
    out = torch.empty_like(x)
    kw = dict(steps=w.steps, coeffs=w.coeffs, mode=w.mode, restart_after=w.restart_after,
              safety=w.safety, compute_dtype=w.compute, sym_updates=sym_updates)
    ws = torch.empty(nsg.workspace_size(w.G, w.R, w.C, **kw), dtype=torch.uint8, device=dev)
    status = torch.zeros(w.G, dtype=torch.int32, device=dev)
    plan = nsg.plan(w.R, w.C, in_dtype=w.dtype, **kw)
    credited, executed = nsg.flops(w.R, w.C, **kw)

    if calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            nsg.copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    t_w = time.perf_counter()
    for _ in range(warmup):
        nsg.orthogonalize(x, out=out, workspace=ws, status=status, **kw)
    torch.cuda.synchronize()
    if min_seconds > 0 and warmup > 0:
        per_call = (time.perf_counter() - t_w) / warmup
        steps = max(steps, min(1000, int(math.ceil(min_seconds / max(per_call, 1e-6)))))

    # timed region: `steps` whole calls, one event between calls and none
    # inside them (the library's per-launch events add a marker pair to every
    # launch: ~6 us each, 10% of a GPT-2-sized call)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        nsg.orthogonalize(x, out=out, workspace=ws, status=status, **kw)
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))

    # per-launch durations: `steps` more calls with a HIP event pair around
    # every launch, recorded by the library on the stream its kernels run on
    nsg.timing_enable(True)
    nsg.timing_collect()
    t1 = time.perf_counter()
    for i in range(steps):
        nsg.orthogonalize(x, out=out, workspace=ws, status=status, **kw)
    torch.cuda.synchronize()
    wall_instrumented = time.perf_counter() - t1
    recs = nsg.timing_collect()
    nsg.timing_enable(False)

    value = w.G * steps / wall
    eff_tflops = credited * w.G * steps / wall / 1e12

    # per-launch durations, matched to the plan (same launch order every step)
    per = len(plan)
    assert len(recs) == per * steps, (len(recs), per, steps)
    by_kernel = {}
    for i, (name, ms) in enumerate(recs):
        e = plan[i % per]
        d = by_kernel.setdefault(name, {"ms": 0.0, "launches": 0, "algo_flops": 0.0, "bytes": 0.0})
        d["ms"] += ms
        d["launches"] += 1
        d["algo_flops"] += algorithmic_flops(e, w.G)
        d["bytes"] += e["bytes"] * w.G
    bytes_per_matrix = sum(e["bytes"] for e in plan)
    label, bound = WORKLOAD_INFO.get(w.name, (f"matrices/s, {w.mode} NS, {w.name}", "mfma"))
    dominant = max((k for k in by_kernel if k.startswith("gemm")), key=lambda k: by_kernel[k]["ms"])
    d = by_kernel[dominant]
    avg_ms = d["ms"] / d["launches"]
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            ent = tr.get(w.name, {}).get(dominant)
            if ent and ent.get("kernel_src") == kernel_source_hash():
                traffic = ent.get("bytes_per_launch")
        except Exception:
            traffic = None
    common = {"kernel": dominant, "traffic": traffic, "avg_launch_ms": round(avg_ms, 4),
              "launches_per_step": d["launches"] // steps}
    if bound == "latency":
        roofline = {"bound": "latency", "achieved": None, "peak": None, "unit": None, "frac": None,
                    "us_per_launch": round(1e3 * sum(v["ms"] for v in by_kernel.values()) / len(recs), 2),
                    "launches_per_step": per, **{k: common[k] for k in ("kernel", "avg_launch_ms")}}
    elif bound == "hbm":
        achieved = d["bytes"] / d["launches"] / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), **common,
                    "algo_bytes_per_launch": d["bytes"] / d["launches"]}
    else:
        achieved = d["algo_flops"] / d["launches"] / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4), **common,
                    "algo_flops_per_launch": d["algo_flops"] / d["launches"]}
    # normalize pass: the norm reads the input; the scale pass reads it again
    # and writes X0 once, or moves nothing when the products read the input in
    # place (16-bit input in the compute dtype, sides multiples of 256)
    norm_bytes = w.G * sum(e["bytes"] for e in plan if e["kind"] in (0, 1))
    in_place = any(e["kind"] == 1 and e["label"] == "scales" for e in plan)
    norm_ms = sum(by_kernel.get(k, {"ms": 0})["ms"] for k in ("norm_reduce", "scale_cast_transpose"))
    kernels = {k: {"ms_per_step": round(v["ms"] / steps, 3),
                   "tflops_algo": round(v["algo_flops"] / (v["ms"] * 1e-3) / 1e12, 1) if v["algo_flops"] else None,
                   "gbs_algo": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1)}
               for k, v in by_kernel.items()}
    # whole call against the HBM roofline of its algorithmic bytes
    hbm_roof_mps = PEAK_HBM_GBS * 1e9 / bytes_per_matrix
    x0_copy_roofline = None
    if in_place:
        es_in = x.element_size()
        x0_bytes = bytes_per_matrix + w.R * w.C * es_in + w.n * w.m * (4 if w.compute == "f32" else 2)
        x0_mps = PEAK_HBM_GBS * 1e9 / x0_bytes
        x0_copy_roofline = {"bytes_per_matrix": x0_bytes, "matrices_per_s": round(x0_mps, 1),
                            "frac": round(value / x0_mps, 4)}
    res = {
        "metric": label,
        "value": round(value, 3),
        "unit": "matrices/s",
        "ms_per_step": round(1e3 * wall / steps, 3),
        "ms_per_call_median": round(per_call[len(per_call) // 2], 3),
        "ms_per_call_iqr": round(per_call[(3 * len(per_call)) // 4] - per_call[len(per_call) // 4], 3),
        "ms_per_call_instrumented": round(1e3 * wall_instrumented / steps, 3),
        "effective_tflops": round(eff_tflops, 2),
        "pct_fp16_peak": round(100 * eff_tflops / PEAK_FP16_TFLOPS, 2),
        "executed_tflops": round(executed * w.G * steps / wall / 1e12, 2),
        "flops_per_matrix": {"credited": credited, "executed": executed},
        "algo_bytes_per_matrix": bytes_per_matrix,
        "hbm_roofline": {"matrices_per_s": round(hbm_roof_mps, 1),
                         "tflops": round(credited * hbm_roof_mps / 1e12, 1),
                         "frac": round(value / hbm_roof_mps, 4),
                         # the same count with the normalized X0 written once
                         # and read back (the method's normalize step taken
                         # literally), for a run that reads the input in place
                         "with_x0_copy": x0_copy_roofline},
        "normalize": {"ms_per_step": round(norm_ms / steps, 3),
                      "algo_bytes": norm_bytes, "input_read_in_place": in_place,
                      "gbs": round(norm_bytes / (norm_ms / steps * 1e-3) / 1e9, 1) if norm_ms else None},
        "kernels": kernels,
        "roofline": roofline,
        "nonfinite_matrices": int(status.sum().item()),
        "input_gen_s": round(t_gen, 1),
        "steps": steps,
        "warmup": warmup,
        "config": {"workload": w.name, "G": w.G, "R": w.R, "C": w.C, "input_dtype": w.dtype,
                   "mode": w.mode if w.R != w.C else "standard (square fallback)", "steps": w.steps,
                   "restart_after": w.restart_after, "safety": w.safety, "coeffs": list(w.coeffs),
                   "compute": w.compute, "accumulate": "f32", "sym_updates": sym_updates},
    }
    del ws, x
    return res, x_cpu, out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time only the named workload (default: the other four buckets too)")
    ap.add_argument("--select-fraction", type=float, default=None,
                    help="time the Dion3 selection front-end: k = ceil(f n) lines of the smaller dimension")
    ap.add_argument("--muon-step", action="store_true",
                    help="time the whole Muon step (momentum, orthogonalization, update) on the bucket")
    ap.add_argument("--general-updates", action="store_true",
                    help="run Q Z + a Q and R Z + a R as general products (default: symmetric kernel)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="calibration: time the vendor BLAS (torch.matmul) on the bucket's product shapes")
    ap.add_argument("--cpu-budget", type=float, default=30.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run the library copy kernel over COPY_BYTES (byte-counter calibration)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store traffic per launch from two rocprofv3 --pmc counter_collection.csv files")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus > 1 is not supported "
                                   "(matrices are independent: the bucket would be split across GPUs)"}))
        sys.exit(2)

    import torch

    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.select_fraction is not None:
        return bench_select(args, w, dev)
    if args.muon_step:
        return bench_muon(args, w, dev)
    if args.blas_reference:
        return bench_blas(args, w, dev)
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"timing {w.name}: {args.warmup} warm-up + {args.steps} timed calls")
    res, x_cpu, out = time_workload(w, dev, args.steps, args.warmup, not args.general_updates,
                                    args.calibrate_copy)
    head = {"metric": res.pop("metric"), "value": res.pop("value"), "unit": res.pop("unit"), "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16" if w.compute == "f16" else w.compute, "data": "synthetic",
            "config": res.pop("config")}
    res.pop("steps")
    res.pop("warmup")
    line = dict(head, **res)
    line["device"] = {"name": props.name, "cus": props.multi_processor_count}
    if not args.no_cpu_baseline:
        log("oracle baseline and parity sample")
        base, idx, ref = cpu_baseline(w, x_cpu, args.cpu_budget)
        line["cpu_baseline"] = base
        line["parity"] = parity_object(out, idx, ref)
    del out, x_cpu
    torch.cuda.empty_cache()
    if not args.no_other_configs and args.workload == DEFAULT_WORKLOAD:
        others = {}
        for name in OTHER_CONFIGS:
            wo = synth.WORKLOADS[name]
            steps = min(args.steps, 10)
            log(f"timing {name}: {min(args.warmup, 3)} warm-up + at least {steps} timed calls (about 0.1 s)")
            r, xo, oo = time_workload(wo, dev, steps, max(1, min(args.warmup, 3)), not args.general_updates,
                                      min_seconds=0.1)
            if not args.no_cpu_baseline:
                idx = PARITY_SAMPLE[name]
                t0 = time.perf_counter()
                classes = None
                if wo.kind == "conditioning":
                    from synth.workloads import conditioning_class_of
                    classes = lambda g, G=wo.G: conditioning_class_of(G, g)
                r["parity"] = parity_object(oo, idx, oracle_outputs(wo, xo, idx), classes)
                r["parity"]["oracle_s"] = round(time.perf_counter() - t0, 1)
            del xo, oo
            torch.cuda.empty_cache()
            others[name] = r
        line["other_configs"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
