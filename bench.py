#!/usr/bin/env python3
"""Throughput of the exact tiled attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one forward (fa_fwd) plus one backward (fa_bwd: D = rowsum(dO * O)
and the fp16 operand copies, then one launch holding the dK/dV and dQ
workgroups) over the whole batch, inputs already resident in HBM.  K steps
are timed between two synchronisations with HIP events recorded on the
stream the kernels run on (torch's current stream, which the binding passes
to the library): that is `value` and ms_per_step.  K more steps then run the
same launches with an event after each (fa_fwd, then fa_bwd as its two
stages: FA_BWD_STAGE_D and FA_BWD_STAGE_GRADS, which is exactly fa_bwd's
launch sequence), which gives each kernel's average duration (kernel_ms,
roofline); those events add a few microseconds between launches, so that
loop is reported separately (ms_per_step_with_kernel_events).  A third loop
launches the dK/dV and dQ workgroups as separate kernels (stages DKDV, DQ)
for their individual times (kernel_ms_staged; not part of the step).

Metric: attention fwd+bwd TFLOPS with the algorithmic FLOP count: 4 d flops
per visible (query, key) pair forward (Q K^T and P V) and 10 d backward
(the recomputed Q K^T, dO V^T, P^T dO, dS^T Q, dS K); causal pairs per head
= N (N + 1) / 2.  The fraction is against MI355X dense bf16 MFMA peak:
256 CU x 2.4 GHz x 4096 flop/clk/CU = 2516.6 TFLOP/s.

Prints one JSON line.  The default workload is the long causal one (B=1,
H=16, N=16384, d=64, bf16), the configuration the target is quoted on.

    python bench.py --decode [--steps K] [--warmup W]

instead times fa_decode (one new query per sequence against a 16384-key
cache: B=16, H=16, d=64, bf16) and reports the rate at which it streams K
and V, against MI355X's 8 TB/s HBM: the decode reads each cached key and
value once and does 4 d flops per key, so it is bound by HBM, not MFMA.

    python bench.py --sweep [--steps K] [--warmup W]

prints one line per point of the sequence-length sweep: H = 16, B = 16384/N,
N = 1K, 2K, 4K, 8K, 16K, d = 64, bf16, causal and non-causal (the same
total tokens at every length).  Any workload of ``workloads.WORKLOADS`` can
be timed with --workload, including key padding (bert_large) and the
block-sparse one; the FLOP count is 4 d (forward) + 10 d (backward) per
visible (query, key) pair, counted exactly under each mask.

    python bench.py --dropout P [--steps K] [--warmup W]

times the same step with dropout at rate P (fa_fwd_dropout, fa_bwd_dropout;
the mask drawn from Philox4x32-10 inside the kernels) and reports it with the
same FLOP count; kernel_ms then holds the forward and the whole backward.
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12    # 2516.6 dense bf16/fp16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


# the sources the forward and 16-bit backward kernels are built from
TRAFFIC_SOURCES = ("fa_api.cpp", "fa_bwd.hip", "fa_device.h", "fa_fwd.hip", "fa_internal.h")


def _code_only(text: str) -> str:
    """C/C++ source without comments and blank-line or trailing-space
    differences (string literals in these sources hold no comment marks)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = (ln.rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_hash() -> str:
    """Hash of the code (comments excluded) of the measured kernels'
    sources; HBM-traffic figures are only reported while it still matches
    the build they were measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "io_aware_tiled_05_amd", "csrc")
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def visible_pairs(w, x):
    """Visible (query, key) pairs of the whole batch: causal, key padding
    (keys j < key_len[b]) and 128 x 128 block masks counted exactly."""
    import numpy as np
    N = w.N
    if w.block_sparse:
        bm = np.asarray(x["block_mask"], dtype=np.int64)
        size = np.minimum(128, N - 128 * np.arange(bm.shape[0])).astype(np.int64)
        return w.B * w.H * int(size @ bm @ size)
    lens = [N] * w.B if x["key_len"] is None else [min(max(int(v), 0), N) for v in x["key_len"]]
    total = 0
    for L in lens:  # causal: query i sees min(i + 1, L) keys
        total += L * (L + 1) // 2 + (N - L) * L if w.causal else N * L
    return w.H * total


def measured_traffic(kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3
    counter summary, or None when absent or taken on other sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


# bwd_fused: the dK/dV and dQ workgroups of fa_bwd in one launch (the timed
# step); bwd_dkdv and bwd_dq: the same bodies launched one at a time (the
# instrumented loop)
KERNEL_KEYS = (("bwd_dkdv_kernel", "bwd_dkdv"), ("bwd_dq_kernel", "bwd_dq"),
               ("bwd_fused_kernel", "bwd_fused"), ("bwd_pre_kernel", "bwd_pre"),
               ("bwd_convert_kernel", "bwd_pre"), ("fwd_kernel", "fwd"))


def kernel_key(name: str):
    for sub, key in KERNEL_KEYS:
        if sub in name:
            return key
    return None


def read_counter_csv(path: str, counter: str):
    """{kernel name: [per-dispatch values]} of one rocprofv3 --pmc csv."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def summarize_counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, out):
    """HBM bytes per launch of each attention kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for a plain device copy of copy_bytes bytes.  Writes
    ``out`` (JSON) tagged with the hash of the kernel sources."""
    def copy_factor(path, counter):
        vals = [v for name, vs in read_counter_csv(path, counter).items()
                if "copyBuffer" in name for v in vs]
        return copy_bytes / (sum(vals) / len(vals) * 1024.0)
    f_fetch = copy_factor(copy_fetch_csv, "FETCH_SIZE")
    f_write = copy_factor(copy_write_csv, "WRITE_SIZE")
    per = {}
    for path, counter, fac, field in ((fetch_csv, "FETCH_SIZE", f_fetch, "fetch_bytes"),
                                      (write_csv, "WRITE_SIZE", f_write, "write_bytes")):
        for name, vals in read_counter_csv(path, counter).items():
            key = kernel_key(name)
            if key is None:
                continue
            # kernels of one key (the two launches of the D pass) add up
            per.setdefault(key, {}).setdefault(field, {})[name] = sum(vals) / len(vals) * 1024 * fac
    kernels = {}
    for key, d in per.items():
        fb = sum(d.get("fetch_bytes", {}).values())
        wb = sum(d.get("write_bytes", {}).values())
        kernels[key] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                        "bytes_per_launch": round(fb + wb)}
    res = {"source_hash": source_hash(),
           "calibration": {"copy_bytes": copy_bytes, "fetch_factor": round(f_fetch, 4),
                           "write_factor": round(f_write, 4)},
           "kernels": kernels}
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    return res


def cpu_baseline(x, w, budget_s=10.0, prefix=8192):
    """The fp64 oracle (forward + backward) on a bounded sample of the same
    workload: whole heads of the causal prefix of ``prefix`` tokens (a causal
    prefix is itself a causal attention problem), one head after another
    until ``budget_s`` of CPU time has been spent."""
    from threadpoolctl import threadpool_info
    from oracle import attention_bwd, attention_fwd
    n = min(prefix, w.N)
    t_total, heads = 0.0, 0
    while heads < w.H and t_total < budget_s:
        sl = (slice(0, 1), slice(heads, heads + 1), slice(0, n))
        q, k, v, dO = (x[name][sl] for name in ("q", "k", "v", "dO"))
        t0 = time.perf_counter()
        attention_fwd(q, k, v, x["scale"], causal=w.causal)
        attention_bwd(q, k, v, dO, x["scale"], causal=w.causal)
        t_total += time.perf_counter() - t0
        heads += 1
    per_head = n * (n + 1) // 2 if w.causal else n * n
    flops = 14 * w.d * per_head * heads
    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    return {
        "value": round(flops / t_total / 1e12, 6),
        "unit": "TFLOPS",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle fwd+bwd on {heads} head(s) x causal prefix of {n} tokens "
                  f"(b=0), {t_total:.1f} s; FLOPs counted as the GPU metric (14 d per pair)",
    }


HBM_PEAK_GBS = 8000.0


def bench_decode(args, fa, torch, np):
    """One JSON line: fa_decode throughput as K/V bytes streamed per second."""
    from workloads import make_decode_inputs
    B, H, Nq, Nk, d = 16, 16, 1, 16384, 64
    fa.load()
    dev = torch.device("cuda:0")
    x = make_decode_inputs(B, H, Nq, Nk, d, "bf16", seed=5)
    q, k, v = (torch.from_numpy(x[n]).to(dev, torch.bfloat16).contiguous() for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_decode_workspace_size(B, H, Nq, Nk, d) // 4 + 4, dtype=torch.float32,
                     device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        fa.fa_decode(q, k, v, scale=x["scale"], out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        fa.fa_decode(q, k, v, scale=x["scale"], out=o, lse=lse, workspace=ws)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    kv_bytes = 2 * B * H * Nk * d * 2          # K and V, bf16, read once
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "decode attention K/V streaming rate, bf16 d=64, 1 GPU",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic N(0,1), seeded",
        "config": {"workload": "decode_long_context", "B": B, "H": H, "Nq": Nq, "Nk": Nk,
                   "d": d},
        "roofline": {"kernel": "decode (partial + merge launches)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }), flush=True)


def bench_workload(args, w, fa, torch, np, with_cpu):
    """One JSON record: K timed steps (forward + the three backward launches,
    or the dropout pair) of workload ``w``."""
    if w.dtype not in ("bf16", "f16"):
        raise SystemExit("bench.py times the 16-bit path")
    if args.dropout > 0 and (w.key_padding or w.block_sparse):
        raise SystemExit("--dropout is timed on dense (optionally causal) workloads")
    from workloads import make_inputs
    fa.load()
    dev = torch.device("cuda:0")
    x = make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    q, k, v, dO = (torch.from_numpy(x[n]).to(dev, tdt).contiguous() for n in ("q", "k", "v", "dO"))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d) // 4, dtype=torch.float32, device=dev)
    scale, causal = x["scale"], w.causal
    kl = None if x["key_len"] is None else torch.from_numpy(x["key_len"]).to(dev)
    bm = None if x["block_mask"] is None else torch.from_numpy(x["block_mask"]).to(dev)
    stream = torch.cuda.current_stream()
    drop_p, drop_seed = float(args.dropout), 0x5EED_0001_2345_6789
    if not 0.0 <= drop_p < 1.0:
        raise SystemExit("--dropout must be in [0, 1)")

    def step(ev=None, stages=None):
        if ev is not None:
            ev[0].record(stream)
        if ev is None and drop_p == 0.0:
            # what a caller runs: one forward and one backward call
            if bm is not None:
                fa.fa_fwd_blocksparse(q, k, v, bm, scale=scale, out=o, lse=lse)
                fa.fa_bwd_blocksparse(q, k, v, o, lse, dO, bm, scale=scale, dq=dq, dk=dk, dv=dv,
                                      workspace=ws)
            else:
                fa.fa_fwd(q, k, v, scale=scale, causal=causal, key_len=kl, out=o, lse=lse)
                fa.fa_bwd(q, k, v, o, lse, dO, scale=scale, causal=causal, key_len=kl, dq=dq,
                          dk=dk, dv=dv, workspace=ws)
            return
        if drop_p > 0.0:
            fa.fa_fwd_dropout(q, k, v, drop_p, drop_seed, 0, scale=scale, causal=causal, out=o,
                              lse=lse)
            if ev is not None:
                ev[1].record(stream)
            fa.fa_bwd_dropout(q, k, v, o, lse, dO, drop_p, drop_seed, 0, scale=scale,
                              causal=causal, dq=dq, dk=dk, dv=dv, workspace=ws)
            if ev is not None:
                ev[2].record(stream)
            return
        if bm is not None:
            fa.fa_fwd_blocksparse(q, k, v, bm, scale=scale, out=o, lse=lse)
        else:
            fa.fa_fwd(q, k, v, scale=scale, causal=causal, key_len=kl, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        for i, st in enumerate(stages):
            fa.fa_bwd_stage(st, q, k, v, o, lse, dO, dq, dk, dv, ws, scale=scale, causal=causal,
                            key_len=kl, block_mask=bm)
            if ev is not None:
                ev[2 + i].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start2, end2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps
    # the step's own launches, an event after each: the forward, the D
    # stage and the one-launch dK/dV + dQ stage (= fa_bwd)
    step_stages = (fa.FA_BWD_STAGE_D, fa.FA_BWD_STAGE_GRADS)
    start2.record(stream)
    for i in range(args.steps):
        step(evs[i], step_stages)
    end2.record(stream)
    torch.cuda.synchronize()
    ms_step_ev = start2.elapsed_time(end2) / args.steps
    names = ("fwd", "bwd") if drop_p > 0.0 else ("fwd", "bwd_pre", "bwd_fused")
    kms = {nm: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
           for j, nm in enumerate(names)}
    kms_staged = None
    if drop_p == 0.0:
        # the dK/dV and dQ workgroups as separate launches (not the step)
        for i in range(args.steps):
            step(evs[i], (fa.FA_BWD_STAGE_D, fa.FA_BWD_STAGE_DKDV, fa.FA_BWD_STAGE_DQ))
        torch.cuda.synchronize()
        kms_staged = {nm: round(float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])), 4)
                      for j, nm in ((2, "bwd_dkdv"), (3, "bwd_dq"))}

    P = visible_pairs(w, x)
    fwd_flops, bwd_flops = 4 * d * P, 10 * d * P
    total_tflops = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
    bwd_ms = kms["bwd"] if drop_p > 0.0 else kms["bwd_pre"] + kms["bwd_fused"]
    fwd_tflops = fwd_flops / (kms["fwd"] * 1e-3) / 1e12
    bwd_tflops = bwd_flops / (bwd_ms * 1e-3) / 1e12

    # algorithmic work per launch of each kernel of the step:
    #   fwd 4 d/pair (Q K^T, P V); bwd_fused 10 d/pair (the recomputed S,
    #   dP, dV, dK, dQ: the one launch of dK/dV and dQ workgroups)
    #   (with dropout the backward is timed as one call: 10 d/pair)
    algo = {"fwd": 4 * d * P, "bwd_fused": 10 * d * P, "bwd": 10 * d * P}
    # traffic: the committed counters were taken on the long causal workload
    with_traffic = drop_p == 0.0 and w.name == "long_causal"

    def roofline_of(kern):
        achieved = algo[kern] / (kms[kern] * 1e-3) / 1e12
        return {"kernel": kern, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(kern) if with_traffic else None}

    # the dominant kernel of the step, and the forward beside it
    dom = max((nm for nm in kms if nm in algo), key=lambda nm: kms[nm])
    roofline = roofline_of(dom)
    roofline_fwd = roofline_of("fwd")

    metric = "attention fwd+bwd TFLOPS & % MFMA peak, bf16 d=64, N=1K-16K, 1 GPU"
    if d != 64:
        metric = metric.replace("d=64", f"d={d}")
    if w.dtype != "bf16":
        metric = metric.replace("bf16", "fp16")
    config = {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": causal,
              "scale": scale, "parallelism": "none (1 GPU)", "visible_pairs": P}
    if kl is not None:
        config["key_len"] = [int(v) for v in x["key_len"]]
    if bm is not None:
        config["block_density"] = round(float(x["block_mask"].mean()), 4)
    if drop_p > 0.0:
        metric = f"attention fwd+bwd with dropout p={drop_p:g} TFLOPS, bf16 d={d}, 1 GPU"
        config["dropout_p"] = drop_p
    out = {
        "metric": metric,
        "value": round(total_tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_with_kernel_events": round(ms_step_ev, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic N(0,1), seeded",
        "config": config,
        "frac_peak": round(total_tflops / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(fwd_tflops, 2),
        "bwd_tflops": round(bwd_tflops, 2),
        "fwd_frac_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
        "bwd_frac_peak": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": {nm: round(v, 4) for nm, v in kms.items()},
        "kernel_ms_staged": kms_staged,
        "wall_s_timed": round(t_wall, 3),
        "roofline": roofline,
        "roofline_fwd": roofline_fwd,
        "cpu_baseline": cpu_baseline(x, w) if with_cpu else None,
    }
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # about 250 ms of work at the default workload: with 5 warm-up steps
    # (12 ms) the first timed loop still ran about 3 % slow, with 40 about
    # 1 % slower than with 200
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="long_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-counters", nargs=5, metavar=("FETCH_CSV", "WRITE_CSV",
                    "COPY_FETCH_CSV", "COPY_WRITE_CSV", "COPY_MIB"),
                    help="write profiles/hbm_traffic.json from rocprofv3 --pmc csv files and exit")
    ap.add_argument("--decode", action="store_true",
                    help="time fa_decode on the long-context decode shape instead")
    ap.add_argument("--sweep", action="store_true",
                    help="one line per point of the sequence-length sweep (H=16, B=16384/N, "
                         "N=1K..16K, d=64, bf16, causal and not) instead")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="time the step with dropout at this rate (secondary line, no oracle leg)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, --steps "
                         "times (the known-size kernel that scales the HBM byte counters)")
    args = ap.parse_args()
    if args.summarize_counters:
        fc, wc, cfc, cwc, mib = args.summarize_counters
        print(json.dumps(summarize_counters(fc, wc, cfc, cwc, int(mib) << 20, TRAFFIC_FILE)))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the per-head kernels run on a single MI355X, and "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import io_aware_tiled_05_amd as fa
    from workloads import SWEEP, WORKLOADS

    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "steps": args.steps}))
        return

    if args.decode:
        bench_decode(args, fa, torch, np)
        return

    if args.sweep:
        for w in SWEEP:
            out = bench_workload(args, w, fa, torch, np, with_cpu=False)
            print(json.dumps(out), flush=True)
        return
    w = WORKLOADS[args.workload]
    with_cpu = not (args.no_cpu_baseline or w.key_padding or w.block_sparse or args.dropout > 0)
    print(json.dumps(bench_workload(args, w, fa, torch, np, with_cpu)), flush=True)


if __name__ == "__main__":
    main()
