#!/usr/bin/env python3
"""Benchmark of the FP4 paged indexer hot path on one MI355X.

A step is one pass of the decode path over one batch of synthetic input: weighted-ReLU
logits for 4 verify rows of one request at context 100,000 (H=32, D=128, MXFP4 keys on
shuffled 64-token pages), then the top-2048 columns of each row.  This is the
configuration the pages time ("[DSv4.1] Speed up the FP4 indexer scorer...", Speed
Tests: 4 verify rows, 32 heads, contexts 16,384 / 100,000 / 400,000).

Timing: inputs are resident in HBM before the timed region.  Steps rotate over enough
independent input/output sets that their total (> 512 MiB) exceeds the 256 MiB
Infinity Cache, so every step reads its keys from HBM.  The K timed steps are
replayed from HIP graphs (as the pages' bench replays CUDA graphs), bracketed by
device synchronisation.  Kernel durations for the roofline are measured separately:
a graph of back-to-back launches of one kernel, replayed between HIP events recorded
on its own stream.

Prints one JSON line.  `--gpus N` with N > 1 is refused: this path runs on one GPU.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD public spec
CSRC = "sparse_attention_fp4_amd/csrc/"
COMMON_SOURCES = [CSRC + "device_common.hpp", CSRC + "fp4idx_internal.hpp", CSRC + "fp4idx_api.hip"]
KERNEL_SOURCES = {"logits": [CSRC + "logits.hip"] + COMMON_SOURCES,
                  "topk": [CSRC + "topk.hip", CSRC + "topk_long.hip"] + COMMON_SOURCES}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--ctx", type=int, default=100_000)
    ap.add_argument("--workload", choices=["verify", "batched"], default="verify",
                    help="verify: 4 rows of one request at --ctx (the headline); batched: 64 "
                         "requests x 1 row, H=64, contexts 4096..131072")
    ap.add_argument("--topk", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-launches", type=int, default=64,
                    help="launches per timed graph replay, per kernel, for the roofline")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain fp32 copy of this many MiB (read N, write N) so "
                         "that a counter profile of this run can scale HBM byte counters")
    return ap.parse_args()


def source_hash(files) -> str:
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per call from the committed rocprofv3 counter summary
    (profiles/<workload>.md: FETCH_SIZE and WRITE_SIZE scaled by a plain copy), or None
    if there is none or the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            key, sep, val = line.strip().partition(": ")
            if sep and key.startswith(kernel + "_"):
                rec[key[len(kernel) + 1:]] = val.strip()
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    v = rec.get("hbm_bytes_per_launch")
    return int(v) if v is not None else None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs the indexer on one GPU only; --gpus {args.gpus} is not supported "
              "(requests are independent: a multi-GPU run would be N copies of this one).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_fp4_amd as fp4
    from sparse_attention_fp4_amd import workloads as wl

    assert torch.cuda.is_available(), "no GPU visible"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.workload == "verify":
        case = wl.config1(args.ctx)
        workload = f"decode_ctx{args.ctx}_h32"
        desc = (f"{workload}: 1 request, 4 verify rows seeing ctx-0..3 keys, H=32, D=128, "
                f"MXFP4, page 64 shuffled, logits + top-{args.topk}")
    else:
        case = wl.config2()
        workload = "batched_decode_b64_h64"
        desc = (f"{workload}: 64 requests x 1 row, H=64, D=128, contexts U[4096,131072], MXFP4 "
                f"E8M0 120..134, page 64 shuffled, logits [64,131072] + top-{args.topk}")
    T, H, k = case.T, case.H, args.topk
    out_cols = case.out_cols

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    base = dict(q=up(case.q_fp4), qs=up(case.q_scale), w=up(case.w), k=up(case.k_fp4),
                ks=up(case.k_scale), bt=up(case.block_table), cu=up(case.cu_seqlens_q),
                lens=up(case.row_lens))
    set_bytes = sum(t.numel() * t.element_size() for t in base.values()) + T * out_cols * 4
    n_sets = int(min(256, max(2, -(-(512 << 20) // set_bytes))))
    if args.steps % n_sets and args.steps < n_sets:
        n_sets = max(2, args.steps)
    sets = []
    for i in range(n_sets):
        s = {n: (t if n in ("cu", "lens", "bt") else t.clone()) for n, t in base.items()}
        s["out"] = torch.empty((T, out_cols), dtype=torch.float32, device=dev)
        s["idx"] = torch.empty((T, k), dtype=torch.int32, device=dev)
        s["val"] = torch.empty((T, k), dtype=torch.float32, device=dev)
        sets.append(s)
    ws_bytes = fp4.topk_workspace_bytes(T, out_cols, k)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def logits(s):
        fp4.logits_paged(s["q"], s["qs"], s["w"], s["k"], s["ks"], s["bt"], s["cu"], s["lens"],
                         fmt="mxfp4", out_cols=out_cols, out=s["out"])

    def topk(s):
        fp4.topk(s["out"], k, s["lens"], out_idx=s["idx"], out_vals=s["val"], workspace=ws)

    def step(s):
        logits(s)
        topk(s)

    # ---- warmup (eager)
    for i in range(args.warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()

    # ---- graphs: one with a step on every set, one with the remainder
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(stream):
        for count in (n_sets, args.steps % n_sets):
            if count == 0:
                graphs.append(None)
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(count):
                    step(sets[i])
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    full, rem = graphs
    for g in graphs:                       # one untimed replay each
        if g is not None:
            g.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly args.steps steps
    reps = args.steps // n_sets
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        full.replay()
    if rem is not None:
        rem.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # ---- warm-cache reference: the same set every step (eager graph of 20 calls)
    gw = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gw, stream=stream):
            for _ in range(20):
                step(sets[0])
    torch.cuda.synchronize()
    gw.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(10):
        gw.replay()
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t1) * 1e3 / 200

    # ---- per-kernel durations: a hipGraph of `kernel_launches` launches of one kernel
    # (cycling over the input sets, so reads stay cache-cold), replayed between two HIP
    # events recorded on the stream the graph runs on; duration = elapsed / launches.
    def time_kernel(fn):
        L = args.kernel_launches
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(gk, stream=stream):
                for i in range(L):
                    fn(sets[i % n_sets])
        torch.cuda.synchronize()
        per = []
        with torch.cuda.stream(stream):
            gk.replay()                                  # untimed
            for _ in range(5):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                gk.replay()
                e1.record(stream)
                per.append((e0, e1))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 / L for a, b in per]
        return float(np.mean(us)), float(np.median(us))

    for s in sets[:4]:
        step(s)
    torch.cuda.synchronize()
    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 18                   # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)                               # reads N MiB, writes N MiB
        torch.cuda.synchronize()
        del src, dst
    logits_us, logits_med = time_kernel(logits)
    topk_us, topk_med = time_kernel(topk)

    # ---- algorithmic bytes (each input once, each output once)
    keys = case.unique_keys()                        # distinct keys read
    G = 4
    pages = -(-keys // case.page_size)
    logits_bytes = (keys * (64 + G)                  # packed nibbles + E8M0 scales
                    + T * H * (64 + G) + T * H * 4   # queries, scales, weights
                    + pages * 4 + (T + 2) * 4        # block table, lengths, cu_seqlens
                    + T * out_cols * 4)              # logits out
    topk_bytes = int(np.minimum(case.row_lens, out_cols).sum()) * 4 + T * 4 + T * k * 8
    pairs = case.visible_pairs()
    kern = {
        "logits": dict(us=logits_us, us_median=logits_med, bytes=logits_bytes),
        "topk": dict(us=topk_us, us_median=topk_med, bytes=topk_bytes),
    }
    dom = max(kern, key=lambda n: kern[n]["us"])
    d = kern[dom]
    achieved = d["bytes"] / (d["us"] * 1e-6) / 1e9
    traffic = load_traffic(dom, workload)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": dom,
                "algorithmic_bytes_per_launch": d["bytes"], "avg_launch_us": round(d["us"], 3)}

    result = {
        "metric": "keys scored/sec + us/call (FP4 paged indexer) at 100k ctx; % HBM roofline",
        "value": round(pairs / (ms_per_step * 1e-3), 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 x e8m0, fp32 accumulate)",
        "data": "synthetic (seeded codes with the pages' distributions)",
        "config": {"workload": desc,
                   "ctx": args.ctx if args.workload == "verify" else "4096..131072",
                   "rows": T, "heads": H, "topk": k,
                   "input_sets_rotated": n_sets, "timing": "hipGraph replay, cache-cold rotation"},
        "us_per_call": {"logits": round(logits_us, 3), "topk": round(topk_us, 3),
                        "step_cold": round(ms_per_step * 1e3, 3),
                        "step_warm_same_buffers": round(warm_ms * 1e3, 3)},
        "roofline": roofline,
        "context": {"pages_sm120_logits_us_at_100k": 59.9,
                    "note": "the pages' SGLang scorer on RTX PRO 6000 (SM120), logits only"},
    }
    for name, kv in kern.items():
        result["us_per_call"][name + "_GBps"] = round(kv["bytes"] / (kv["us"] * 1e-6) / 1e9, 1)

    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        threads = min(T, orc.max_threads())
        tc = time.perf_counter()
        ref, _, _ = orc.logits_paged(case.fmt, case.q_fp4, case.q_scale, case.w, case.k_fp4,
                                     case.k_scale, case.block_table, case.cu_seqlens_q,
                                     case.row_lens, case.page_size, out_cols, n_threads=threads)
        orc.topk(ref, k, case.row_lens, n_threads=threads)
        cpu_s = time.perf_counter() - tc
        result["cpu_baseline"] = {
            "value": round(pairs / cpu_s, 1), "unit": "keys/s", "cores": threads, "kind": "oracle",
            "sample": f"one full step (logits for all {T} rows x {out_cols} columns, then top-{k}), "
                      f"{cpu_s:.1f} s"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
