#!/usr/bin/env python3
"""Benchmark of the extend-attention hot path on one MI355X.

One step = the whole path over one batch: the unified KV index build, then
extend attention (device planner, attention kernel, split merge).  Inputs
are seeded synthetic tensors already resident in HBM; several copies are
rotated so that the working set exceeds the 256 MiB last-level cache.

Prints ONE JSON line:
  value     causal-adjusted TFLOP/s of the whole step (visible (query, key)
            pairs x Hq x 2 (Lq + Lv), divided by the mean step time)
  roofline  the attention kernel alone: its TFLOP/s from HIP events recorded
            on its own stream around every launch in the timed region,
            against the MI355X dense bf16 MFMA peak (or its algorithmic
            bytes against the HBM peak for batches under the ridge)
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  workloads the same figures (step and kernel times, bound, fraction of the
            binding roofline, oracle sample) for every other workload, when
            no --workload is named
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "fp32": 157.3}  # TFLOP/s: dense MFMA bf16, fp32 vector/MFMA
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "llama8b"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="one workload only (default: the llama8b headline plus every other workload)")
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated (0 = enough to exceed 512 MiB)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--other-cpu-seconds", type=float, default=4.0,
                    help="target CPU time of each other workload's oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel", default="auto", help="attention kernel preference: auto, dl, attn")
    ap.add_argument("--op", default="attention", choices=["attention", "index", "store", "gather", "decode"],
                    help="attention: the hot path; index: the unified index build alone (indptr scan and index "
                         "copy); store / gather: the KV-cache store of the new tokens or the "
                         "request-to-token index gather of the same batch, reported in GB/s against HBM; "
                         "decode: decode attention on a decode batch (--workload decode_llama8b, decode_long, "
                         "decode_mla), GB/s against HBM")
    ap.add_argument("--path", default="two-part", choices=["two-part", "unified"],
                    help="two-part: prefix through kv_indices, new tokens from k/v_extend (the index build "
                         "runs beside it); unified: attention reads every key through the index build's output")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "attention_traffic.json"),
                    help="HBM bytes per attention launch measured with rocprofv3 counters")
    ap.add_argument("--decode-traffic-json", default=os.path.join(ROOT, "profiles", "decode_traffic.json"),
                    help="HBM bytes per decode call (attention + merge launches) measured with rocprofv3 counters")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (calibrates the HBM byte counters)")
    return ap.parse_args()


def cpu_baseline(w, target_s):
    """The oracle, as it is, on a sample of rows of the same workload."""
    import oracle

    rng = np.random.default_rng(123)
    cores = oracle.max_threads()
    e = w.extend_lens.astype(np.int64)
    p = w.prefix_lens.astype(np.int64)
    seq_of = np.repeat(np.arange(w.bs), e)
    pos = np.arange(w.total_q) - np.repeat(w.qo_indptr[:-1].astype(np.int64), e)
    keys_per_row = p[seq_of] + pos + 1
    flop_per_row = keys_per_row * w.cfg.hq * 2.0 * (w.cfg.lq + w.cfg.lv)

    def run(n):
        rows = np.sort(rng.choice(w.total_q, size=min(n, w.total_q), replace=False))
        t0 = time.perf_counter()
        oracle.extend_attention_workload(w, rows=rows)
        return time.perf_counter() - t0, float(flop_per_row[rows].sum()), len(rows)

    dt, fl, n = run(32)
    rate = fl / max(dt, 1e-6)
    want_rows = int(min(w.total_q, max(32, target_s * rate / float(flop_per_row.mean()))))
    if want_rows > n:
        dt, fl, n = run(want_rows)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {w.total_q} new-token rows (all {w.cfg.hq} heads) of the same batch, "
                      f"{fl / 1e9:.1f} GFLOP in {dt:.1f} s, fp64 C loops with OpenMP"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU; sharding across GPUs is not built).", file=sys.stderr)
        return 2

    import torch
    import paged_kv_extend_amd as pkv
    import workloads as wl

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 5}))
        return 0

    if not os.path.exists(pkv.LIB_PATH):
        from paged_kv_extend_amd import _build
        _build.build()
    torch.cuda.init()
    pkv.extend_attention_prefer_kernel(args.kernel)
    dev = torch.device("cuda", 0)
    if args.op == "decode":
        return bench_decode(args, dev, torch, pkv)
    name = args.workload or DEFAULT_WORKLOAD
    if args.op != "attention":
        return bench_copy_op(args, wl.get(name), dev, torch, pkv)
    line = bench_attention(args, name, dev, args.cpu_seconds)
    if args.workload is None:
        # every other workload, one after another, in the same run
        line["workloads"] = {}
        for other in wl.CONFIG_ORDER + wl.AUX_CONFIGS:
            if other != name:
                torch.cuda.empty_cache()
                line["workloads"][other] = brief(bench_attention(args, other, dev, args.other_cpu_seconds))
    print(json.dumps(line), flush=True)
    return 0


def brief(line):
    """The per-workload figures of a bench line."""
    r = line["roofline"]
    out = {"description": line["config"]["description"], "dtype": line["dtype"],
           "ms_per_step": line["ms_per_step"], "ms_per_launch": r["ms_per_launch"],
           "step_tflops": line["value"], "kernel": r["kernel"], "bound": r["bound"], "achieved": r["achieved"],
           "peak": r["peak"], "unit": r["unit"], "frac": r["frac"], "traffic": r["traffic"],
           "causal_gflop": line["config"]["causal_gflop"], "algorithmic_mb": line["config"]["algorithmic_mb"]}
    if "tflops" in r:
        out["kernel_tflops"] = r["tflops"]
    if "cpu_baseline" in line:
        out["cpu_baseline"] = line["cpu_baseline"]
    return out


def bench_attention(args, name, dev, cpu_seconds):
    """The whole path on one workload: index build + extend attention per step."""
    import torch
    import paged_kv_extend_amd as pkv
    import workloads as wl

    w = wl.get(name)
    flops = w.causal_flops()
    algo_bytes = w.algorithmic_bytes()
    copies = args.copies or max(1, min(16, int(np.ceil(512e6 / algo_bytes))))
    sets = [wl.to_torch(w, dev) for _ in range(copies)]
    for s in sets:
        s["uni"] = (torch.empty(w.bs + 1, dtype=torch.int32, device=dev),
                    torch.empty(w.num_prefix + w.total_q, dtype=torch.int64, device=dev),
                    torch.empty(w.bs, dtype=torch.int32, device=dev))
        desc = pkv.make_desc(s["q"], s["k_ext"], s["v_ext"], s["o"], s["k_pool"], s["v_pool"], w.bs,
                             w.num_prefix)
        s["ws"] = torch.empty(pkv.extend_attention_workspace_size(desc), dtype=torch.uint8, device=dev)
    kernel = pkv.extend_attention_kernel_name(desc, s["k_ext"], s["v_ext"], s["k_pool"], s["v_pool"])

    def step(i):
        s = sets[i % copies]
        pkv.build_unified_kv_indices(s["kv_indptr"], s["kv_indices"], s["extend_start_loc"],
                                     s["extend_seq_lens"], s["extend_kv_indices"], w.bs, out=s["uni"])
        if args.path == "unified":
            u_indptr, u_indices, u_plens = s["uni"]
            pkv.extend_attention_fwd_unified(s["q"], s["o"], s["k_pool"], s["v_pool"], s["qo_indptr"], u_indptr,
                                             u_indices, u_plens, sm_scale=w.sm_scale, logit_cap=w.logit_cap,
                                             workspace=s["ws"])
        else:
            pkv.extend_attention_fwd(s["q"], s["k_ext"], s["v_ext"], s["o"], s["k_pool"], s["v_pool"],
                                     s["qo_indptr"], s["kv_indptr"], s["kv_indices"], sm_scale=w.sm_scale,
                                     logit_cap=w.logit_cap, workspace=s["ws"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    pkv.profile_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pkv.profile_enable(False)
    attn_ms_total, calls = pkv.profile_read()
    ms_per_step = start.elapsed_time(stop) / args.steps
    ms_attn = attn_ms_total / max(calls, 1)

    del sets
    peak = PEAK[w.cfg.dtype]
    # the kernel's bound: products above the ridge (peak flop/s over HBM
    # bytes/s), HBM below it (short extends over long prefixes)
    hbm_bound = flops / algo_bytes < peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    achieved = flops / (ms_attn * 1e-3) / 1e12
    traffic = None
    if os.path.exists(args.traffic_json) and args.path == "two-part":
        with open(args.traffic_json) as f:
            tj = json.load(f)
        rec = tj.get("records", {}).get(name)
        if rec and tj.get("kernel_source_sha") == kernel_source_sha():
            traffic = rec.get("bytes_per_launch")
    line = {
        "metric": "extend-attention TFLOP/s (causal-adjusted) + % of bf16 MFMA peak, 1 GPU",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.cfg.dtype,
        "data": "synthetic",
        "config": {"workload": w.cfg.name, "description": w.cfg.description, "bs": w.bs,
                   "q_heads": w.cfg.hq, "kv_heads": w.cfg.hkv, "lq": w.cfg.lq, "lv": w.cfg.lv,
                   "extend_tokens": w.total_q, "prefix_tokens": w.num_prefix, "seed": w.cfg.seed,
                   "causal_gflop": round(flops / 1e9, 3), "algorithmic_mb": round(algo_bytes / 1e6, 2),
                   "input_copies_rotated": copies, "wall_s_timed": round(wall, 3), "path": args.path},
        "mfma_frac_step": round(flops / (ms_per_step * 1e-3) / 1e12 / peak, 4),
        "roofline": ({"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 2),
                      "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                      "traffic": traffic, "ms_per_launch": round(ms_attn, 4),
                      "hbm_gbs_algorithmic": round(algo_bytes / (ms_attn * 1e-3) / 1e9, 1)} if not hbm_bound else
                     {"bound": "hbm", "kernel": kernel, "achieved": round(algo_bytes / (ms_attn * 1e-3) / 1e9, 1),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(algo_bytes / (ms_attn * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "traffic": traffic, "ms_per_launch": round(ms_attn, 4),
                      "tflops": round(achieved, 2)}),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, cpu_seconds)
    return line


def bench_copy_op(args, w, dev, torch, pkv):
    """Unified index build, KV-cache store or request-to-token gather of the workload's batch, timed over
    rotated input copies."""
    c = w.cfg
    esz = 2 if c.dtype == "bf16" else 4
    sets = []
    if args.op == "index":
        # every prefix and new-token index read once and written once, the
        # indptr read and the unified indptr written, three length arrays
        n_p, n_e = w.num_prefix, w.total_q
        nbytes = 16 * (n_p + n_e) + 8 * (w.bs + 1) + 12 * w.bs
        copies = args.copies or max(1, min(16, int(np.ceil(64e6 / max(nbytes, 1)))))

        def t(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).astype(dt)).to(dev)
        for _ in range(copies):
            sets.append(dict(kvp=t(w.kv_indptr, np.int32), kvi=t(w.kv_indices, np.int64),
                             esl=t(w.extend_start_loc, np.int32), elen=t(w.extend_lens, np.int32),
                             eki=t(w.extend_kv_indices, np.int64),
                             out=(torch.empty(w.bs + 1, dtype=torch.int32, device=dev),
                                  torch.empty(max(n_p + n_e, 1), dtype=torch.int64, device=dev),
                                  torch.empty(w.bs, dtype=torch.int32, device=dev))))

        def step(i):
            d = sets[i % copies]
            pkv.build_unified_kv_indices(d["kvp"], d["kvi"], d["esl"], d["elen"], d["eki"], w.bs, out=d["out"])
        metric, what = "unified KV index build GB/s (indptr scan and index copy), 1 GPU", "index_build_kernel"
    elif args.op == "store":
        import workloads as wl
        row_bytes = c.lq * esz + (0 if c.v_aliases_k else c.lv * esz)
        nbytes = 2 * w.total_q * c.hkv * row_bytes  # each new row read once and written once
        copies = args.copies or max(1, min(16, int(np.ceil(512e6 / nbytes))))
        for _ in range(copies):
            d = wl.to_torch(w, dev)
            d["loc"] = d["extend_kv_indices"]
            sets.append(d)

        def step(i):
            d = sets[i % copies]
            pkv.store_kv_cache(d["k_ext"], d["v_ext"], d["k_pool"], d["v_pool"], d["loc"])
        metric, what = "KV-cache store GB/s (new tokens' K/V into the pool), 1 GPU", "store_kv_kernel"
    else:
        stride = int(max(1, w.prefix_lens.max()))
        table = np.zeros((w.bs, stride), np.int32)
        for b in range(w.bs):
            p0, p1 = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
            table[b, :p1 - p0] = w.kv_indices[p0:p1]
        nbytes = w.num_prefix * (4 + 8) + (w.bs + 1) * 4 + w.bs * (8 + 4)
        copies = args.copies or max(1, min(16, int(np.ceil(64e6 / max(nbytes, 1)))))
        for _ in range(copies):
            sets.append(dict(table=torch.from_numpy(table).to(dev),
                             rpi=torch.arange(w.bs, dtype=torch.int64, device=dev),
                             lens=torch.from_numpy(w.prefix_lens.astype(np.int32)).to(dev),
                             out=(torch.empty(w.bs + 1, dtype=torch.int32, device=dev),
                                  torch.empty(max(w.num_prefix, 1), dtype=torch.int64, device=dev))))

        def step(i):
            d = sets[i % copies]
            pkv.gather_kv_indices(d["table"], d["rpi"], d["lens"], capacity=w.num_prefix, out=d["out"])
        metric, what = "request-to-token index gather GB/s, 1 GPU", "gather_indices_kernel"
    # these kernels run for microseconds, less than the host needs to issue a
    # call: one pass over the input copies is captured in a HIP graph and the
    # replays are timed (the kernels record no memset, so they replay as run)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(args.warmup, 1)):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(copies):
            step(i)
    reps = max(1, -(-args.steps // copies))
    graph.replay()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (reps * copies)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": metric, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "timing": "HIP graph of one pass over the input copies, replays timed",
        "vs_baseline": None, "dtype": c.dtype if args.op == "store" else "int64", "data": "synthetic",
        "config": {"workload": c.name, "op": args.op, "bytes_per_step": int(nbytes), "input_copies_rotated": copies},
        "roofline": {"bound": "hbm", "kernel": what, "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4), "traffic": None}}), flush=True)
    return 0


def bench_decode(args, dev, torch, pkv):
    """Decode attention over one decode batch per step, input copies rotated."""
    import workloads as wl

    name = args.workload if args.workload in wl.DECODE_CONFIGS else "decode_llama8b"
    d = wl.decode_get(name)
    c = d.cfg
    nbytes = d.algorithmic_bytes()
    flops = float(d.key_lens.astype(np.int64).sum()) * c.hq * 2.0 * (c.lq + c.lv)
    copies = args.copies or max(1, min(16, int(np.ceil(512e6 / nbytes))))
    sets = []
    for _ in range(copies):
        t = wl.decode_to_torch(d, dev)
        desc = pkv.make_desc(t["q"], None, None, t["o"], t["k_pool"], t["v_pool"], d.bs, d.num_keys)
        t["ws"] = torch.empty(pkv.decode_attention_workspace_size(desc), dtype=torch.uint8, device=dev)
        sets.append(t)

    def step(i):
        t = sets[i % copies]
        pkv.decode_attention_fwd(t["q"], t["o"], t["k_pool"], t["v_pool"], t["kv_indptr"], t["kv_indices"],
                                 sm_scale=d.sm_scale, logit_cap=d.logit_cap, workspace=t["ws"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    pkv.profile_enable(True)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    stop.record()
    torch.cuda.synchronize()
    pkv.profile_enable(False)
    kern_ms, calls = pkv.profile_read()
    ms_kernel = kern_ms / max(calls, 1)
    ms = start.elapsed_time(stop) / args.steps
    gbs_kernel = nbytes / (ms_kernel * 1e-3) / 1e9
    traffic = None
    if os.path.exists(args.decode_traffic_json):
        with open(args.decode_traffic_json) as f:
            tj = json.load(f)
        if tj.get("workload") == name and tj.get("kernel_source_sha") == kernel_source_sha(DECODE_SOURCES):
            traffic = tj.get("bytes_per_launch")
    line = {
        "metric": "decode attention GB/s (algorithmic HBM bytes), 1 GPU", "value": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": c.dtype, "data": "synthetic",
        "config": {"workload": name, "description": c.description, "bs": d.bs, "keys": d.num_keys,
                   "algorithmic_mb": round(nbytes / 1e6, 2), "gflop": round(flops / 1e9, 3),
                   "input_copies_rotated": copies},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": round(gbs_kernel, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs_kernel / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "ms_per_launch": round(ms_kernel, 4),
                     "tflops": round(flops / (ms_kernel * 1e-3) / 1e12, 2)},
    }
    if not args.no_cpu_baseline:
        import oracle

        per_req = d.key_lens.astype(np.float64) * (c.hkv * (c.lq + (0 if c.v_aliases_k else c.lv)) * 2 + 8)
        rng = np.random.default_rng(123)
        order = rng.permutation(d.bs)
        t0 = time.perf_counter()
        oracle.decode_attention(d.q, d.k_pool, d.v_pool, d.kv_indptr, d.kv_indices, d.sm_scale, d.logit_cap,
                                c.dtype, seqs=order[:1])
        dt1 = max(time.perf_counter() - t0, 1e-6)
        n = int(min(d.bs, max(1, args.cpu_seconds / dt1)))
        t0 = time.perf_counter()
        oracle.decode_attention(d.q, d.k_pool, d.v_pool, d.kv_indptr, d.kv_indices, d.sm_scale, d.logit_cap,
                                c.dtype, seqs=order[:n])
        dt = time.perf_counter() - t0
        b = float(per_req[order[:n]].sum())
        line["cpu_baseline"] = {"value": round(b / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.max_threads(),
                                "kind": "oracle",
                                "sample": f"{n} of {d.bs} requests (all heads), {b / 1e6:.0f} MB of K/V in {dt:.1f} s, "
                                          "fp64 C loops with OpenMP"}
    print(json.dumps(line), flush=True)
    return 0


ATTENTION_SOURCES = ("device_common.h", "pkv_internal.h", "attention.hip", "attention_dl.hip", "plan.hip")
DECODE_SOURCES = ("device_common.h", "pkv_internal.h", "decode.hip")


def kernel_source_sha(files=ATTENTION_SOURCES):
    import hashlib

    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_extend_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
