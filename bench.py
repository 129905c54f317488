"""Benchmark of the decode hot path (score -> top-k -> sparse attention) on one
MI355X.  Prints ONE JSON line.

Workload (default): the batched-decode configuration — 32 sequences with
context lengths uniform in [8192, 32768] (seed 1), one query each, 32 query
heads / 4 KV heads, head_dim 128, bf16; indexer 8 heads x 128 bf16, ratio 4,
budget 2048 (512 blocks).  `--config c3` selects the 8 x 131072 long-context
decode with the e4m3 index plane instead.

A step is one pass of the whole hot path over one batch: canonical indexer
scores, block top-k and sparse gather attention, all resident in HBM.  Key
compression is an ingest-time pass and is timed separately (`compress_ms`).
Steps rotate over several device copies of the inputs (more distinct bytes
than the 256 MB last-level cache holds), so a step cannot be served from a
cache warmed by the previous one.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="c2", choices=["c2", "c3"])
    p.add_argument("--replicas", type=int, default=0, help="input copies to rotate over (0=auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="only run a plain device-to-device copy of this many MiB (5 times) "
                        "to calibrate the FETCH_SIZE / WRITE_SIZE counters, then exit")
    return p.parse_args()


def algorithmic_bytes(wl):
    """Per-step bytes the method must move: index scan over
    visible compressed keys, K/V rows of the selected token set, q and out,
    indexer query/weights and the idx row.  Scores are an intermediate and are
    excluded.  Returns (step_bytes, attention_bytes, score_bytes)."""
    sp = wl.spec
    s_kv = 2 if sp.kv_dtype == "bf16" else 4
    s_kc = {"bf16": 2, "f32": 4, "e4m3": 1}[sp.kc_dtype]
    s_scale = 4 if sp.kc_dtype == "e4m3" else 0
    s_qi = 2 if sp.idx_dtype == "bf16" else 4
    K = sp.budget // sp.ratio
    attn = score = 0
    for L in wl.visible_lengths():
        L = int(L)
        nb = L // sp.ratio
        tail = L - nb * sp.ratio
        T = min(L, K * sp.ratio + tail)
        score += nb * (sp.d_idx * s_kc + s_scale) + sp.h_idx * sp.d_idx * s_qi + 4 * sp.h_idx
        attn += T * 2 * sp.hkv * sp.d * s_kv + sp.hq * sp.d * 2 * s_kv + 4 * K
    return score + attn, attn, score


def cpu_baseline(wl, seconds):
    """The oracle, as it stands, on a bounded sample: all queries of the
    workload, repeated until about `seconds` of wall time."""
    import oracle
    sp = wl.spec
    kc, kc_scale = oracle.compress(wl.k_idx.float().numpy(), wl.kv_offsets, sp.ratio, sp.kc_dtype)
    kcv = oracle.kc_values(kc, sp.kc_dtype)
    blk = wl.blk_offsets()
    Ls = wl.visible_lengths()
    seqs = []
    for s in range(wl.num_seqs):
        a, b = int(wl.kv_offsets[s]), int(wl.kv_offsets[s + 1])
        seqs.append((wl.K[a:b].float().numpy(), wl.V[a:b].float().numpy(),
                     kcv[blk[s]:blk[s + 1]], None if kc_scale is None else kc_scale[blk[s]:blk[s + 1]],
                     wl.q[s:s + 1].float().numpy(), wl.q_idx[s:s + 1].float().numpy(),
                     wl.w[s:s + 1].numpy(), Ls[s:s + 1]))
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    done = 0
    reps = 0
    while True:
        # parallel over queries: one call per sequence uses 1 query, so batch
        # the sequences through a thread pool of oracle calls
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda a: oracle.run_queries(*a, sp.ratio, sp.budget, sp.softmax_scale,
                                                     n_threads=1), seqs))
        done += len(seqs)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x all {len(seqs)} decode queries of the workload "
                      f"(score+sort+fp64 attention per query; compression excluded), "
                      f"{dt:.1f} s on {threads} threads of {os.cpu_count()} host cpus"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    if args.calibrate_copy_mb:
        n = args.calibrate_copy_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 5}))
        return
    import qsa_workloads as W
    from indexer_selected_sparse_amd import pipeline

    spec = W.CONFIGS[args.config]
    wl = W.make(spec)
    step_bytes, attn_bytes, score_bytes = algorithmic_bytes(wl)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    base = pipeline.upload(wl, dev, decode=True)

    # compression (ingest pass), timed on its own
    base.compress()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(5):
        base.compress()
    ev1.record()
    torch.cuda.synchronize()
    compress_ms = ev0.elapsed_time(ev1) / 5

    R = args.replicas or max(2, math.ceil(2 * 256e6 / step_bytes) + 1)
    reps = [base]
    for _ in range(R - 1):
        c = pipeline.DeviceProblem(**{**base.__dict__})
        c.K, c.V = base.K.clone(), base.V.clone()
        c.kc = base.kc.clone()
        c.kc_scale = None if base.kc_scale is None else base.kc_scale.clone()
        c.q, c.q_idx, c.w = base.q.clone(), base.q_idx.clone(), base.w.clone()
        reps.append(c)
    torch.cuda.synchronize()

    for s in range(args.warmup):
        reps[s % R].step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        p = reps[s % R]
        e = evs[s]
        e[0].record()
        p.score()
        e[1].record()
        p.topk()
        e[2].record()
        p.attend()
        e[3].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    t_score = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    t_topk = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    t_attn = np.mean([e[2].elapsed_time(e[3]) for e in evs])

    qps = wl.total_q / (ms_step / 1e3)
    attn_gbps = attn_bytes / (t_attn * 1e-3) / 1e9
    rec = {
        "metric": "sparse-attn decode queries/s + achieved HBM GB/s (% roofline) at 32K-128K ctx",
        "value": qps, "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec.name, "num_seqs": wl.num_seqs, "queries_per_step": wl.total_q,
                   "context": (f"U[{spec.len_range[0]},{spec.len_range[1]}]" if spec.len_range
                               else str(wl.lens[0])),
                   "heads": f"{spec.hq}/{spec.hkv}x{spec.d}", "indexer": f"{spec.h_idx}x{spec.d_idx} {spec.kc_dtype}",
                   "ratio": spec.ratio, "budget": spec.budget, "seed": spec.seed,
                   "input_replicas": R},
        "roofline": {"bound": "hbm", "achieved": attn_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": attn_gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "qsa_sparse_attn_decode (gather attention + split combine)",
                     "bytes_per_launch": attn_bytes, "avg_ms": float(t_attn)},
        "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_bytes": step_bytes,
        "kernel_ms": {"index_score": float(t_score), "topk": float(t_topk),
                      "sparse_attn": float(t_attn)},
        "index_score_gbps": score_bytes / (t_score * 1e-3) / 1e9,
        "compress_ms": compress_ms,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
