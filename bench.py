"""Benchmark of the hot path (indexer score -> block top-k -> sparse attention)
on one MI355X.  Prints ONE JSON line.

Workloads (synthetic, seeded; see qsa_workloads):
  batched_decode (default)  32 sequences, context U[8192, 32768] (seed 1),
                one query each, 32 query heads / 4 KV heads x 128, bf16;
                indexer 8 x 128 bf16, ratio 4, budget 2048 (512 blocks).
  long_decode   8 x 131072 tokens, 64/8 heads, e4m3 compressed index keys
                with per-block fp32 scales.
  chunked_prefill  an 8193-query causal chunk on a 32768-token prefix;
                indexer scores on the matrix cores, certified top-k, causal
                sparse prefill attention.

A step is one pass of the whole hot path over one batch with every input
resident in HBM.  `value` is queries per second of the step replayed from a
HIP graph that holds the step on each input copy in turn (as the step runs
inside a larger captured graph, without a graph-launch boundary between
steps); `step_ms.graph_one_step` replays one graph per step instead, and
`step_ms.eager` launches the step call by call.  Key compression is an ingest-time pass, timed on its
own (`compress_ms`); with --ingest each decode step first appends every
sequence's newest token (qsa_ingest: its raw key into the ring, the block
it completes, its K/V rows), as a serving step does.  Decode steps rotate over several device copies of the
inputs (more distinct bytes than the 256 MB last-level cache holds), so a
step is not served from a cache warmed by the previous one.

A decode step runs as qsa_decode_step, timed as its two halves: the scorer
(scores + per-chunk candidate lists) and the attention call whose workgroups
select their own part of the selection from the lists (--unfused-step: a
finish launch selects, then the plain attention call).

`roofline` describes the dominant kernel: for decode, the sparse attention
call (selection from the lists + gather kernel + split combine), timed with
HIP events on the stream it runs on; achieved = algorithmic bytes (the
selected K/V rows, q, out and the idx row; the lists, about 0.2% of that, are
not counted) / its mean duration.  `traffic` comes
from the FETCH_SIZE / WRITE_SIZE counter summary under profiles/, used only
while the attention source is unchanged since the counters were taken.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak
# L2 read bandwidth: 16 channels x 128 B/clk per XCD, 8 XCDs, 2.4 GHz
L2_PEAK_GBPS = 16 * 128 * 8 * 2.4
ATTN_SRC = os.path.join(ROOT, "indexer_selected_sparse_amd", "csrc", "qsa_attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_decode_hbm_traffic.md")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="batched_decode",
                   choices=["batched_decode", "long_decode", "chunked_prefill"])
    p.add_argument("--replicas", type=int, default=0, help="input copies to rotate over (0=auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="time eager launches only (default: replay the step from a HIP graph)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--paged", type=int, default=0, metavar="PAGE_SIZE",
                   help="keep K, V and the indexer caches in page pools of PAGE_SIZE tokens "
                        "(random physical page order) and call the paged entry points")
    p.add_argument("--ingest", action="store_true",
                   help="decode: each step first appends every sequence's newest token "
                        "(qsa_ingest: raw key into the ring, the block it completes, K/V rows)")
    p.add_argument("--kc-dtype", default=None, choices=["f32", "bf16", "e4m3", "fp4"],
                   help="store the compressed index keys in this format instead of the workload's "
                        "(fp4: E2M1 values with one E8M0 scale per 32 dims)")
    p.add_argument("--budget", type=int, default=0,
                   help="token budget instead of the workload's (e.g. 8192: budget/ratio = 2048 "
                        "blocks, the other value the pages' model validator allows)")
    p.add_argument("--local-blocks", type=int, default=0,
                   help="decode: also keep the last N complete blocks of every query (union with "
                        "its top-k selection, qsa_topk_blocks_local)")
    p.add_argument("--token-pool", default=None, choices=["max", "mean"],
                   help="decode: select blocks from pooled token scores (every token scored on its "
                        "raw indexer key, each block reduced by max or mean) instead of compressed keys")
    p.add_argument("--layers", type=int, default=1,
                   help="decode: one step runs this many attention layers (layer 0 is the workload; "
                        "the others draw their own K, V, q on the device)")
    p.add_argument("--unfused-ingest", action="store_true",
                   help="with --ingest: the append and the scores as two launches instead of one")
    p.add_argument("--unfused-layers", action="store_true",
                   help="with --layers: one attention launch per layer instead of one per full layer "
                        "and its shared layers")
    p.add_argument("--full-every", type=int, default=1,
                   help="with --layers: layer l has its own indexer when l %% F == 0; the others reuse "
                        "the previous full layer's selection")
    p.add_argument("--unfused-select", action="store_true",
                   help="decode: scores and top-k as two calls (qsa_index_score, qsa_topk_blocks) instead of "
                        "qsa_index_score_topk")
    p.add_argument("--unfused-step", action="store_true",
                   help="decode: the selection as its own launch (qsa_index_score_topk, then "
                        "qsa_sparse_attn_decode) instead of inside the attention kernel (qsa_decode_step, "
                        "timed as its two halves)")
    p.add_argument("--no-long", action="store_true",
                   help="batched_decode: skip the long_decode sub-record (the 128K end of the metric)")
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="only run a plain device-to-device copy of this many MiB (5 times) "
                        "to calibrate the FETCH_SIZE / WRITE_SIZE counters, then exit")
    return p.parse_args()


def token_counts(wl):
    """Per query: (L, nb, |T|) with |T| = min(L, K*ratio + tail)."""
    sp = wl.spec
    K = sp.budget // sp.ratio
    out = []
    for L in wl.visible_lengths():
        L = int(L)
        nb = L // sp.ratio
        out.append((L, nb, min(L, K * sp.ratio + (L - nb * sp.ratio))))
    return out


def algorithmic_bytes(wl, tokens=None):
    """Per-step bytes the decode method must move: index scan over the visible
    compressed keys, K/V rows of the selected token set, q and out, indexer
    query/weights and the idx row.  Scores are an intermediate and are
    excluded.  `tokens`: per-query |T| to use instead of the top-k rule (a
    selection with the recent window kept).  Returns (step_bytes,
    attention_bytes, score_bytes)."""
    sp = wl.spec
    s_kv = 2 if sp.kv_dtype == "bf16" else 4
    s_kc = {"bf16": 2, "f32": 4, "e4m3": 1, "fp4": 0.5}[sp.kc_dtype]
    s_scale = {"e4m3": 4, "fp4": sp.d_idx // 32}.get(sp.kc_dtype, 0)
    s_qi = 2 if sp.idx_dtype == "bf16" else 4
    K = sp.budget // sp.ratio
    attn = score = 0
    for j, (L, nb, T) in enumerate(token_counts(wl)):
        if tokens is not None:
            T = int(tokens[j])
        score += nb * (sp.d_idx * s_kc + s_scale) + sp.h_idx * sp.d_idx * s_qi + 4 * sp.h_idx
        attn += T * 2 * sp.hkv * sp.d * s_kv + sp.hq * sp.d * 2 * s_kv + 4 * K
    return score + attn, attn, score


def ingest_bytes(wl):
    """Per-step bytes of appending one token per sequence: read its raw key
    and K/V rows, write them to the ring and the caches, and for a sequence
    whose length is a multiple of ratio read ratio-1 ring rows and write the
    compressed key (+ scale) of the completed block."""
    sp = wl.spec
    s_kv = 2 if sp.kv_dtype == "bf16" else 4
    s_k = 2 if sp.idx_dtype == "bf16" else 4
    s_kc = {"bf16": 2, "f32": 4, "e4m3": 1, "fp4": 0.5}[sp.kc_dtype]
    s_scale = {"e4m3": 4, "fp4": sp.d_idx // 32}.get(sp.kc_dtype, 0)
    tot = 0
    for L in wl.lens:
        tot += 2 * (sp.d_idx * s_k + 2 * sp.hkv * sp.d * s_kv)
        if int(L) % sp.ratio == 0:
            tot += (sp.ratio - 1) * sp.d_idx * s_k + sp.d_idx * s_kc + s_scale
    return tot


def prefill_flops(wl):
    """(indexer flops over visible (query, block) pairs, attention flops:
    QK and PV over each query's token set)."""
    sp = wl.spec
    idx = attn = 0
    for L, nb, T in token_counts(wl):
        idx += 2 * nb * sp.h_idx * sp.d_idx
        attn += 4 * T * sp.hq * sp.d
    return idx, attn


def recorded_traffic(workload):
    """Bytes per launch from the counter summary, if it was taken on the
    current attention source; else None."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", txt, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    src_hash = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    ent = rec.get("workloads", {}).get(workload)
    if rec.get("attn_source_sha256") != src_hash or ent is None:
        return None
    return ent["hbm_bytes_per_launch"]


def cpu_baseline(wl, seconds, prefill):
    """The oracle, as it stands, on a bounded sample of the workload's queries
    (all of them for decode; a fixed 64-query subset for prefill), repeated
    until about `seconds` of wall time."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    sp = wl.spec
    kc, kc_scale = oracle.compress(wl.k_idx.float().numpy(), wl.kv_offsets, sp.ratio, sp.kc_dtype)
    kcv = oracle.kc_values(kc, sp.kc_dtype, kc_scale)
    kc_scale = oracle.score_scale(kc_scale, sp.kc_dtype)
    blk = wl.blk_offsets()
    Ls = wl.visible_lengths()
    qseq = wl.query_seq()
    if prefill:
        rng = np.random.default_rng(12345)
        qids = np.sort(rng.choice(wl.total_q, min(64, wl.total_q), replace=False))
    else:
        qids = np.arange(wl.total_q)
    jobs = []
    for s in range(wl.num_seqs):
        a, b = int(wl.kv_offsets[s]), int(wl.kv_offsets[s + 1])
        Kf, Vf = wl.K[a:b].float().numpy(), wl.V[a:b].float().numpy()
        kcs = kcv[blk[s]:blk[s + 1]]
        scs = None if kc_scale is None else kc_scale[blk[s]:blk[s + 1]]
        for i in qids[qseq[qids] == s]:
            jobs.append((Kf, Vf, kcs, scs, wl.q[i:i + 1].float().numpy(),
                         wl.q_idx[i:i + 1].float().numpy(), wl.w[i:i + 1].numpy(), Ls[i:i + 1]))
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    done = reps = 0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(lambda j: oracle.run_queries(*j, sp.ratio, sp.budget, sp.softmax_scale,
                                                     n_threads=1), jobs))
            done += len(jobs)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    what = "decode queries" if not prefill else "prefill queries (seeded subset)"
    return {"value": done / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"{reps} x {len(jobs)} {what} of the workload (score + full sort + fp64 "
                      f"attention per query; compression excluded), {dt:.1f} s on {threads} "
                      f"threads of {os.cpu_count()} host cpus"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the benchmark times the path on one MI355X; "
                                   "--gpus must be 1"}))
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
    rec = measure(args, args.workload, cpu=not args.no_cpu_baseline)
    if args.workload == "batched_decode" and not args.no_long and not any(
            (args.paged, args.ingest, args.kc_dtype, args.budget, args.local_blocks, args.token_pool,
             args.layers > 1)):
        # the 128K end of the metric in the same run: its own step time,
        # queries/s and roofline fractions (no CPU baseline)
        lr = measure(args, "long_decode", cpu=False)
        rec["long_decode"] = {k: lr[k] for k in ("config", "value", "unit", "ms_per_step", "step_ms_percentiles",
                                                 "kernel_ms", "roofline", "step_hbm_gbps", "step_hbm_frac",
                                                 "step_bytes", "index_score_gbps") if k in lr}
    print(json.dumps(rec), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measure(args, workload, cpu):
    """Time the hot path of one workload; returns its JSON record."""
    import torch
    log(f"{workload}: generating inputs")
    import qsa_workloads as W
    from indexer_selected_sparse_amd import QSA_SCORE_MFMA, pipeline

    spec = W.CONFIGS[workload]
    prefill = workload == "chunked_prefill"
    if args.budget and args.budget != spec.budget:
        spec = dataclasses.replace(spec, budget=args.budget)
    if args.kc_dtype and args.kc_dtype != spec.kc_dtype:
        if prefill:
            print(json.dumps({"error": "--kc-dtype runs the decode workloads (matrix-core prefill "
                                       "scores take bf16 compressed keys)"}))
            sys.exit(2)
        spec = dataclasses.replace(spec, kc_dtype=args.kc_dtype)
    wl = W.make(spec)
    step_bytes, attn_bytes, score_bytes = algorithmic_bytes(wl)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    base = pipeline.upload(wl, dev, decode=not prefill, mfma_ws=prefill)
    if args.paged:
        if prefill:
            print(json.dumps({"error": "--paged runs the decode workloads (matrix-core prefill "
                                       "scores read contiguous caches only)"}))
            sys.exit(2)
        base = pipeline.page(base, wl.lens, args.paged, seed=spec.seed)
    if args.ingest and prefill:
        print(json.dumps({"error": "--ingest runs the decode workloads"}))
        sys.exit(2)

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
    if args.ingest:
        pipeline.attach_ingest(base, wl)
        step_bytes += ingest_bytes(wl)
    if args.token_pool:
        if prefill:
            print(json.dumps({"error": "--token-pool runs the decode workloads"}))
            sys.exit(2)
        from indexer_selected_sparse_amd import QSA_POOL_MAX, QSA_POOL_MEAN
        pipeline.set_token_pool(base, QSA_POOL_MAX if args.token_pool == "max" else QSA_POOL_MEAN)
        # the scan reads every raw key (and writes token scores) instead of the compressed keys
        sp_ = spec
        s_k = 2 if sp_.idx_dtype == "bf16" else 4
        extra = sum(int(L) * sp_.d_idx * s_k for L in wl.visible_lengths()) - \
            sum((int(L) // sp_.ratio) * sp_.d_idx * {"bf16": 2, "f32": 4, "e4m3": 1, "fp4": 0.5}[sp_.kc_dtype]
                for L in wl.visible_lengths())
        step_bytes += extra
        score_bytes += extra
    if args.local_blocks:
        if prefill:
            print(json.dumps({"error": "--local-blocks runs the decode workloads"}))
            sys.exit(2)
        pipeline.set_local_blocks(base, args.local_blocks)
        base.score()
        base.topk()
        torch.cuda.synchronize()
        # the union's size depends on the selection: count its tokens
        valid = (base.idx >= 0).sum(dim=1).cpu().numpy()
        tok = [int(v) * spec.ratio + (L - (L // spec.ratio) * spec.ratio)
               for v, L in zip(valid, (int(x) for x in wl.visible_lengths()))]
        step_bytes, attn_bytes, score_bytes = algorithmic_bytes(wl, tok)

    if prefill:
        R = args.replicas or 1      # the score matrix alone (336 MB) exceeds the LLC
    else:
        R = args.replicas or max(2, math.ceil(2 * 256e6 / (step_bytes * max(1, args.layers))) + 1)
    reps = [base]
    for _ in range(R - 1):
        c = pipeline.DeviceProblem(**{**base.__dict__})
        c.K, c.V = base.K.clone(), base.V.clone()
        c.kc = base.kc.clone()
        c.kc_scale = None if base.kc_scale is None else base.kc_scale.clone()
        c.q, c.q_idx, c.w = base.q.clone(), base.q_idx.clone(), base.w.clone()
        if base.ing is not None:
            c.ing = pipeline.IngestState(
                pipeline.KeyRing(base.ing.ring.keys.clone(), base.ing.ring.window.clone()),
                base.ing.k_new.clone(), base.ing.k_row.clone(), base.ing.v_row.clone(),
                base.ing.status.clone())
        reps.append(c)
    torch.cuda.synchronize()

    n_layers = max(1, args.layers)
    stacks = None
    if n_layers > 1:
        if prefill or args.ingest or args.token_pool or args.local_blocks or args.no_graph:
            print(json.dumps({"error": "--layers runs the plain decode step, replayed from a graph"}))
            sys.exit(2)
        gen = torch.Generator(device=dev).manual_seed(spec.seed + 101)

        def fresh(t):
            return torch.randn(t.shape, generator=gen, device=dev, dtype=torch.float32).to(t.dtype)

        def layer_of(p, l):
            c = pipeline.DeviceProblem(**{**p.__dict__})
            c.K, c.V, c.q = fresh(p.K), fresh(p.V), fresh(p.q)
            c.out = torch.zeros_like(p.out)
            if l % args.full_every == 0:
                c.q_idx, c.k_idx = fresh(p.q_idx), fresh(p.k_idx)
                c.w = torch.rand(p.w.shape, generator=gen, device=dev)
                c.kc = p.kc.clone()
                c.kc_scale = None if p.kc_scale is None else p.kc_scale.clone()
                c.scores = torch.zeros_like(p.scores)
                c.idx = p.idx.clone()
                c.compress()
            return c

        stacks = [pipeline.LayerStack([p] + [layer_of(p, l) for l in range(1, n_layers)], args.full_every,
                                      fused=not args.unfused_layers)
                  for p in reps]
        torch.cuda.synchronize()
        n_full = sum(stacks[0].full)
        step_bytes = n_full * score_bytes + n_layers * attn_bytes + (step_bytes - score_bytes - attn_bytes)

    # with --ingest, the append and the canonical scores run as one launch
    # unless --unfused-ingest asks for the two calls
    fuse_ing = bool(args.ingest) and not args.unfused_ingest and not prefill and base.ingest_fusable()

    def ingest(p):
        if p.ing is not None and not fuse_ing:
            p.ingest()

    # scores and their selection as one qsa_index_score_topk call (the
    # scorer writes per-chunk candidate lists, a small finish selects)
    fuse_sel = (not prefill and not fuse_ing and not args.unfused_select and base.select_fusable())
    # a decode step as qsa_decode_step: the scorer writes the lists and each
    # attention workgroup selects its own part from them; timed as the step's
    # two halves (qsa_index_score_lists, qsa_sparse_attn_decode_lists), which
    # launch the same kernels as the one call
    fuse_step = fuse_sel and stacks is None and not args.unfused_step and base.step_fusable()
    # with the append inside the scoring launch, the same two halves
    # (qsa_ingest_index_score_lists, then qsa_sparse_attn_decode_lists)
    fuse_ing_step = fuse_ing and stacks is None and not args.unfused_step and base.ingest_step_fusable()

    def score(p):
        if fuse_ing_step:
            p.ingest_score_lists()
        elif fuse_ing:
            p.ingest_score()
        elif prefill:
            p.score(QSA_SCORE_MFMA)
        elif fuse_step:
            p.score_lists()
        elif fuse_sel:
            p.score_topk()
        else:
            p.score()

    def topk(p):
        if not fuse_sel and not fuse_ing_step:
            p.topk(certified=prefill)

    def attend(p):
        if fuse_step or fuse_ing_step:
            p.attend_lists()
        else:
            p.attend()

    log(f"{workload}: {R} input copies resident; timing {args.steps} steps")
    for s in range(args.warmup):
        p = reps[s % R]
        ingest(p)
        score(p)
        topk(p)
        attend(p)
    torch.cuda.synchronize()

    # events are recorded on torch's current stream, which is the stream
    # every library call below is enqueued on
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        p = reps[s % R]
        e = evs[s]
        e[4].record()
        ingest(p)
        e[0].record()
        score(p)
        e[1].record()
        topk(p)
        e[2].record()
        attend(p)
        e[3].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    eager_ms_step = dt * 1e3 / args.steps
    t_score = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    t_topk = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    t_attn = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    # fused: the append runs inside the scoring launch (its time is in index_score)
    t_ingest = float(np.mean([e[4].elapsed_time(e[0]) for e in evs])) if args.ingest and not fuse_ing else None

    # The whole step captured once per input copy in a HIP graph and replayed:
    # the way a serving loop runs it (no call synchronises or allocates, so
    # the step captures as is).  Kernel times above come from the eager loop.
    graphs = []
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for p in reps:                      # settle lazy initialisation outside capture
                ingest(p)
                score(p)
                topk(p)
                attend(p)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        if stacks is not None:
            with torch.cuda.stream(side):
                for st_ in stacks:
                    st_.step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
        for k_, p in enumerate(reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                if stacks is not None:
                    stacks[k_].step()
                else:
                    ingest(p)
                    score(p)
                    topk(p)
                    attend(p)
            graphs.append(g)
        # The step on every input copy in turn, captured as one graph: the way
        # the step runs inside a larger captured graph (a decode iteration's
        # layers), where one kernel follows another without a graph-launch
        # boundary (measured: about 4 us per boundary between single-step
        # replays).  `value` is timed with it: steps // R replays, then the
        # remaining steps % R steps from the single-step graphs, so exactly
        # `steps` steps in all; the single-step replay time is reported beside
        # it (step_ms.graph_one_step).
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for k_, p in enumerate(reps):
                if stacks is not None:
                    stacks[k_].step()
                else:
                    ingest(p)
                    score(p)
                    topk(p)
                    attend(p)
        for s_ in range(args.warmup):
            graphs[s_ % R].replay()
        g_all.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(args.steps):
            graphs[s_ % R].replay()
        torch.cuda.synchronize()
        one_step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        t0 = time.perf_counter()
        for _ in range(args.steps // R):
            g_all.replay()
        for s_ in range(args.steps % R):
            graphs[s_].replay()
        torch.cuda.synchronize()
        graph_ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
        # the distribution over steps comes from a second pass with an event
        # before every replay (an event record between replays costs a few
        # microseconds itself, so this pass is not the one `value` is from)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        for s_ in range(args.steps):
            marks[s_].record()
            graphs[s_ % R].replay()
        marks[args.steps].record()
        torch.cuda.synchronize()
        per_step = np.array([marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps)])
    else:
        per_step = np.array([e[4].elapsed_time(e[3]) for e in evs])
    ms_step = graph_ms_step if graphs else eager_ms_step
    pct = {"p10": float(np.percentile(per_step, 10)), "p50": float(np.percentile(per_step, 50)),
           "p90": float(np.percentile(per_step, 90)), "mean": float(per_step.mean()),
           "source": ("HIP events between consecutive graph replays (a second pass of the same steps; the "
                      "events add their own cost to each step)") if graphs else "HIP events per eager step"}

    qps = wl.total_q * n_layers / (ms_step / 1e3)
    rec = {
        "metric": "sparse-attn decode queries/s + achieved HBM GB/s (% roofline) at 32K-128K ctx",
        "value": qps, "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{spec.name}", "num_seqs": wl.num_seqs, "queries_per_step": wl.total_q * n_layers,
                   "context": (f"U[{spec.len_range[0]},{spec.len_range[1]}]" if spec.len_range
                               else str(wl.lens[0])),
                   "heads": f"{spec.hq}/{spec.hkv}x{spec.d}", "indexer": f"{spec.h_idx}x{spec.d_idx} {spec.kc_dtype}",
                   "ratio": spec.ratio, "budget": spec.budget, "seed": spec.seed,
                   "input_replicas": R, "score_and_select": "one call" if fuse_sel else "two calls",
                   "selection": ("inside the attention kernel (qsa_decode_step)" if fuse_step else
                                 "inside the attention kernel (qsa_ingest_index_score_lists + "
                                 "qsa_sparse_attn_decode_lists)" if fuse_ing_step else
                                 "own launch" if not prefill else "certified top-k launch"),
                   **({"paged_page_size": args.paged} if args.paged else {}),
                   **({"layers": n_layers, "full_every": args.full_every, "fused_layers": not args.unfused_layers,
                       "layers_with_own_indexer": sum(stacks[0].full)} if stacks is not None else {}),
                   **({"local_blocks": args.local_blocks} if args.local_blocks else {}),
                   **({"token_pool": args.token_pool} if args.token_pool else {}),
                   **({"ingest": "one token per sequence", "ingest_fused_with_scores": fuse_ing,
                       "ring_capacity": int(base.ing.ring.keys.shape[1])} if args.ingest else {})},
        "step_ms_percentiles": pct,
        "kernel_ms": {**({"ingest_index_score_lists": t_score, "sparse_attn_select": t_attn} if fuse_ing_step else
                         {"index_score_lists": t_score, "sparse_attn_select": t_attn} if fuse_step else
                         {"index_score_topk": t_score, "sparse_attn": t_attn} if fuse_sel else
                         {"index_score": t_score, "topk": t_topk, "sparse_attn": t_attn}),
                      **({"ingest": t_ingest} if t_ingest is not None else {})},
        "step_ms": {"graph": graph_ms_step if graphs else None,
                    "graph_one_step": one_step_ms if graphs else None, "eager": eager_ms_step},
        "compress_ms": compress_ms,
    }
    if prefill:
        f_idx, f_attn = prefill_flops(wl)
        # every query gathers its own token set, so the launch moves its
        # algorithmic bytes (34 GB for 84 MB of distinct K/V) through L2: the
        # bound is the L2's bandwidth (counters: profiles/
        # prefill_indexer_mfma_and_gather_l2_counters.md)
        gbps = attn_bytes / (t_attn * 1e-3) / 1e9
        rec["roofline"] = {"bound": "l2", "achieved": gbps, "peak": L2_PEAK_GBPS, "unit": "GB/s",
                           "frac": gbps / L2_PEAK_GBPS, "traffic": None,
                           "kernel": "qsa_sparse_attn_prefill (causal gather attention)",
                           "bytes_per_launch": attn_bytes, "avg_ms": t_attn}
        ach = f_attn / (t_attn * 1e-3) / 1e12
        # QK and PV run on the bf16 matrix cores (PV as two bf16 terms of the
        # probabilities, counted once here)
        rec["mfma_attention"] = {"tflops": ach, "peak": MFMA_BF16_PEAK_TFLOPS, "util": ach / MFMA_BF16_PEAK_TFLOPS,
                                 "flops_per_launch": f_attn}
        mf = f_idx / (t_score * 1e-3) / 1e12
        rec["mfma_indexer"] = {"tflops": mf, "peak": MFMA_BF16_PEAK_TFLOPS,
                               "util": mf / MFMA_BF16_PEAK_TFLOPS, "flops_per_launch": f_idx,
                               "avg_ms": t_score}
    else:
        attn_gbps = attn_bytes / (t_attn * 1e-3) / 1e9
        traffic = None if (args.paged or args.kc_dtype or args.budget or args.local_blocks
                           or args.token_pool) else recorded_traffic(spec.name)
        rec["roofline"] = {"bound": "hbm", "achieved": attn_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": attn_gbps / HBM_PEAK_GBPS, "traffic": traffic,
                           "kernel": ("qsa_sparse_attn_decode_lists (per-part selection from the candidate "
                                      "lists + gather attention + split combine)" if fuse_step or fuse_ing_step else
                                      "qsa_sparse_attn_decode (gather attention + split combine)"),
                           "bytes_per_launch": attn_bytes, "avg_ms": t_attn}
        rec["step_hbm_gbps"] = step_bytes / (ms_step * 1e-3) / 1e9
        rec["step_hbm_frac"] = rec["step_hbm_gbps"] / HBM_PEAK_GBPS
        rec["step_bytes"] = step_bytes
        rec["index_score_gbps"] = score_bytes / (t_score * 1e-3) / 1e9
    if args.ingest:
        torch.cuda.synchronize()
        ok = all(bool((p.ing.status == 0).all()) for p in reps)
        if not ok:
            print(json.dumps({"error": "ingest reported a non-zero status"}))
            sys.exit(1)
    if cpu:
        log(f"{workload}: oracle baseline on the host cores")
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, prefill)
    return rec


if __name__ == "__main__":
    main()
