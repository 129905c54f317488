"""GPU parity: every entry point through the C ABI vs the CPU oracle.

Compressed keys, canonical scores and selected block indices must match bit
for bit; attention outputs must be within the stated tolerance of the fp64
oracle.  Small cases span several workgroup tiles and ragged tails; the
full-size cases use the benchmark's launch configuration and compare sampled
queries.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import qsa_workloads as W
from tests.parity import check_idx, check_out, full_check, gpu_available, run_gpu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _print(*a):
    print(*a, flush=True)


# ------------------------------------------------------------ small cases
SMALL = [
    # (spec, lens, n_q or None, overrides)
    ("tiny", W.TINY_DECODE, [4096], None, {}),
    ("tiny_ragged", W.TINY_DECODE, [1027, 4099, 333, 2], None, {"budget": 256}),
    ("batched_small", W.BATCHED_DECODE, [3001, 1234, 777, 5002, 2049, 2052], None, {}),
    ("batched_budget64", W.BATCHED_DECODE, [1500, 903, 64, 65, 3], None, {"budget": 64}),
    ("long_small_e4m3", W.LONG_DECODE, [6001, 3003, 1000], None, {"budget": 512}),
    ("long_small_fp4", W.LONG_DECODE, [6001, 3003, 1000, 37], None, {"budget": 512, "kc_dtype": "fp4"}),
    # budget/ratio = 2048: dense up to L = 8195, sparse from 8196
    ("long_k2048", W.LONG_DECODE, [20000, 9000, 8195, 8196, 700], None, {"budget": 8192}),
    ("batched_k2048", W.BATCHED_DECODE, [30001, 8196, 12000], None, {"budget": 8192}),
    ("prefill_small", W.CHUNKED_PREFILL, [1500], [300], {"budget": 256}),
    ("verify_small", W.VERIFY, [2044, 2050, 2051, 2052, 2055, 2064], None, {}),
    ("verify_full_shape", W.VERIFY, None, None, {}),
]


@pytest.mark.parametrize("name,spec,lens,nq,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_configs(name, spec, lens, nq, over):
    sp = dataclasses.replace(spec, **over) if over else spec
    wl = W.make(sp, lens=lens, n_q=nq, seed=sp.seed + 100)
    _print(f"[parity] {name}: lens={wl.lens[:6]} n_q={wl.n_q[:6]} budget={sp.budget}")
    _, _, worst = full_check(wl)
    _print(f"[parity] {name}: ok, worst err/limit = {worst:.3f}")


DTYPES = [
    ("q_f32_kc_f32", "f32", "f32", "f32"),
    ("q_bf16_kc_bf16", "bf16", "bf16", "bf16"),
    ("q_bf16_kc_e4m3", "bf16", "bf16", "e4m3"),
    ("q_f32_kc_e4m3", "f32", "f32", "e4m3"),
    ("q_bf16_kc_f32", "bf16", "bf16", "f32"),
    ("q_f32_kc_bf16", "f32", "f32", "bf16"),
    ("q_bf16_kc_fp4", "bf16", "bf16", "fp4"),
]


@pytest.mark.parametrize("name,kv,idx_dt,kc_dt", DTYPES, ids=[d[0] for d in DTYPES])
# (heads, dims): query rows of 2 to 64 (chunk, head) steps, so every load
# count of the scorer's vector query path (one partial load, 1, 2, 4 and 8
# loads) and its scalar path (64 steps) meet the oracle
@pytest.mark.parametrize("h_idx,d_idx", [(1, 64), (2, 64), (2, 128), (4, 64), (4, 128), (8, 128), (16, 64),
                                         (16, 128)])
def test_indexer_dtype_and_shape_matrix(name, kv, idx_dt, kc_dt, h_idx, d_idx):
    sp = dataclasses.replace(W.BATCHED_DECODE, kv_dtype=kv, idx_dtype=idx_dt, kc_dtype=kc_dt, h_idx=h_idx,
                             d_idx=d_idx, hq=8, hkv=2, budget=128)
    wl = W.make(sp, lens=[900, 517, 131], seed=7)
    full_check(wl)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 4), (32, 4), (32, 2)])
@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_gqa_group_sizes(hq, hkv, kv):
    sp = dataclasses.replace(W.BATCHED_DECODE, hq=hq, hkv=hkv, kv_dtype=kv, budget=256)
    wl = W.make(sp, lens=[1400, 77, 2100], seed=11)
    full_check(wl)


@pytest.mark.parametrize("ratio", [1, 2, 8, 16, 64])
def test_other_ratios(ratio):
    sp = dataclasses.replace(W.BATCHED_DECODE, ratio=ratio, budget=64 * ratio, hq=8, hkv=1)
    wl = W.make(sp, lens=[64 * ratio * 3 + ratio - 1, 100, ratio * 70 + 1], seed=13)
    full_check(wl)


def test_prefill_ragged_chunks_and_empty_sequence():
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=128)
    wl = W.make(sp, lens=[700, 300, 90, 1025], n_q=[33, 0, 90, 1], seed=17)
    full_check(wl)


def test_equal_scores_pick_lowest_blocks():
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=256)
    wl = W.make(sp, lens=[4000, 2000], seed=19)
    wl.q_idx.zero_()                       # every score is +0: ties everywhere
    res, ref, _ = full_check(wl)
    assert np.array_equal(res["idx"][0], np.arange(64))
    assert np.array_equal(res["idx"][1], np.arange(64))


def test_nonpositive_scores_with_some_ties():
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=512)
    wl = W.make(sp, lens=[6000, 3001], seed=23)
    # half of the indexer heads get no weight, making many scores exactly 0
    wl.w[:, ::2] = 0.0
    full_check(wl)


def test_decode_equals_prefill_row_and_two_chunks_equal_one():
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=256)
    wl = W.make(sp, lens=[2500], n_q=[40], seed=29)
    res_all, _ = run_gpu(wl)
    # the same sequence as two chunks: the first 17 queries, then the rest
    a = dataclasses.replace(wl)
    cut = 17
    first = W.Workload(sp, [wl.lens[0] - (40 - cut)], [cut], np.array([0, wl.lens[0] - 23]),
                       np.array([0, cut]), wl.K[: wl.lens[0] - 23], wl.V[: wl.lens[0] - 23],
                       wl.k_idx[: wl.lens[0] - 23], wl.q[:cut], wl.q_idx[:cut], wl.w[:cut])
    second = W.Workload(sp, wl.lens, [40 - cut], wl.kv_offsets, np.array([0, 40 - cut]),
                        wl.K, wl.V, wl.k_idx, wl.q[cut:], wl.q_idx[cut:], wl.w[cut:])
    r1, _ = run_gpu(first)
    r2, _ = run_gpu(second)
    assert np.array_equal(np.concatenate([r1["idx"], r2["idx"]]), res_all["idx"])
    assert np.array_equal(np.concatenate([r1["out"], r2["out"]]), res_all["out"])
    # the last query alone, as a decode batch: same selection bits; the
    # decode entry point splits the blocks (its output is not bit-identical
    # to the prefill row), so its output is held to the oracle at the stated
    # tolerance, like every other output
    last = W.Workload(sp, wl.lens, [1], wl.kv_offsets, np.array([0, 1]), wl.K, wl.V, wl.k_idx,
                      wl.q[39:], wl.q_idx[39:], wl.w[39:])
    r3, _ = run_gpu(last, decode=True)
    assert np.array_equal(r3["idx"][0], res_all["idx"][39])
    ref_last = oracle.run_workload(last)
    check_idx(r3, ref_last, [0])
    check_out(last, r3, ref_last, [0])
    ref_all = oracle.run_workload(wl)
    check_idx(res_all, ref_all, np.arange(wl.total_q))
    check_out(wl, res_all, ref_all, np.arange(wl.total_q))
    del a


# ------------------------------------------------------------ full sizes
def _sample(total, k, seed=0):
    rng = np.random.default_rng(seed)
    pick = set([0, total - 1]) | set(rng.choice(total, min(k, total), replace=False).tolist())
    return np.array(sorted(pick), dtype=np.int64)


@pytest.mark.parametrize("cfg", ["tiny_decode", "batched_decode", "verify"])
def test_full_size_all_queries(cfg):
    wl = W.make(W.CONFIGS[cfg])
    _print(f"[parity] full {cfg}: B={wl.num_seqs} total_q={wl.total_q} max_len={max(wl.lens)}")
    _, _, worst = full_check(wl)
    _print(f"[parity] full {cfg}: ok, worst err/limit = {worst:.3f}")


def test_full_size_long_context_e4m3():
    wl = W.make(W.LONG_DECODE)
    _print(f"[parity] full long decode: B={wl.num_seqs} len={wl.lens[0]}")
    _, _, worst = full_check(wl)
    _print(f"[parity] full long decode: ok, worst err/limit = {worst:.3f}")


def test_full_size_chunked_prefill_all_queries():
    # all 8193 queries of the chunk: compressed keys, every canonical score,
    # every selection and every output against the oracle
    wl = W.make(W.CHUNKED_PREFILL)
    _print(f"[parity] full chunked prefill: total_q={wl.total_q}, every query")
    _, _, worst = full_check(wl)
    _print(f"[parity] full chunked prefill: ok, worst err/limit = {worst:.3f}")


@pytest.mark.parametrize("n", [255, 256, 257])
def test_decode_batches_at_the_scorer_row_limit(n):
    # decode batches of up to 256 rows score only their visible 256-block
    # groups, each wave finding its (row, group) from the offsets of four rows
    # per lane; 257 rows keep the dense (row, group) grid.  The rows mix no
    # complete block, exact multiples of 256 blocks, one block past them and
    # ragged lengths, so rows without groups sit between others.  Scores are
    # first set to NaN, so a group that no workgroup scored shows in the bits.
    from indexer_selected_sparse_amd import pipeline
    from tests.parity import check_scores
    sp = dataclasses.replace(W.BATCHED_DECODE, hq=8, hkv=2, budget=64)
    rng = np.random.default_rng(40 + n)
    pick = [1, 3, 4 * 256, 4 * 256 + 3, 4 * 256 + 4, 4 * 512, 4 * 768 + 2]
    lens = [int(pick[j % len(pick)]) if j % 3 else int(rng.integers(1, 7000)) for j in range(n)]
    wl = W.make(sp, lens=lens, seed=40 + n)
    dp = pipeline.upload(wl, "cuda")
    dp.compress()
    dp.scores.fill_(float("nan"))
    dp.idx.fill_(-9)
    dp.step()
    torch.cuda.synchronize()
    q = np.arange(wl.total_q)
    ref = oracle.run_workload(wl, want_scores=True)
    res = {"scores": dp.scores.cpu().numpy(), "idx": dp.idx.cpu().numpy(),
           "out": dp.out.float().cpu().numpy().astype(np.float64)}
    check_scores(wl, res, ref, q)
    check_idx(res, ref, q)
    check_out(wl, res, ref, q)
    _print(f"[parity] {n} decode rows: ok")


@pytest.mark.parametrize("ratio", [4, 8])
@pytest.mark.parametrize("kc_dtype", ["bf16", "e4m3", "fp4"])
def test_compress_from_first_block(ratio, kc_dtype):
    # qsa_compress_keys with first_block: blocks before first_block[s] keep
    # what they held, the rest equal the oracle's.  Ratio 4 takes the kernel
    # whose waves request all rows of their four blocks together (blocks
    # before the start, or past the row's end, are read in place of a block
    # that exists and are not stored); ratio 8 the runtime-ratio loop.  The
    # starts fall on a wave's first block, inside a wave, at the row's end
    # and past it.
    import indexer_selected_sparse_amd as Q
    from indexer_selected_sparse_amd import pipeline
    sp = dataclasses.replace(W.BATCHED_DECODE, ratio=ratio, budget=64 * ratio, kc_dtype=kc_dtype, hq=8, hkv=1)
    lens = [ratio * 37 + 3, ratio * 16, ratio * 5 + 1, ratio * 70 + ratio - 1, 2, ratio * 9]
    starts = [0, 4, 6, 17, 0, 9]
    wl = W.make(sp, lens=lens, seed=44 + ratio)
    dp = pipeline.upload(wl, "cuda")
    kc_u8 = dp.kc.view(torch.uint8)
    kc_u8.fill_(0x5A)
    if dp.kc_scale is not None:
        dp.kc_scale.view(torch.uint8).fill_(0x3C)
    rows = dp.kc.shape[0]
    before = kc_u8.cpu().numpy().copy()
    sc_u8 = None if dp.kc_scale is None else dp.kc_scale.view(torch.uint8).reshape(rows, -1)
    sc_before = None if sc_u8 is None else sc_u8.cpu().numpy().copy()
    fb = torch.tensor(starts, dtype=torch.int64, device="cuda")
    Q.compress_keys(dp.k_idx, ratio, dp.batch, dp.kc, dp.kc_scale, first_block=fb)
    torch.cuda.synchronize()
    got = kc_u8.cpu().numpy()
    sc_got = None if sc_u8 is None else sc_u8.cpu().numpy()
    ref_kc, ref_sc = oracle.compress(wl.k_idx.float().numpy(), wl.kv_offsets, ratio, kc_dtype)
    ref_u8 = np.ascontiguousarray(ref_kc).view(np.uint8).reshape(ref_kc.shape[0], -1)
    ref_sc_u8 = None if ref_sc is None else np.ascontiguousarray(ref_sc).view(np.uint8).reshape(ref_kc.shape[0], -1)
    row = 0
    for s, L in enumerate(lens):
        for b in range(L // ratio):
            if b < starts[s]:
                assert np.array_equal(got[row], before[row]), f"seq {s} block {b} (before the start) was written"
                if sc_got is not None:
                    assert np.array_equal(sc_got[row], sc_before[row]), f"seq {s} block {b}: scale written"
            else:
                assert np.array_equal(got[row], ref_u8[row]), f"seq {s} block {b}: kc differs from the oracle"
                if sc_got is not None:
                    assert np.array_equal(sc_got[row], ref_sc_u8[row]), f"seq {s} block {b}: scale differs"
            row += 1
    assert row == ref_kc.shape[0]
    _print(f"[parity] compress from first_block, ratio {ratio} {kc_dtype}: ok ({row} blocks)")


def test_batch_without_queries_writes_nothing():
    # a prefill batch whose sequences append no queries (total_q = 0): every
    # call succeeds, launches nothing that writes, and leaves its outputs as
    # they were (one sentinel row each)
    import indexer_selected_sparse_amd as Q
    from indexer_selected_sparse_amd import pipeline
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=256)
    wl = W.make(sp, lens=[1500, 300], n_q=[4, 2], seed=45)
    dp = pipeline.upload(wl, "cuda")
    dp.compress()
    b = dp.batch
    zero_q = torch.zeros(len(wl.lens) + 1, dtype=torch.int64, device="cuda")
    empty = Q.Batch(b.kv_offsets, b.blk_offsets, zero_q, 0, b.max_kv_len, 1)
    K = sp.budget // sp.ratio
    scores = torch.full((1, dp.scores.shape[1]), 7.0, dtype=torch.float32, device="cuda")
    idx = torch.full((1, K), 5, dtype=torch.int32, device="cuda")
    out = torch.full((1,) + tuple(dp.out.shape[1:]), 3.0, dtype=dp.out.dtype, device="cuda")
    Q.index_score(dp.q_idx, dp.w, dp.kc, dp.kc_scale, dp.ratio, empty, scores)
    tws = torch.empty(max(Q.topk_workspace_size(empty, sp.budget, sp.ratio), 1), dtype=torch.uint8, device="cuda")
    Q.topk_blocks(scores, sp.budget, sp.ratio, empty, idx, ws=tws)
    sws = torch.empty(max(Q.score_topk_workspace_size(empty, sp.budget, sp.ratio), 1), dtype=torch.uint8,
                      device="cuda")
    Q.index_score_topk(dp.q_idx, dp.w, dp.kc, dp.kc_scale, sp.budget, sp.ratio, empty, scores, idx, sws)
    Q.sparse_attn_prefill(dp.q, dp.K, dp.V, dp.softmax_scale, idx, sp.budget, sp.ratio, empty, out)
    torch.cuda.synchronize()
    assert bool((scores == 7.0).all()) and bool((idx == 5).all()) and bool((out.float() == 3.0).all())


def test_decode_workspace_reused_across_batch_shapes():
    # one decode workspace shared by batches of different shapes, used
    # alternately: each shape must reproduce its first result bit for bit
    # (the workspace carries no state between calls)
    from indexer_selected_sparse_amd import pipeline
    big = W.make(W.BATCHED_DECODE, lens=[9000 + 997 * j for j in range(24)], seed=31)
    small = W.make(dataclasses.replace(W.LONG_DECODE, kc_dtype="bf16"), lens=[20000, 12000, 30001], seed=32)
    dps = [pipeline.upload(wl, "cuda") for wl in (big, small)]
    ws = torch.zeros(max(dp.attn_ws.numel() for dp in dps), dtype=torch.uint8, device="cuda")
    for dp in dps:
        dp.attn_ws = ws
        dp.compress()
    outs = []
    for rnd in range(3):
        for k, dp in enumerate(dps):
            dp.step()
            torch.cuda.synchronize()
            o = dp.out.clone()
            if rnd == 0:
                outs.append(o)
            else:
                assert torch.equal(o, outs[k]), f"round {rnd} batch {k} differs"
    for wl, o in zip((big, small), outs):
        ref = oracle.run_workload(wl, query_ids=np.arange(min(wl.total_q, 4)))
        from tests.parity import check_out
        check_out(wl, {"out": o.float().cpu().numpy().astype(np.float64)}, ref, np.arange(min(wl.total_q, 4)))


def test_graph_replays_match_eager():
    # the whole decode step captured in a HIP graph and replayed several
    # times, with eager work and synchronisation between replays
    from indexer_selected_sparse_amd import pipeline
    wl = W.make(W.BATCHED_DECODE, lens=[8200 + 1711 * j for j in range(12)], seed=33)
    dp = pipeline.upload(wl, "cuda")
    dp.compress()
    dp.step()
    torch.cuda.synchronize()
    eager = (dp.scores.clone(), dp.idx.clone(), dp.out.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dp.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dp.step()
    for rep in range(4):
        dp.scores.fill_(-1.0)
        dp.idx.fill_(-5)
        dp.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # scores past a row's visible blocks are left untouched by design
        nbs = [int(L) // wl.spec.ratio for L in wl.visible_lengths()]
        for r, nb in enumerate(nbs):
            assert torch.equal(dp.scores[r, :nb], eager[0][r, :nb]), f"replay {rep}: scores row {r}"
        assert torch.equal(dp.idx, eager[1]), f"replay {rep}: idx differs from the eager step"
        assert torch.equal(dp.out, eager[2]), f"replay {rep}: out differs from the eager step"
        dp.step()                       # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("budget", [2048, 8192])
def test_maximum_row_length(budget):
    # the longest row the library accepts: 131072 complete blocks (plus a
    # ragged tail of 3 tokens), with K = 512 and K = 2048
    sp = dataclasses.replace(W.LONG_DECODE, hq=8, hkv=1, budget=budget)
    wl = W.make(sp, lens=[4 * 131072 + 3], seed=91)
    _print(f"[parity] max row: L={wl.lens[0]} budget={budget}")
    full_check(wl)
