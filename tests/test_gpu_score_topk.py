"""qsa_index_score_topk (canonical scores and their block top-k in one call,
selecting from the scorer's per-chunk candidate lists when a certificate
allows) against the oracle and against the two separate calls.

Scores and indices must match the oracle bit for bit on every row, whether
the row was selected from its lists or from its whole score row.  The rows
below are built so that both happen: independent scores (the lists
suffice), winners clustered in a few chunks, all-equal scores and duplicated
keys (the certificate fails and the row falls back), ties at the threshold
spread over chunks, negative weights, K = 2048 and the longest rows.  Which
path each row takes is computed on the host from the oracle's scores with
the lists' rule (`_certified`), so the tests know that both paths ran.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import indexer_selected_sparse_amd as Q
import oracle
import qsa_workloads as W
from indexer_selected_sparse_amd import pipeline
from tests.parity import check_compress, check_idx, check_out, check_scores, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _list_len(nb, K):
    m = -(-64 * K // nb)
    s = 0
    while s * s < m:
        s += 1
    return min(64, m + 4 * s + 3)


def _keys(row):
    u = np.asarray(row, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return np.where(u & 0x80000000, (~u) & 0xffffffff, u | 0x80000000)


def _certified(row, K):
    """Whether the lists certify this row's selection (None: dense regime)."""
    nb = len(row)
    if nb <= K:
        return None
    keys = _keys(row)
    kk = _list_len(nb, K)
    listed, mcut = [], 0
    for c in range(0, nb, 64):
        seg = keys[c:c + 64]
        order = np.lexsort((np.arange(len(seg)), -seg.astype(np.int64)))
        top = seg[order[:kk]]
        listed.extend(top.tolist())
        if len(seg) > kk:
            mcut = max(mcut, int(top[-1]))
    if len(listed) < K:
        return False
    T = sorted(listed, reverse=True)[K - 1]
    return T > 0 and mcut < T


def _run(wl, paged=0):
    dp = pipeline.upload(wl, "cuda")
    dp.compress()
    if paged:
        dp = pipeline.page(dp, wl.lens, paged, seed=7, extra_pages=2)
    dp.scores.fill_(float("nan"))
    dp.idx.fill_(-9)
    dp.score_topk()
    torch.cuda.synchronize()
    got = {"scores": dp.scores.cpu().numpy(), "idx": dp.idx.cpu().numpy()}
    # the two separate calls on the same inputs
    sc2 = torch.full_like(dp.scores, float("nan"))
    idx2 = torch.full_like(dp.idx, -9)
    Q.index_score(dp.q_idx, dp.w, dp.kc, dp.kc_scale, dp.ratio, dp.batch, sc2, paging=dp.paging)
    Q.topk_blocks(sc2, dp.budget, dp.ratio, dp.batch, idx2, ws=dp.topk_ws_canon)
    torch.cuda.synchronize()
    return dp, got, sc2.cpu().numpy(), idx2.cpu().numpy()


def _check(wl, paged=0, expect=None):
    sp = wl.spec
    dp, got, sc2, idx2 = _run(wl, paged)
    q = np.arange(wl.total_q)
    ref = oracle.run_workload(wl, want_scores=True, want_out=False)
    check_scores(wl, got, ref, q)
    check_idx(got, ref, q)
    assert np.array_equal(got["idx"], idx2), "combined call and separate calls select differently"
    K = sp.budget // sp.ratio
    paths = [_certified(ref["scores"][i], K) for i in q]
    n_lists = sum(p is True for p in paths)
    n_fall = sum(p is False for p in paths)
    print(f"[score_topk] rows={len(q)} lists={n_lists} fallback={n_fall} dense={len(q) - n_lists - n_fall}",
          flush=True)
    if expect == "lists":
        assert n_lists > 0 and n_fall == 0, paths
    elif expect == "fallback":
        assert n_fall > 0, paths
    elif expect == "both":
        assert n_lists > 0 and n_fall > 0, paths
    return dp, ref, paths


@pytest.mark.parametrize("kc_dtype", ["bf16", "e4m3", "fp4"])
def test_independent_scores_take_the_lists(kc_dtype):
    sp = dataclasses.replace(W.BATCHED_DECODE, kc_dtype=kc_dtype)
    rng = np.random.default_rng(11)
    lens = [int(x) for x in rng.integers(2100, 33000, 24)] + [2051, 2052, 4096 * 4 + 3]
    _check(W.make(sp, lens=lens, seed=501), expect="lists")


def test_long_rows_e4m3_and_paged():
    sp = dataclasses.replace(W.LONG_DECODE, hq=8, hkv=1)
    wl = W.make(sp, lens=[131072, 99999, 65536 + 5], seed=502)
    _check(wl, expect="lists")
    _check(wl, paged=256, expect="lists")


def test_fp32_operands_take_the_rounded_scorer():
    wl = W.make(dataclasses.replace(W.TINY_DECODE, budget=1024), lens=[4096, 9000, 5000], seed=503)
    _check(wl, expect="lists")


def test_clustered_winners_fall_back():
    # blocks of one token range get keys four times larger: their scores beat
    # almost everything, so a few chunks hold more winners than their lists
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=2048)
    wl = W.make(sp, lens=[20000, 9000, 30001, 4000], seed=504)
    a = int(wl.kv_offsets[0]) + 4 * 3000
    wl.k_idx[a:a + 4 * 300] *= 4.0
    b = int(wl.kv_offsets[2]) + 4 * 7000
    wl.k_idx[b:b + 4 * 700] *= 4.0
    _, _, paths = _check(wl, expect="both")
    assert paths[0] is False and paths[2] is False


def test_all_equal_scores_fall_back_to_lowest_blocks():
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=1024)
    wl = W.make(sp, lens=[6000, 3001], seed=505)
    wl.q_idx.zero_()
    dp, ref, _ = _check(wl, expect="fallback")
    assert np.array_equal(dp.idx.cpu().numpy()[0], np.arange(256))


def test_duplicated_keys_give_ties_across_chunks():
    # the second half of every row repeats the first half's raw keys, so
    # every score occurs twice, 64-block chunks apart: the threshold is a tie
    # shared by two chunks, and the lower block must win
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=512)
    lens = [4 * 2 * 1000 + 1, 4 * 2 * 3000, 4 * 2 * 700 + 2]
    wl = W.make(sp, lens=lens, seed=506)
    for s, n in enumerate(lens):
        a = int(wl.kv_offsets[s])
        half = 4 * (n // 8)
        wl.k_idx[a + half:a + 2 * half] = wl.k_idx[a:a + half]
    _check(wl)


def test_negative_weights():
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=1024)
    wl = W.make(sp, lens=[9000, 15000, 5002], seed=507)
    wl.w[:, 1::2] *= -1.0
    _check(wl)


def test_k2048_rows():
    sp = dataclasses.replace(W.LONG_DECODE, hq=8, hkv=1, budget=8192)
    wl = W.make(sp, lens=[131072 + 3, 40000, 8196, 8195], seed=508)
    _check(wl)


def test_many_rows_take_the_plain_launches():
    # more than 256 query rows: the scores and the single-workgroup top-k
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=256)
    wl = W.make(sp, lens=[3000, 2500], n_q=[200, 150], seed=509)
    _check(wl)


def test_full_batched_decode_step_and_outputs():
    # the benchmark's workload: the combined call inside the decode step,
    # outputs against the oracle too
    wl = W.make(W.BATCHED_DECODE)
    dp, ref, paths = _check(wl, expect="lists")
    dp.attend()
    torch.cuda.synchronize()
    refo = oracle.run_workload(wl)
    check_out(wl, {"out": dp.out.float().cpu().numpy().astype(np.float64)}, refo, np.arange(wl.total_q))
