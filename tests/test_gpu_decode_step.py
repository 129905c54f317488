"""qsa_decode_step (scores, selection inside the attention kernel, attention)
against the oracle and against the separate calls.

Scores and idx must match the oracle bit for bit and the outputs lie within
the stated tolerance; moreover idx and the outputs must equal, bit for bit,
qsa_index_score_topk followed by qsa_sparse_attn_decode on the same batch
(same kernels, same split of each query's blocks), and the two halves
(qsa_index_score_lists, qsa_sparse_attn_decode_lists) must equal the one call.
The cases reach every way the attention workgroups select: from the lists,
from the whole score row when the certificate fails (clustered winners,
all-equal scores) or the lists exceed the workgroup's LDS (K = 2048 on long
rows), the dense regime and rows with no complete block, paged caches, every
key format, and the batches that run the separate kernels instead (fp32 K/V,
more than 256 queries).
"""
import dataclasses

import numpy as np
import pytest
import torch

import indexer_selected_sparse_amd as Q
import oracle
import qsa_workloads as W
from indexer_selected_sparse_amd import pipeline
from tests.parity import check_idx, check_out, check_scores, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _print(*a):
    print(*a, flush=True)


def _bits(t):
    t = t.detach().contiguous()
    return t.view(torch.int16) if t.dtype in (torch.bfloat16,) else t.view(torch.int32)


def _run(wl, paged=0, oracle_check=True):
    dp = pipeline.upload(wl, "cuda", decode=True)
    dp.compress()
    if paged:
        dp = pipeline.page(dp, wl.lens, paged, seed=5, extra_pages=2)
    dp.scores.fill_(float("nan"))
    dp.idx.fill_(-9)
    dp.out.zero_()
    dp.decode_step()
    torch.cuda.synchronize()
    got = {"scores": dp.scores.cpu().numpy(), "idx": dp.idx.cpu().numpy(),
           "out": dp.out.float().cpu().numpy().astype(np.float64)}
    fused_out = dp.out.clone()
    # the separate calls on the same inputs
    sc2 = torch.full_like(dp.scores, float("nan"))
    idx2 = torch.full_like(dp.idx, -9)
    out2 = torch.zeros_like(dp.out)
    Q.index_score_topk(dp.q_idx, dp.w, dp.kc, dp.kc_scale, dp.budget, dp.ratio, dp.batch, sc2, idx2, dp.sel_ws,
                       paging=dp.paging)
    Q.sparse_attn_decode(dp.q, dp.K, dp.V, dp.softmax_scale, idx2, dp.budget, dp.ratio, dp.batch, out2, dp.attn_ws,
                         paging=dp.paging)
    # the two halves
    sc3 = torch.full_like(dp.scores, float("nan"))
    idx3 = torch.full_like(dp.idx, -9)
    out3 = torch.zeros_like(dp.out)
    Q.index_score_lists(dp.q_idx, dp.w, dp.kc, dp.kc_scale, dp.q, dp.K, dp.V, dp.softmax_scale, dp.budget,
                        dp.ratio, dp.batch, sc3, dp.step_ws, paging=dp.paging)
    Q.sparse_attn_decode_lists(dp.q, dp.K, dp.V, dp.softmax_scale, dp.budget, dp.ratio, dp.batch, sc3, idx3, out3,
                               dp.step_ws, paging=dp.paging)
    torch.cuda.synchronize()
    assert torch.equal(dp.idx, idx2), "decode step and separate calls select differently"
    assert torch.equal(_bits(fused_out), _bits(out2)), "decode step output differs from the separate calls"
    assert torch.equal(dp.idx, idx3) and torch.equal(_bits(fused_out), _bits(out3)), "halves differ"
    if oracle_check:
        q = np.arange(wl.total_q)
        ref = oracle.run_workload(wl, want_scores=True)
        check_scores(wl, got, ref, q)
        check_idx(got, ref, q)
        worst = check_out(wl, got, ref, q)
        _print(f"[decode_step] {wl.spec.name} lens={list(wl.lens)[:4]}...: oracle ok, worst err/limit {worst:.3f}")
    return dp


def test_batched_decode_full_size():
    _run(W.make(W.BATCHED_DECODE))


def test_long_decode_full_size():
    _run(W.make(W.LONG_DECODE))


@pytest.mark.parametrize("kc_dtype", ["bf16", "e4m3", "fp4"])
def test_key_formats_and_ragged_rows(kc_dtype):
    sp = dataclasses.replace(W.BATCHED_DECODE, kc_dtype=kc_dtype, budget=512)
    _run(W.make(sp, lens=[9001, 2051, 2, 530, 518, 4099, 20002, 3], seed=601))


def test_shorter_rows_list_more_than_the_longest():
    # each attention workgroup requests, before its row's length is known,
    # the most entries any row of at most max_kv_len tokens can list.  At
    # K = 512 the longest row here (8292 blocks) lists 1950 entries, while
    # rows of 8191 and 8190 blocks list 2560 (20 per chunk against 15), the
    # most of any length up to 8292: they fill the request exactly, and a
    # request sized by the longest row would cut off their last chunks
    _run(W.make(W.BATCHED_DECODE, lens=[4 * 8292, 4 * 8191 + 3, 4 * 8190, 4 * 6554, 4 * 6553 + 1, 20000],
                seed=609))


def test_loose_max_kv_len_gives_the_same_step():
    # max_kv_len is only the host's bound on the lengths: it sizes the
    # scorer's grid (a slot per 256-block group of a row that long), the
    # lists' row stride and the entries each attention workgroup requests
    # before its row's length is known.  Four times the longest row must give
    # the same scores, selection and outputs bit for bit; at that bound
    # (31000 blocks) a row could list 6305 entries, so the attention also
    # switches from the 4-group to the 8-group register selection.
    wl = W.make(W.BATCHED_DECODE, lens=[9001, 20000, 4097, 31000, 2051, 100, 7750 * 4], seed=610)
    dp = pipeline.upload(wl, "cuda", decode=True)
    dp.compress()
    dp.scores.fill_(float("nan"))
    dp.decode_step()
    torch.cuda.synchronize()
    b = dp.batch
    loose = Q.Batch(b.kv_offsets, b.blk_offsets, b.q_offsets, b.total_q, 4 * b.max_kv_len, b.max_q_per_seq)
    ld = -(-loose.max_kv_len // dp.ratio)
    sc2 = torch.full((b.total_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    idx2 = torch.full_like(dp.idx, -9)
    out2 = torch.zeros_like(dp.out)
    ws2 = torch.empty(max(Q.decode_step_workspace_size(dp.q, dp.K, dp.V, dp.softmax_scale, dp.budget, dp.ratio,
                                                       loose), 1), dtype=torch.uint8, device="cuda")
    Q.decode_step(dp.q_idx, dp.w, dp.kc, dp.kc_scale, dp.q, dp.K, dp.V, dp.softmax_scale, dp.budget, dp.ratio,
                  loose, sc2, idx2, out2, ws2)
    torch.cuda.synchronize()
    for r, L in enumerate(wl.lens):
        nb = L // dp.ratio
        assert torch.equal(_bits(sc2[r, :nb]), _bits(dp.scores[r, :nb])), f"row {r}: scores differ"
    assert torch.equal(idx2, dp.idx), "selection differs under the loose bound"
    assert torch.equal(_bits(out2), _bits(dp.out)), "outputs differ under the loose bound"
    _print(f"[decode_step] loose max_kv_len {loose.max_kv_len} (tight {b.max_kv_len}): identical")


def test_no_row_holds_a_complete_block():
    # every row shorter than one block: no scores, no lists (the scorer's grid
    # is sized from zero blocks), every row dense over its tail tokens
    _run(W.make(W.BATCHED_DECODE, lens=[1, 2, 3, 3, 1], seed=611))


def test_paged_caches():
    sp = dataclasses.replace(W.LONG_DECODE, hq=16, hkv=2, budget=1024)
    _run(W.make(sp, lens=[20000, 7001, 1024 * 4 + 2], seed=602), paged=128)


def test_clustered_winners_select_from_the_row():
    sp = W.BATCHED_DECODE
    wl = W.make(sp, lens=[20000, 9000, 30001, 4000], seed=603)
    a = int(wl.kv_offsets[0]) + 4 * 3000
    wl.k_idx[a:a + 4 * 300] *= 4.0
    b = int(wl.kv_offsets[2]) + 4 * 7000
    wl.k_idx[b:b + 4 * 700] *= 4.0
    _run(wl)


def test_all_equal_scores_take_the_lowest_blocks():
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=1024)
    wl = W.make(sp, lens=[6000, 3001, 40000], seed=604)
    wl.q_idx.zero_()
    dp = _run(wl)
    assert np.array_equal(dp.idx.cpu().numpy()[0], np.arange(256))


def test_duplicated_keys_and_negative_weights():
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=512)
    lens = [4 * 2 * 1000 + 1, 4 * 2 * 3000, 4 * 2 * 700 + 2]
    wl = W.make(sp, lens=lens, seed=605)
    for s, n in enumerate(lens):
        a = int(wl.kv_offsets[s])
        half = 4 * (n // 8)
        wl.k_idx[a + half:a + 2 * half] = wl.k_idx[a:a + half]
    wl.w[:, 1::2] *= -1.0
    _run(wl)


def test_k2048_long_rows_exceed_the_lds_lists():
    # K = 2048: rows of 32768 and 15000 blocks list 7680 and 5640 entries (the
    # 8-group register path); 65536 blocks list 13312 (the lists staged in LDS)
    sp = dataclasses.replace(W.LONG_DECODE, hq=8, hkv=1, budget=8192)
    _run(W.make(sp, lens=[131072 + 3, 262144 + 1, 60000, 8196, 8195, 100], seed=606))


def test_fp32_and_large_batches_run_the_separate_kernels():
    _run(W.make(W.TINY_DECODE, lens=[4096, 1500, 3], seed=607))
    sp = dataclasses.replace(W.BATCHED_DECODE, hq=8, hkv=2, budget=256)
    rng = np.random.default_rng(608)
    lens = [int(x) for x in rng.integers(1000, 3000, 300)]
    _run(W.make(sp, lens=lens, seed=608), oracle_check=False)


def test_graph_replays_match_eager():
    wl = W.make(W.BATCHED_DECODE, lens=[8200 + 1711 * j for j in range(12)], seed=609)
    dp = pipeline.upload(wl, "cuda", decode=True)
    dp.compress()
    dp.decode_step()
    torch.cuda.synchronize()
    eager = (dp.idx.clone(), dp.out.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dp.decode_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dp.decode_step()
    for rep in range(4):
        dp.idx.fill_(-5)
        dp.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dp.idx, eager[0]), f"replay {rep}: idx"
        assert torch.equal(_bits(dp.out), _bits(eager[1])), f"replay {rep}: out"
        dp.decode_step()
        torch.cuda.synchronize()


# --- the decode step with the append inside the scoring launch ------------------
# qsa_ingest_index_score_lists + qsa_sparse_attn_decode_lists.  attach_ingest()
# re-appends every sequence's newest token with the values the caches already
# hold, so the step must give the plain decode step's scores, idx and outputs
# bit for bit; the rows whose newest token completes a block (L % ratio == 0)
# take their last list entry from the append's score.

def _ingest_run(wl, paged=0):
    ref = pipeline.upload(wl, "cuda", decode=True)
    ref.compress()
    if paged:
        ref = pipeline.page(ref, wl.lens, paged, seed=9, extra_pages=2)
    ref.decode_step()
    torch.cuda.synchronize()
    dp = pipeline.upload(wl, "cuda", decode=True)
    dp.compress()
    if paged:
        dp = pipeline.page(dp, wl.lens, paged, seed=9, extra_pages=2)
    pipeline.attach_ingest(dp, wl)
    assert dp.ingest_step_fusable()
    dp.scores.fill_(float("nan"))
    dp.idx.fill_(-9)
    dp.out.zero_()
    dp.ingest_score_lists()
    dp.attend_lists()
    torch.cuda.synchronize()
    assert bool((dp.ing.status == 0).all()), dp.ing.status.tolist()
    Ls = wl.visible_lengths()
    for r, L in enumerate(Ls):
        nb = int(L) // wl.spec.ratio
        assert torch.equal(dp.scores[r, :nb], ref.scores[r, :nb]), f"row {r}: scores differ"
    assert torch.equal(dp.idx, ref.idx), "selection differs from the plain decode step"
    assert torch.equal(_bits(dp.out), _bits(ref.out)), "outputs differ from the plain decode step"
    assert torch.equal(dp.kc.view(torch.uint8), ref.kc.view(torch.uint8)), "compressed keys changed"
    n_slot = sum(1 for L in Ls if int(L) % wl.spec.ratio == 0 and int(L) // wl.spec.ratio > wl.spec.budget // wl.spec.ratio)
    _print(f"[ingest step] {wl.spec.name}: {n_slot} of {len(Ls)} rows filled their last list entry from the append")
    return dp


def test_ingest_step_batched_decode():
    _ingest_run(W.make(W.BATCHED_DECODE))


def test_ingest_step_long_decode():
    _ingest_run(W.make(W.LONG_DECODE))


def test_ingest_step_new_block_wins():
    # the block each sequence's newest token completes gets keys four times
    # larger, so it is selected: the filled slot decides the selection
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=512)
    lens = [4 * 3000, 4 * 2200 + 2, 4 * 5000, 4 * 641, 4 * 2048, 4 * 4097 + 1]
    wl = W.make(sp, lens=lens, seed=610)
    for s, n in enumerate(lens):
        if n % 4 == 0:
            a = int(wl.kv_offsets[s]) + n - 4
            wl.k_idx[a:a + 4] *= 16.0
    dp = _ingest_run(wl)
    ref = oracle.run_workload(wl, want_scores=True, want_out=False)
    check_idx({"idx": dp.idx.cpu().numpy()}, ref, np.arange(wl.total_q))
    got = dp.idx.cpu().numpy()
    # a ReLU score can still be small for a large key, so count rather than
    # require every boosted block
    hits = sum(int((n // 4 - 1) in got[s]) for s, n in enumerate(lens) if n % 4 == 0)
    _print(f"[ingest step] boosted new blocks selected: {hits} of {sum(n % 4 == 0 for n in lens)}")
    assert hits >= 1


@pytest.mark.parametrize("kc_dtype", ["e4m3", "fp4"])
def test_ingest_step_key_formats(kc_dtype):
    sp = dataclasses.replace(W.BATCHED_DECODE, kc_dtype=kc_dtype, budget=512)
    _ingest_run(W.make(sp, lens=[9000, 2052, 4 * 777, 520, 4 * 129, 20004, 33], seed=611))


def test_ingest_step_paged():
    sp = dataclasses.replace(W.LONG_DECODE, hq=16, hkv=2, budget=1024)
    _ingest_run(W.make(sp, lens=[20000, 7000, 4 * 1024 + 4], seed=612), paged=128)


def test_ingest_step_k2048_lists_in_lds():
    sp = dataclasses.replace(W.LONG_DECODE, hq=8, hkv=1, budget=8192)
    _ingest_run(W.make(sp, lens=[131072, 60000, 8196, 8192 + 64, 100], seed=613))


def test_ingest_step_fallback_rows():
    sp = W.BATCHED_DECODE
    wl = W.make(sp, lens=[20000, 9000, 30000, 4000], seed=614)
    a = int(wl.kv_offsets[0]) + 4 * 3000
    wl.k_idx[a:a + 4 * 300] *= 4.0
    b = int(wl.kv_offsets[2]) + 4 * 7000
    wl.k_idx[b:b + 4 * 700] *= 4.0
    _ingest_run(wl)
