"""Debug mode (QSA_DEBUG=1): device-side argument contents are checked before
a call's kernels run, and a violation comes back as QSA_ERR_DEVICE_ASSERT
with nothing launched.

Every corrupted input below is chosen so that the call's own kernels would
still stay inside the buffers even if the check let it through (spare rows,
a spare page, a wide score row; out-of-range block ids are "no token" to
the attention kernels), so no case can fault the GPU.  A clean step in debug
mode must equal the same step without it, bit for bit.
"""
import dataclasses

import pytest
import torch

import indexer_selected_sparse_amd as Q
import qsa_workloads as W
from indexer_selected_sparse_amd import pipeline
from tests.parity import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture
def debug_mode(monkeypatch):
    monkeypatch.setenv("QSA_DEBUG", "1")


def _i64(xs):
    return torch.tensor(xs, dtype=torch.int64, device="cuda")


def _decode_problem():
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=64, hq=8, hkv=2)
    wl = W.make(sp, lens=[100, 200], seed=301)
    dp = pipeline.upload(wl, "cuda")
    dp.compress()
    dp.step()
    torch.cuda.synchronize()
    return wl, dp


def _expect_assert(fn, fragment):
    with pytest.raises(Q.QsaError) as e:
        fn()
    assert e.value.status == Q.QSA_ERR_DEVICE_ASSERT, e.value.message
    assert fragment in e.value.message, e.value.message
    assert "nothing was launched" in e.value.message
    print(f"[debug] rejected: {e.value.message}", flush=True)


def test_clean_step_in_debug_mode_equals_normal_step(monkeypatch):
    wl, dp = _decode_problem()
    ref = (dp.scores.clone(), dp.idx.clone(), dp.out.clone())
    monkeypatch.setenv("QSA_DEBUG", "1")
    dp.scores.zero_()
    dp.idx.fill_(-3)
    dp.out.zero_()
    dp.compress()
    dp.step()
    torch.cuda.synchronize()
    for r, L in enumerate(wl.lens):
        nb = L // wl.spec.ratio
        assert torch.equal(dp.scores[r, :nb], ref[0][r, :nb])
    assert torch.equal(dp.idx, ref[1])
    assert torch.equal(dp.out.view(torch.int16), ref[2].view(torch.int16))


def test_length_past_max_kv_len(debug_mode):
    wl, dp = _decode_problem()
    b = dp.batch
    # the batch claims max_kv_len 150 while sequence 1 holds 200 tokens; the
    # score row is 64 wide (>= 50 blocks), so even an unchecked launch stays
    # inside it
    bad = Q.Batch(b.kv_offsets, b.blk_offsets, None, b.total_q, 150, 1)
    scores = torch.zeros((2, 64), device="cuda")
    _expect_assert(lambda: Q.index_score(dp.q_idx, dp.w, dp.kc, dp.kc_scale, dp.ratio, bad, scores),
                   "kv_offsets")


def test_block_offsets_not_prefix_sums(debug_mode):
    wl, dp = _decode_problem()
    b = dp.batch
    # 25 and 50 blocks: offsets [0, 25, 75]; pass [0, 25, 74] (sequence 1
    # would still read rows 25..74 of the 75 stored)
    bad = Q.Batch(b.kv_offsets, _i64([0, 25, 74]), None, b.total_q, b.max_kv_len, 1)
    _expect_assert(lambda: Q.index_score(dp.q_idx, dp.w, dp.kc, dp.kc_scale, dp.ratio, bad, dp.scores),
                   "blk_offsets")


def test_selected_block_outside_visible_range(debug_mode):
    wl, dp = _decode_problem()
    for bad_id in (100, -2):
        idx = dp.idx.clone()
        idx[0, 3] = bad_id            # sequence 0 has 25 complete blocks
        _expect_assert(lambda: Q.sparse_attn_decode(dp.q, dp.K, dp.V, dp.softmax_scale, idx, dp.budget,
                                                    dp.ratio, dp.batch, dp.out, dp.attn_ws), "idx")


def test_query_offsets(debug_mode):
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=64, hq=8, hkv=2)
    wl = W.make(sp, lens=[100, 200], n_q=[2, 3], seed=302)
    dp = pipeline.upload(wl, "cuda")
    dp.compress()
    dp.step()
    torch.cuda.synchronize()
    b = dp.batch
    # q_offsets[B] = 5 but total_q claims 4 (grids cover 4 queries)
    bad = Q.Batch(b.kv_offsets, b.blk_offsets, b.q_offsets, 4, b.max_kv_len, 3)
    _expect_assert(lambda: Q.sparse_attn_prefill(dp.q, dp.K, dp.V, dp.softmax_scale, dp.idx, dp.budget, dp.ratio,
                                                 bad, dp.out), "q_offsets")
    # three queries in sequence 1 but max_q_per_seq claims 2
    bad = Q.Batch(b.kv_offsets, b.blk_offsets, b.q_offsets, b.total_q, b.max_kv_len, 2)
    _expect_assert(lambda: Q.sparse_attn_prefill(dp.q, dp.K, dp.V, dp.softmax_scale, dp.idx, dp.budget, dp.ratio,
                                                 bad, dp.out), "q_offsets")


def test_page_id_outside_pools(debug_mode, monkeypatch):
    monkeypatch.delenv("QSA_DEBUG")
    wl, dp = _decode_problem()
    pdp = pipeline.page(dp, wl.lens, 64, seed=3, extra_pages=2)
    pg = pdp.paging
    P = pg.page_size
    # pools get one spare page past the declared count: an unchecked read of
    # the bad page id (= the declared count) still lands inside the allocation
    K = torch.cat([pdp.K, torch.zeros((P,) + tuple(pdp.K.shape[1:]), dtype=pdp.K.dtype, device="cuda")])
    V = torch.cat([pdp.V, torch.zeros((P,) + tuple(pdp.V.shape[1:]), dtype=pdp.V.dtype, device="cuda")])
    table = pg.block_table.clone()
    table[1, 1] = pg.num_pages
    bad = Q.Paging(table, pg.num_pages, P)
    out = torch.zeros_like(dp.out)
    torch.cuda.synchronize()
    monkeypatch.setenv("QSA_DEBUG", "1")
    _expect_assert(lambda: Q.sparse_attn_decode(pdp.q, K, V, pdp.softmax_scale, pdp.idx, pdp.budget, pdp.ratio,
                                                pdp.batch, out, pdp.attn_ws, paging=bad), "block_table")
    assert not out.any(), "the rejected call wrote its output"
    # the same call with the table intact passes the check and runs
    Q.sparse_attn_decode(pdp.q, K, V, pdp.softmax_scale, pdp.idx, pdp.budget, pdp.ratio, pdp.batch, out,
                         pdp.attn_ws, paging=pg)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), dp.out.view(torch.int16))
