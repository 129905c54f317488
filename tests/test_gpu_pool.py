"""Selection from pooled token scores (canonical token scores on the raw
indexer keys -> qsa_pool_scores -> block top-k -> attention) against the
oracle: token scores, pooled scores and selections bit for bit, outputs
within the stated tolerance."""
import dataclasses

import numpy as np
import pytest
import torch

import indexer_selected_sparse_amd as Q
import oracle
import qsa_workloads as W
from indexer_selected_sparse_amd import pipeline
from tests.parity import check_out, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MODES = {"max": Q.QSA_POOL_MAX, "mean": Q.QSA_POOL_MEAN}


def _check(wl, mode, paged=0):
    sp = wl.spec
    dp = pipeline.upload(wl, "cuda")
    dp.compress()
    if paged:
        dp = pipeline.page(dp, wl.lens, paged, seed=8)
    pipeline.set_token_pool(dp, MODES[mode])
    dp.step()
    torch.cuda.synchronize()
    tok_g = dp.tok_scores.cpu().numpy()
    blk_g = dp.scores.cpu().numpy()
    idx_g = dp.idx.cpu().numpy()
    out_g = dp.out.float().cpu().numpy().astype(np.float64)
    Ls, qseq = wl.visible_lengths(), wl.query_seq()
    K = sp.budget // sp.ratio
    exp_out = np.zeros((wl.total_q, sp.hq, sp.d))
    for i in range(wl.total_q):
        L, s = int(Ls[i]), int(qseq[i])
        a, b = int(wl.kv_offsets[s]), int(wl.kv_offsets[s + 1])
        kraw = wl.k_idx[a:a + L].float().numpy()
        tok = oracle.score_row(wl.q_idx[i].float().numpy(), wl.w[i].numpy(), kraw)
        assert np.array_equal(tok_g[i, :L].view(np.uint32), tok.view(np.uint32)), (i, "token scores")
        blk = oracle.pool_scores(tok, sp.ratio, mode)
        nb = len(blk)
        assert np.array_equal(blk_g[i, :nb].view(np.uint32), blk.view(np.uint32)), (i, "pooled scores")
        idx = oracle.topk_row(blk, K)
        assert np.array_equal(idx_g[i], idx), (i, idx_g[i][:8], idx[:8])
        toks = oracle.token_set(idx, sp.ratio, L)
        exp_out[i] = oracle.attn(wl.q[i].float().numpy(), wl.K[a:b].float().numpy(),
                                 wl.V[a:b].float().numpy(), toks, sp.softmax_scale)
    check_out(wl, {"out": out_g}, {"out": exp_out}, np.arange(wl.total_q))


@pytest.mark.parametrize("mode", ["max", "mean"])
@pytest.mark.parametrize("paged", [0, 64])
def test_decode_pooled(mode, paged):
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=256)
    wl = W.make(sp, lens=[3001, 1234, 777, 80, 259, 260], seed=51)
    _check(wl, mode, paged)


def test_prefill_rows_pooled():
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=256)
    wl = W.make(sp, lens=[1500], n_q=[120], seed=52)
    _check(wl, "max")


def test_pool_ratio_8_mean():
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=512, ratio=8, hq=8, hkv=1)
    wl = W.make(sp, lens=[5000, 4099, 300], seed=53)
    _check(wl, "mean")
