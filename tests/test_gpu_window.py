"""Top-k with the recent window kept (qsa_topk_blocks_local) and attention
over the union, against the oracle: the union rows bit for bit, the outputs
within the stated tolerance."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import qsa_workloads as W
from indexer_selected_sparse_amd import pipeline
from tests.parity import check_out, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _check(wl, w, mfma=False):
    sp = wl.spec
    dp = pipeline.upload(wl, "cuda", mfma_ws=mfma)
    dp.compress()
    pipeline.set_local_blocks(dp, w)
    dp.step(mfma=mfma)
    torch.cuda.synchronize()
    got_idx = dp.idx.cpu().numpy()
    got_out = dp.out.float().cpu().numpy().astype(np.float64)
    ref = oracle.run_workload(wl, want_out=False)
    Ls = wl.visible_lengths()
    qseq = wl.query_seq()
    K = sp.budget // sp.ratio
    exp_out = np.zeros((wl.total_q, sp.hq, sp.d))
    for i in range(wl.total_q):
        L = int(Ls[i])
        nb = L // sp.ratio
        want = oracle.window_union(ref["idx"][i], nb, w)
        assert np.array_equal(got_idx[i], want), (i, L, got_idx[i][:8], want[:8])
        s = int(qseq[i])
        a, b = int(wl.kv_offsets[s]), int(wl.kv_offsets[s + 1])
        toks = oracle.token_set(want, sp.ratio, L)
        exp_out[i] = oracle.attn(wl.q[i].float().numpy(), wl.K[a:b].float().numpy(),
                                 wl.V[a:b].float().numpy(), toks, sp.softmax_scale)
        assert len(toks) <= (K + w) * sp.ratio + sp.ratio - 1
    check_out(wl, {"out": got_out}, {"out": exp_out}, np.arange(wl.total_q))


@pytest.mark.parametrize("w", [1, 8, 32])
def test_decode_window(w):
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=256)
    wl = W.make(sp, lens=[3001, 1234, 777, 80, 5002, 259, 292], seed=41)
    _check(wl, w)


def test_decode_window_e4m3_long():
    sp = dataclasses.replace(W.LONG_DECODE, budget=512)
    wl = W.make(sp, lens=[9000, 2100, 2051], seed=42)
    _check(wl, 32)


def test_prefill_window_certified_topk():
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=256)
    wl = W.make(sp, lens=[1500], n_q=[300], seed=43)
    _check(wl, 16, mfma=True)
