"""A multi-layer decode step with shared indexers (pipeline.LayerStack)
against the oracle: full layers select from their own indexer, shared
layers attend their own K/V with the last full layer's selection."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import qsa_workloads as W
from indexer_selected_sparse_amd import pipeline
from tests.parity import check_out, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("n_layers,full_every", [(4, 2), (5, 3), (3, 1)])
def test_shared_indexer_layers(n_layers, full_every):
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=256)
    lens = [3001, 1234, 777, 80, 2052]
    wls = [W.make(sp, lens=lens, seed=60 + 7 * l) for l in range(n_layers)]
    layers = []
    for l, wl in enumerate(wls):
        dp = pipeline.upload(wl, "cuda")
        if l % full_every == 0:
            dp.compress()
        layers.append(dp)
    stack = pipeline.LayerStack(layers, full_every)
    stack.step()
    torch.cuda.synchronize()
    Ls, qseq = wls[0].visible_lengths(), wls[0].query_seq()
    sel = None
    for l, (wl, dp) in enumerate(zip(wls, layers)):
        if l % full_every == 0:
            ref = oracle.run_workload(wl)
            sel = ref["idx"]
            assert np.array_equal(dp.idx.cpu().numpy(), sel), l
            exp = ref["out"]
        else:
            assert dp.idx.data_ptr() == layers[l - l % full_every].idx.data_ptr()
            exp = np.zeros((wl.total_q, sp.hq, sp.d))
            for i in range(wl.total_q):
                s = int(qseq[i])
                a, b = int(wl.kv_offsets[s]), int(wl.kv_offsets[s + 1])
                toks = oracle.token_set(sel[i], sp.ratio, int(Ls[i]))
                exp[i] = oracle.attn(wl.q[i].float().numpy(), wl.K[a:b].float().numpy(),
                                     wl.V[a:b].float().numpy(), toks, sp.softmax_scale)
        got = dp.out.float().cpu().numpy().astype(np.float64)
        check_out(wl, {"out": got}, {"out": exp}, np.arange(wl.total_q))
