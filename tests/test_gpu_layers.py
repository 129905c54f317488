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


@pytest.mark.parametrize("n_layers,full_every,paged", [(4, 4, False), (11, 11, False), (6, 3, True)])
def test_fused_layers_equal_per_layer_calls(n_layers, full_every, paged):
    """One layered attention launch per full layer and its shared layers gives
    every layer's output bit for bit as its own decode call (11 layers: a
    group beyond the 8-layer launch limit splits)."""
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=512)
    lens = [5000, 1234, 777, 80, 2052, 4099, 3, 1]
    wls = [W.make(sp, lens=lens, seed=90 + l) for l in range(n_layers)]

    def build(fused):
        layers = []
        table = None
        for l, wl in enumerate(wls):
            dp = pipeline.upload(wl, "cuda")
            if l % full_every == 0:
                dp.compress()
            if paged:
                dp = pipeline.page(dp, lens, 64, seed=5)
                if table is None:
                    table = dp.paging
                else:   # one block table for every layer's pools
                    assert torch.equal(dp.paging.block_table, table.block_table)
                    dp.paging = table
            layers.append(dp)
        return pipeline.LayerStack(layers, full_every, fused=fused)

    a, b = build(True), build(False)
    assert a.group_ws is not None
    a.step()
    b.step()
    torch.cuda.synchronize()
    for l, (x, y) in enumerate(zip(a.layers, b.layers)):
        assert torch.equal(x.idx, y.idx), l
        assert torch.equal(x.out.view(torch.int16), y.out.view(torch.int16)), l
    # the per-layer outputs also match the oracle on the first shared layer
    wl, dp = wls[1], a.layers[1]
    sel = oracle.run_workload(wls[0])["idx"]
    Ls, qseq = wl.visible_lengths(), wl.query_seq()
    exp = np.zeros((wl.total_q, sp.hq, sp.d))
    for i in range(wl.total_q):
        s = int(qseq[i])
        a0, b0 = int(wl.kv_offsets[s]), int(wl.kv_offsets[s + 1])
        toks = oracle.token_set(sel[i], sp.ratio, int(Ls[i]))
        exp[i] = oracle.attn(wl.q[i].float().numpy(), wl.K[a0:b0].float().numpy(),
                             wl.V[a0:b0].float().numpy(), toks, sp.softmax_scale)
    check_out(wl, {"out": dp.out.float().cpu().numpy().astype(np.float64)}, {"out": exp},
              np.arange(wl.total_q))


@pytest.mark.parametrize("cfg,lens", [("tiny_decode", [4096, 1500]), ("batched_decode", [9000, 1234, 80, 20000, 4099])])
def test_layers_api_each_layer_its_own_scale(cfg, lens):
    """qsa_sparse_attn_decode_layers with a different q, K, V and softmax scale
    per layer equals each layer's own decode call bit for bit (bf16: one
    layered launch; fp32: the per-layer launches it falls back to)."""
    import indexer_selected_sparse_amd as Q
    sp = W.CONFIGS[cfg]
    base = pipeline.upload(W.make(sp, lens=lens, seed=71), "cuda")
    base.compress()
    base.score()
    base.topk()
    gen = torch.Generator(device="cuda").manual_seed(5)

    def fresh(t):
        return torch.randn(t.shape, generator=gen, device="cuda", dtype=torch.float32).to(t.dtype)

    n = 3
    layers = [(base.q, base.K, base.V, base.softmax_scale)]
    for l in range(1, n):
        layers.append((fresh(base.q), fresh(base.K), fresh(base.V), base.softmax_scale * (1.0 + 0.25 * l)))
    outs = [torch.full_like(base.out, float("nan")) for _ in range(n)]
    nws = Q.attn_layers_workspace_size(*layers[0], n, base.budget, base.ratio, base.batch)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    Q.sparse_attn_decode_layers(layers, base.idx, base.budget, base.ratio, base.batch, outs, ws)
    torch.cuda.synchronize()
    for l, (q, K, V, sc) in enumerate(layers):
        ref = torch.full_like(base.out, float("nan"))
        one = Q.attn_workspace_size(q, K, V, sc, base.budget, base.ratio, base.batch)
        w1 = torch.empty(max(one, 1), dtype=torch.uint8, device="cuda")
        Q.sparse_attn_decode(q, K, V, sc, base.idx, base.budget, base.ratio, base.batch, ref, w1)
        torch.cuda.synchronize()
        bits = torch.int16 if ref.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(outs[l].view(bits), ref.view(bits)), l
