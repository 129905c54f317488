"""GPU parity of the paged entry points (K/V, raw and compressed indexer keys
in page pools addressed through a per-sequence block table).

Paging only moves rows, so every paged call must reproduce its contiguous
counterpart bit for bit: compressed keys (gathered back out of the pool),
canonical scores, the selection and the attention output; the contiguous
calls are checked against the oracle in test_gpu_parity, and every paged
case here is also checked against the oracle directly (compressed keys,
scores and indices bit for bit, outputs within tolerance).  The pools hold each sequence's pages in a
random physical order among extra pages filled with garbage; table entries a
sequence does not use point at page 0.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import qsa_workloads as W
from tests.parity import check_compress, check_idx, check_out, check_scores, full_check, gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _pool_like(t, rows, gen):
    """A pool of `rows` rows shaped like t's rows, filled with garbage."""
    shape = (rows,) + tuple(t.shape[1:])
    if t.dtype == torch.uint8:
        return torch.randint(0, 255, shape, generator=gen, dtype=torch.uint8).to(t.device)
    return (torch.randn(shape, generator=gen) * 7.0).to(t.dtype).to(t.device)


def _run_paged(name, spec, lens, nq, page_size, extra_pages=5, seed=0):
    import indexer_selected_sparse_amd as Q
    from indexer_selected_sparse_amd import pipeline
    wl = W.make(spec, lens=lens, n_q=nq, seed=spec.seed + 100)
    decode = nq is None
    dp = pipeline.upload(wl, "cuda", decode=decode)
    r, P = spec.ratio, page_size
    print(f"[paged] {name}: lens={list(wl.lens)[:6]} page_size={P} ratio={r}", flush=True)
    # reference: the contiguous path
    dp.compress()
    dp.score()
    dp.topk()
    dp.attend()
    torch.cuda.synchronize()

    # block table: pages of every sequence at random physical pages
    B = len(wl.lens)
    npg = [math.ceil(n / P) for n in wl.lens]
    num_pages = sum(npg) + extra_pages
    max_pages = max(1, max(npg))
    rng = np.random.default_rng(seed)
    phys = rng.permutation(num_pages)[:sum(npg)]
    table = np.zeros((B, max_pages), dtype=np.int32)
    kv_off = np.concatenate([[0], np.cumsum(wl.lens)])
    gen = torch.Generator().manual_seed(seed)
    Kp = _pool_like(dp.K, num_pages * P, gen)
    Vp = _pool_like(dp.V, num_pages * P, gen)
    Xp = _pool_like(dp.k_idx, num_pages * P, gen)
    kcp = _pool_like(dp.kc, num_pages * (P // r), gen)
    kcsp = None if dp.kc_scale is None else torch.full((num_pages * (P // r),), 3.0e38, device="cuda")
    u = 0
    for s in range(B):
        for j in range(npg[s]):
            p = int(phys[u]); u += 1
            table[s, j] = p
            a, n = int(kv_off[s]) + j * P, min(P, wl.lens[s] - j * P)
            for src, dst in ((dp.K, Kp), (dp.V, Vp), (dp.k_idx, Xp)):
                dst[p * P:p * P + n] = src[a:a + n]
    pg = Q.Paging(torch.from_numpy(table).cuda(), num_pages, P)

    # compress into the pool; gather the pool rows back in logical order
    Q.compress_keys(Xp, r, dp.batch, kcp, kcsp, paging=pg)
    torch.cuda.synchronize()
    rows = np.concatenate([table[s, np.arange(n // r) // (P // r)].astype(np.int64) * (P // r)
                           + np.arange(n // r) % (P // r) for s, n in enumerate(wl.lens)])
    nblk = len(rows)
    rows_t = torch.from_numpy(rows).cuda()
    got, exp = kcp[rows_t], dp.kc[:nblk]
    if got.dtype != torch.uint8:
        got, exp = got.contiguous().view(torch.uint8), exp.contiguous().view(torch.uint8)
    assert torch.equal(got, exp), "compressed keys differ"
    if kcsp is not None:
        assert torch.equal(kcsp[rows_t], dp.kc_scale[:nblk]), "kc_scale differs"

    # scores from the pool
    sc = torch.full_like(dp.scores, float("nan"))
    Q.index_score(dp.q_idx, dp.w, kcp, kcsp, r, dp.batch, sc, paging=pg)
    torch.cuda.synchronize()
    Ls = wl.visible_lengths()
    got_s, exp_s = sc.cpu().numpy(), dp.scores.cpu().numpy()
    for i in range(wl.total_q):
        nb = int(Ls[i]) // r
        assert np.array_equal(got_s[i, :nb].view(np.uint32), exp_s[i, :nb].view(np.uint32)), \
            f"scores differ in row {i}"
    idx = torch.full_like(dp.idx, -7)
    Q.topk_blocks(sc, dp.budget, r, dp.batch, idx, ws=dp.topk_ws_canon)
    torch.cuda.synchronize()
    assert torch.equal(idx, dp.idx)

    # attention from the pools
    out = torch.zeros_like(dp.out)
    fn = Q.sparse_attn_decode if decode else Q.sparse_attn_prefill
    fn(dp.q, Kp, Vp, dp.softmax_scale, idx, dp.budget, r, dp.batch, out, dp.attn_ws, paging=pg)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8) if out.dtype == torch.bfloat16 else out,
                       dp.out.view(torch.uint8) if dp.out.dtype == torch.bfloat16 else dp.out), \
        f"attention output differs (max {float((out.float() - dp.out.float()).abs().max()):.3g})"
    print(f"[paged] {name}: paged == contiguous (kc, scores, idx, out)", flush=True)

    # and the paged results themselves against the oracle
    res = {"kc": kcp[rows_t].cpu(), "kc_scale": None if kcsp is None else kcsp[rows_t].cpu(),
           "scores": got_s, "idx": idx.cpu().numpy(), "out": out.float().cpu().numpy().astype(np.float64)}
    ref = oracle.run_workload(wl, want_scores=True)
    q = np.arange(wl.total_q)
    check_compress(wl, res, ref)
    check_scores(wl, res, ref, q)
    check_idx(res, ref, q)
    worst = check_out(wl, res, ref, q)
    print(f"[paged] {name}: paged results == oracle (worst err/limit {worst:.3f})", flush=True)
    return wl


CASES = [
    ("batched_bf16_page64", W.BATCHED_DECODE, [3001, 1234, 777, 5002, 2049, 2052], None, 64, {}),
    ("batched_bf16_page16", W.BATCHED_DECODE, [1500, 903, 64, 65, 3], None, 16, {"budget": 64}),
    ("long_e4m3_page256", W.LONG_DECODE, [6001, 3003, 1000], None, 256, {"budget": 512}),
    ("tiny_f32_page32", W.TINY_DECODE, [1027, 4099, 333, 2], None, 32, {"budget": 256}),
    ("ratio16_page16", W.BATCHED_DECODE, [16 * 70 + 5, 300, 16 * 130], None, 16,
     {"ratio": 16, "budget": 64 * 16, "hq": 8, "hkv": 1}),
    ("prefill_page128", W.CHUNKED_PREFILL, [1500], [300], 128, {"budget": 256}),
    ("verify_page64", W.VERIFY, [2044, 2050, 2051, 2052, 2055, 2064], [4] * 6, 64, {}),
]


@pytest.mark.parametrize("name,spec,lens,nq,page,over", CASES, ids=[c[0] for c in CASES])
def test_paged_equals_contiguous(name, spec, lens, nq, page, over):
    sp = dataclasses.replace(spec, **over) if over else spec
    _run_paged(name, sp, lens, nq, page)


def test_paged_case_against_oracle():
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=256)
    wl = _run_paged("oracle_case", sp, [2100, 517, 3333], None, 32)
    full_check(wl)          # the contiguous path (== paged, above) against the oracle


def test_pipeline_page_step_equals_contiguous():
    # pipeline.page(): the helper the benchmark's --paged option uses
    from indexer_selected_sparse_amd import pipeline
    sp = dataclasses.replace(W.LONG_DECODE, budget=512)
    wl = W.make(sp, lens=[4001, 2222, 517], seed=5)
    dp = pipeline.upload(wl, "cuda", decode=True)
    dp.compress()
    dp.step()
    pdp = pipeline.page(dp, wl.lens, 128, seed=1, extra_pages=3)
    pdp.idx, pdp.out = torch.full_like(dp.idx, -7), torch.zeros_like(dp.out)
    pdp.compress()
    pdp.step()
    torch.cuda.synchronize()
    assert torch.equal(pdp.idx, dp.idx)
    assert torch.equal(pdp.out.view(torch.uint8), dp.out.view(torch.uint8))
