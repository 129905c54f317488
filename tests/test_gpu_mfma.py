"""GPU parity of the prefill indexer on the matrix cores and of the
certifying top-k.

QSA_SCORE_MFMA scores sum in an order the hardware picks, so they are checked
against a per-block bound of the canonical value:
    |a_b - c_b| <= 4 (D + H + 2) 2^-23 * sum_h |w_h| |q_h| |kc_b|
(twice the worst-case summation bound of both evaluations, Higham, Accuracy
and Stability of Numerical Algorithms, section 4.2, with Cauchy-Schwarz for
the products).  The selection made from them with `recheck` must equal the
oracle's canonical selection bit for bit, and entries past a query's visible
blocks must be left untouched.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import qsa_workloads as W
from tests.parity import (check_compress, check_idx, check_out, full_check, gpu_available,
                          run_gpu)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SENTINEL = -7.25


def _print(*a):
    print(*a, flush=True)


def bound_per_block(wl, query_ids):
    """E[j, b] for query query_ids[j] and every block b of its sequence (fp64)."""
    sp = wl.spec
    kc, kc_scale = oracle.compress(wl.k_idx.float().numpy(), wl.kv_offsets, sp.ratio, sp.kc_dtype)
    kcv = oracle.kc_values(kc, sp.kc_dtype).astype(np.float64)
    kn = np.linalg.norm(kcv, axis=1)
    if kc_scale is not None:
        kn = kn * kc_scale.astype(np.float64)
    blk = wl.blk_offsets()
    qseq = wl.query_seq()
    qi = wl.q_idx.double().numpy()
    w = wl.w.double().numpy()
    c = 4.0 * (sp.d_idx + sp.h_idx + 2) * 2.0 ** -23
    out = []
    for i in query_ids:
        s = int(qseq[i])
        F = float(np.sum(np.abs(w[i]) * np.linalg.norm(qi[i], axis=1)))
        out.append(c * F * kn[blk[s]:blk[s + 1]] + (1.0 + np.abs(w[i]).sum()) * 2.0 ** -100)
    return out


def mfma_scores(wl):
    """Compress + MFMA scores only (scores pre-filled with a sentinel)."""
    from indexer_selected_sparse_amd import QSA_SCORE_MFMA, pipeline
    dp = pipeline.upload(wl, "cuda", decode=False, mfma_ws=True)
    dp.scores.fill_(SENTINEL)
    dp.compress()
    dp.score(QSA_SCORE_MFMA)
    torch.cuda.synchronize()
    return dp, dp.scores.cpu().numpy()


def check_bound(wl, got_scores, query_ids):
    ref = oracle.run_workload(wl, query_ids=query_ids, want_scores=True, want_out=False)
    Ls = wl.visible_lengths()
    E = bound_per_block(wl, query_ids)
    worst = 0.0
    for j, i in enumerate(query_ids):
        nb = int(Ls[i]) // wl.spec.ratio
        a = got_scores[i, :nb].astype(np.float64)
        c = ref["scores"][j].astype(np.float64)
        err = np.abs(a - c)
        e = E[j][:nb]
        bad = np.nonzero(err > e)[0]
        assert len(bad) == 0, (f"query {i} block {bad[0]}: |mfma - canonical| = {err[bad[0]]:.3g} "
                               f"> bound {e[bad[0]]:.3g}")
        assert np.all(got_scores[i, nb:] == SENTINEL), f"query {i}: wrote past its visible blocks"
        if nb:
            worst = max(worst, float(np.max(err / e)))
    return worst


# (name, H, D, lens, n_q, overrides)
SHAPES = [(f"h{h}_d{d}", h, d) for h in (1, 2, 4, 8, 16) for d in (64, 128)]


@pytest.mark.parametrize("name,h,d", SHAPES, ids=[s[0] for s in SHAPES])
def test_mfma_scores_within_bound_and_selection_exact(name, h, d):
    sp = dataclasses.replace(W.CHUNKED_PREFILL, h_idx=h, d_idx=d, budget=256)
    # two sequences, query counts spanning several 256/H-query workgroups
    # and a ragged last group, plus a causal triangle over several chunks
    wl = W.make(sp, lens=[1500, 2100], n_q=[300, 37], seed=41 + h + d)
    _print(f"[mfma] {name}: lens={wl.lens} n_q={wl.n_q}")
    _, got = mfma_scores(wl)
    q = np.arange(wl.total_q)
    worst = check_bound(wl, got, q)
    _print(f"[mfma] {name}: bound ok (max err/bound {worst:.3g})")
    res, ref, wr = full_check(wl, mfma=True)
    _print(f"[mfma] {name}: idx exact, out worst err/limit {wr:.3f}")


@pytest.mark.parametrize("ratio", [1, 16])
def test_mfma_other_ratios(ratio):
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=64 * ratio, ratio=ratio)
    wl = W.make(sp, lens=[3000 if ratio == 16 else 700], n_q=[90], seed=51 + ratio)
    _, got = mfma_scores(wl)
    check_bound(wl, got, np.arange(wl.total_q))
    full_check(wl, mfma=True)


def test_mfma_decode_batch_and_verify_window():
    # one query per sequence (decode layout) and the verify config's shape
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=512)
    wl = W.make(sp, lens=[5000, 3333, 700, 4097], seed=61)
    full_check(wl, mfma=True)
    wl5 = W.make(W.VERIFY, seed=W.VERIFY.seed + 200)
    _print(f"[mfma] verify: lens={wl5.lens[:4]}... n_q={wl5.n_q[:4]}...")
    full_check(wl5, mfma=True)


def test_recheck_accepts_canonical_scores_all_dtypes():
    # the certifying top-k on canonical scores (any dtype pair) is exact too
    for idx_dt, kc_dt, kv in (("f32", "f32", "f32"), ("bf16", "e4m3", "bf16"), ("f32", "bf16", "bf16")):
        sp = dataclasses.replace(W.TINY_DECODE, idx_dtype=idx_dt, kc_dtype=kc_dt, kv_dtype=kv, budget=256,
                                 h_idx=4, d_idx=64)
        wl = W.make(sp, lens=[4000, 2500, 900], seed=71)
        from indexer_selected_sparse_amd import pipeline
        ref = oracle.run_workload(wl, want_scores=False)
        dp = pipeline.upload(wl, "cuda", mfma_ws=True)
        dp.compress()
        dp.score()
        dp.topk(certified=True)
        torch.cuda.synchronize()
        assert np.array_equal(dp.idx.cpu().numpy(), ref["idx"]), (idx_dt, kc_dt)


def test_flat_rows_take_the_whole_row_recompute():
    # all weights zero: every score is exactly 0, the undecided band is the
    # whole row (more than the candidate buffer), which is then recomputed
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=256)
    wl = W.make(sp, lens=[12000], n_q=[20], seed=81)
    wl.w[:] = 0.0
    res, ref, _ = full_check(wl, mfma=True)
    assert np.array_equal(res["idx"][0], np.arange(64))


def test_half_zero_weights_many_exact_ties():
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=512)
    wl = W.make(sp, lens=[9000], n_q=[64], seed=83)
    wl.w[:, ::2] = 0.0
    wl.q_idx[:, 1::2] = -wl.q_idx[:, 1::2].abs()   # remaining heads mostly negative: many zeros
    full_check(wl, mfma=True)


def test_full_size_chunked_prefill_mfma_all_queries():
    # all 8193 queries: every matrix-core score within its bound of the
    # oracle's canonical score, every certified selection bit for bit and
    # every output within tolerance
    wl = W.make(W.CHUNKED_PREFILL)
    q = np.arange(wl.total_q)
    _print(f"[mfma] full chunked prefill: total_q={wl.total_q}, every query")
    res, dp = run_gpu(wl, mfma=True)
    ref = oracle.run_workload(wl, query_ids=q, want_scores=True)
    check_compress(wl, res, ref)
    check_idx(res, ref, q)
    worst = check_out(wl, res, ref, q)
    Ls = wl.visible_lengths()
    step = 512
    for j0 in range(0, len(q), step):
        part = q[j0:j0 + step]
        E = bound_per_block(wl, part)
        for jj, i in enumerate(part):
            nb = int(Ls[i]) // wl.spec.ratio
            err = np.abs(res["scores"][i, :nb].astype(np.float64) - ref["scores"][j0 + jj])
            assert np.all(err <= E[jj][:nb]), f"query {i}: MFMA score outside its bound"
    _print(f"[mfma] full chunked prefill: idx exact on all queries, out worst err/limit {worst:.3f}")
