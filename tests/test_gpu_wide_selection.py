"""Selections wider than the 128 slots a wave of the matrix-core attention
kernel holds in registers.

A part's selected blocks are split over the 4 waves of a workgroup; when one
wave's share exceeds 128 slots (prefill with K = budget/ratio > 512, a window
that widens the row past 512, or a decode batch large enough that few parts
are used) the kernel keeps the wave's slot table in LDS.  Each case here is
built to take that path and is checked against the oracle: indices bit for
bit, outputs within the stated tolerance.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import qsa_workloads as W
from indexer_selected_sparse_amd import pipeline
from tests.parity import check_out, full_check, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _print(*a):
    print(*a, flush=True)


def test_prefill_k2048():
    # budget 8192, ratio 4: K = 2048 blocks, one part per (query, KV head),
    # so each wave walks 512 slots; queries from dense (L <= 8195) to sparse
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=8192)
    wl = W.make(sp, lens=[12000, 8200], n_q=[5, 8], seed=201)
    _print(f"[wide] prefill K=2048: lens={wl.lens} n_q={wl.n_q}")
    _, _, worst = full_check(wl)
    _print(f"[wide] prefill K=2048: ok, worst err/limit = {worst:.3f}")


def test_prefill_k2048_certified_scores():
    sp = dataclasses.replace(W.CHUNKED_PREFILL, budget=8192)
    wl = W.make(sp, lens=[10500], n_q=[6], seed=202)
    full_check(wl, mfma=True)


def test_decode_k2048_many_units():
    # 48 sequences x 4 KV heads = 192 units: three parts of 683 slots, so a
    # wave's share is 171 slots
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=8192)
    rng = np.random.default_rng(203)
    lens = [int(x) for x in rng.integers(8300, 10000, 48)]
    wl = W.make(sp, lens=lens, seed=203)
    _print(f"[wide] decode K=2048, 48 seqs: lens {min(lens)}..{max(lens)}")
    _, _, worst = full_check(wl)
    _print(f"[wide] decode K=2048: ok, worst err/limit = {worst:.3f}")


def test_decode_k1024_one_part():
    # 128 sequences x 4 KV heads = 512 units: one part of 1024 slots, 256 per wave
    sp = dataclasses.replace(W.BATCHED_DECODE, budget=4096, hq=8, hkv=4)
    rng = np.random.default_rng(204)
    lens = [int(x) for x in rng.integers(4200, 5200, 128)]
    wl = W.make(sp, lens=lens, seed=204)
    _print(f"[wide] decode K=1024, 128 seqs: lens {min(lens)}..{max(lens)}")
    _, _, worst = full_check(wl)
    _print(f"[wide] decode K=1024: ok, worst err/limit = {worst:.3f}")


@pytest.mark.parametrize("mfma", [False, True])
def test_prefill_window_past_512(mfma):
    # the chunked-prefill shape (32/4 heads, indexer 8 x 128, budget 2048)
    # with a window of 8 blocks: rows of K + 8 = 520 slots, 130 per wave
    sp = W.CHUNKED_PREFILL
    w = 8
    wl = W.make(sp, lens=[5000], n_q=[12], seed=205)
    dp = pipeline.upload(wl, "cuda", mfma_ws=mfma)
    dp.compress()
    pipeline.set_local_blocks(dp, w)
    dp.step(mfma=mfma)
    torch.cuda.synchronize()
    got_idx = dp.idx.cpu().numpy()
    got_out = dp.out.float().cpu().numpy().astype(np.float64)
    ref = oracle.run_workload(wl, want_out=False)
    Ls = wl.visible_lengths()
    exp_out = np.zeros((wl.total_q, sp.hq, sp.d))
    a, b = int(wl.kv_offsets[0]), int(wl.kv_offsets[1])
    Kf, Vf = wl.K[a:b].float().numpy(), wl.V[a:b].float().numpy()
    for i in range(wl.total_q):
        L = int(Ls[i])
        want = oracle.window_union(ref["idx"][i], L // sp.ratio, w)
        assert np.array_equal(got_idx[i], want), (i, L)
        toks = oracle.token_set(want, sp.ratio, L)
        exp_out[i] = oracle.attn(wl.q[i].float().numpy(), Kf, Vf, toks, sp.softmax_scale)
    check_out(wl, {"out": got_out}, {"out": exp_out}, np.arange(wl.total_q))
