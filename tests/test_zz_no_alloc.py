"""qsa_sparse_attn_decode_static (decode attention whose split partials live
in the library's static device array, for callers that cannot allocate)
against qsa_sparse_attn_decode with a caller workspace: bit for bit, on
consecutive calls of different shapes (the second smaller than the first,
then the first again), so stale contents of the shared array cannot leak
into a later call.  Both are called through the C ABI."""
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


def _problem(spec, lens, seed):
    wl = W.make(spec, lens=lens, seed=seed)
    dp = pipeline.upload(wl, "cuda")
    dp.compress()
    dp.score()
    dp.topk()
    torch.cuda.synchronize()
    return wl, dp


def _both(dp):
    ref = torch.zeros_like(dp.out)
    got = torch.full_like(dp.out, 3.0)
    Q.sparse_attn_decode(dp.q, dp.K, dp.V, dp.softmax_scale, dp.idx, dp.budget, dp.ratio, dp.batch, ref,
                         dp.attn_ws)
    Q.sparse_attn_decode_static(dp.q, dp.K, dp.V, dp.softmax_scale, dp.idx, dp.budget, dp.ratio, dp.batch, got)
    torch.cuda.synchronize()
    return ref, got


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_static_scratch_equals_workspace_on_consecutive_calls():
    big_wl, big = _problem(W.BATCHED_DECODE, [8200 + 977 * j for j in range(24)], seed=401)
    small_wl, small = _problem(dataclasses.replace(W.LONG_DECODE, kc_dtype="bf16", hq=16, hkv=2),
                               [9000, 3001, 2052], seed=402)
    print(f"[static] big: {big_wl.total_q} queries, small: {small_wl.total_q} queries", flush=True)
    outs = []
    for k, (wl, dp) in enumerate(((big_wl, big), (small_wl, small), (big_wl, big))):
        ref, got = _both(dp)
        assert _same(ref, got), f"call {k}: static-scratch output differs from the workspace call"
        outs.append(got)
    # and the second (smaller) call's output is within the oracle's tolerance
    q = np.arange(small_wl.total_q)
    r = oracle.run_workload(small_wl, query_ids=q)
    check_out(small_wl, {"out": outs[1].float().cpu().numpy().astype(np.float64)}, r, q)


def test_static_scratch_single_part_and_fp32():
    # a batch large enough for one part per query (the partials go unused);
    # fp32 takes the register-staged kernel with its own part count
    wl, dp = _problem(dataclasses.replace(W.BATCHED_DECODE, hq=8, hkv=4), [3000 + 5 * j for j in range(160)],
                      seed=403)
    ref, got = _both(dp)
    assert _same(ref, got)
    wl, dp = _problem(W.TINY_DECODE, [4096, 1500], seed=404)
    ref, got = _both(dp)
    assert _same(ref, got)
