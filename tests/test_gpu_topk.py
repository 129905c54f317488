"""GPU parity of qsa_topk_blocks on given score rows (canonical scores).

Rows are fed straight to the C ABI and the selected block indices must equal
the oracle's selection bit for bit: the K largest (score, -index) pairs in
ascending index order, -1 padded, identity in the dense regime (nb <= K).
Few-row batches whose rows have at most 8192 blocks take the fused
single-workgroup select (sample bracket, in-LDS candidate lists, exact radix
select); longer rows take the two-kernel classify / finish select.  Every case
runs on both: once as given and once with a 40000-block row appended.  The
cases include rows whose bracket cannot hold (top scores hidden between the
sampled segments, all-equal rows), which must fall back to the exact
whole-row select, and rows with exact ties across the threshold.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


_LONG = np.random.default_rng(99).random(40000).astype(np.float32)


def _run(rows, budget=2048, ratio=4):
    """rows: list of 1-D float32 arrays (one per query; nb = len(row)).  Runs
    the batch as given, then (for few-row batches) with a 40000-block row
    appended so that the two-kernel select handles the same rows."""
    n = _run_once(rows, budget, ratio)
    if len(rows) < 256 and max(len(r) for r in rows) <= 8192:
        _run_once(list(rows) + [_LONG], budget, ratio)
    return n


def _run_once(rows, budget, ratio):
    import indexer_selected_sparse_amd as Q
    K = budget // ratio
    lens = [len(r) * ratio + (i % ratio) for i, r in enumerate(rows)]   # ragged tails
    ld = max(len(r) for r in rows) + 1          # >= ceil(max_kv_len / ratio)
    sc = np.zeros((len(rows), ld), dtype=np.float32)
    for i, r in enumerate(rows):
        sc[i, :len(r)] = r
    batch = Q.Batch.from_lengths(lens, None, ratio=ratio, device="cuda")
    scores = torch.from_numpy(sc).cuda()
    idx = torch.full((len(rows), K), -7, dtype=torch.int32, device="cuda")
    n = Q.topk_workspace_size(batch, budget, ratio, None)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda") if n else None
    Q.topk_blocks(scores, budget, ratio, batch, idx, ws=ws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for i, r in enumerate(rows):
        exp = oracle.topk_row(r.astype(np.float32), K)
        assert np.array_equal(got[i], exp), (
            f"row {i} (nb={len(r)}): first difference at slot "
            f"{int(np.argmax(got[i] != exp))}: gpu {got[i][:8]} oracle {exp[:8]}")
    return n


def _relu_like(rng, n):
    # non-negative, like the method's scores: a sum of weighted ReLUs
    x = rng.standard_normal((n, 8)).astype(np.float32)
    w = rng.random(8).astype(np.float32)
    return (np.maximum(x, 0) * w).sum(axis=1).astype(np.float32)


def test_random_rows_short_and_long():
    rng = np.random.default_rng(1)
    rows = [_relu_like(rng, n) for n in (513, 1000, 2048, 2049, 5000, 8192, 20000, 32768, 77777)]
    n = _run(rows)
    assert n > 0          # few rows: the multi-workgroup path with its lists


def test_dense_boundary_rows():
    rng = np.random.default_rng(2)
    rows = [_relu_like(rng, n) for n in (1, 511, 512, 513, 514)]
    _run(rows)


def test_exact_ties_across_the_threshold():
    rng = np.random.default_rng(3)
    # small integers: thousands of exact ties, the threshold falls inside a
    # run of equal scores (ties go to the lower block index)
    rows = [rng.integers(0, 40, n).astype(np.float32) for n in (1500, 6000, 32768)]
    _run(rows)


def test_top_scores_hidden_between_sampled_segments():
    # 64 segments of 32 consecutive blocks, evenly spread, are sampled; the
    # largest scores sit between them, so the bracket misses and the exact
    # whole-row select takes over
    nb = 32768
    step = (nb - 32) // 63
    rng = np.random.default_rng(4)
    r = (rng.random(nb).astype(np.float32) * 0.5).astype(np.float32)
    hidden = np.concatenate([np.arange(j * step + 100, j * step + 110) for j in range(63)])
    r[hidden] = 10.0 + rng.random(len(hidden)).astype(np.float32)
    _run([r, _relu_like(rng, 12345)])


def test_all_equal_rows():
    rows = [np.zeros(n, dtype=np.float32) for n in (700, 2048, 4000, 32768)]
    rows.append(np.full(9000, 3.5, dtype=np.float32))
    _run(rows)


def test_many_rows_take_the_single_workgroup_path():
    rng = np.random.default_rng(5)
    rows = [_relu_like(rng, int(n)) for n in rng.integers(400, 3000, 300)]
    n = _run(rows)
    assert n == 0         # beyond the few-row limit no lists are kept


def test_small_budget_and_other_ratio():
    rng = np.random.default_rng(6)
    rows = [_relu_like(rng, n) for n in (70, 100, 5000, 40000)]
    _run(rows, budget=256, ratio=4)
    _run(rows, budget=2048, ratio=16)


def test_fused_path_edge_cases():
    # rows of at most 8192 blocks: the fused single-workgroup select (and,
    # through _run, the two-kernel select with a long row appended)
    rng = np.random.default_rng(7)
    # exact ties across the threshold
    _run([rng.integers(0, 40, n).astype(np.float32) for n in (1500, 6000, 8192)])
    # top scores hidden between the sampled segments -> exact fallback
    nb = 8192
    step = (nb - 32) // 63
    r = (rng.random(nb).astype(np.float32) * 0.5).astype(np.float32)
    hidden = np.concatenate([np.arange(j * step + 40, j * step + 50) for j in range(63)])
    r[hidden] = 10.0 + rng.random(len(hidden)).astype(np.float32)
    _run([r, _relu_like(rng, 3000)])
    # all-equal rows
    _run([np.zeros(n, dtype=np.float32) for n in (700, 2048, 4000, 8192)] + [np.full(5000, 3.5, np.float32)])
    # negative and mixed-sign scores
    _run([rng.standard_normal(n).astype(np.float32) for n in (600, 4097, 8191)])


def test_k2048_rows():
    # budget/ratio = 2048, the other block count the pages' model validator
    # allows: dense rows (nb <= 2048), the boundary, and sparse rows on both
    # the few-row and the many-row paths, with ties
    rng = np.random.default_rng(21)
    rows = [_relu_like(rng, n) for n in (100, 2048, 2049, 4097, 8192, 20000, 32768)]
    rows.append(rng.integers(0, 30, 9000).astype(np.float32))
    _run(rows, budget=8192)
    many = [_relu_like(rng, int(n)) for n in rng.integers(1800, 6000, 300)]
    _run(many, budget=8192)
