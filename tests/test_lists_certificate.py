"""The candidate-list certificate, checked on the CPU by brute force.

The scorer lists each 64-block chunk's best list_len(nb, K) blocks (by score
desc, index asc) with the chunk's cutoff (the key of its last listed block,
or 0 when the chunk is listed whole); with the append inside the scoring
launch, the chunk of the block a row's newest token completes lists one
block fewer and the selection fills its last slot with that block.  The
selection from the lists is taken only when T, the K-th largest listed key,
is positive and every cutoff is strictly below it.  These tests emulate
that rule in plain numpy, independently of the kernels, and check on many
rows — random, tied, clustered, all-equal, with zeros and negative scores,
ragged last chunks — that whenever the certificate holds, the selection
equals the exact top-K of the whole row (ties to the lower index), and that
the rows the kernels' tests rely on really take both paths.
"""
import math

import numpy as np
import pytest

CHUNK = 64


def list_len(nb, K):
    m = -(-CHUNK * K // nb)
    s = math.isqrt(m)
    if s * s < m:
        s += 1
    return min(CHUNK, m + 4 * s + 3)


def order_keys(row):
    u = np.asarray(row, dtype=np.float32).view(np.uint32).astype(np.int64)
    return np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)


def exact_topk(keys, K):
    """Ascending block ids of the K largest (key desc, index asc)."""
    order = np.lexsort((np.arange(len(keys)), -keys))
    return np.sort(order[:K])


def build_lists(keys, K, new_block=False):
    """(entries as (key, block) in list order, cutoffs) as the scorer writes
    them; with new_block the last block is left out of its chunk's choice and
    appended as the chunk's last entry (what the selection fills in)."""
    nb = len(keys)
    kk = list_len(nb, K)
    entries, cuts = [], []
    for c0 in range(0, nb, CHUNK):
        blocks = np.arange(c0, min(c0 + CHUNK, nb))
        cand = blocks[blocks != nb - 1] if new_block and c0 <= nb - 1 < c0 + CHUNK else blocks
        cap = kk - 1 if new_block and c0 <= nb - 1 < c0 + CHUNK else kk
        order = cand[np.lexsort((cand, -keys[cand]))]
        chosen = np.sort(order[:cap])
        cuts.append(int(keys[order[cap - 1]]) if len(cand) > cap else 0)
        chunk_entries = [(int(keys[b]), int(b)) for b in chosen]
        chunk_entries += [(0, -1)] * (cap - len(chosen))          # padding: key 0
        if new_block and c0 <= nb - 1 < c0 + CHUNK:
            chunk_entries.append((int(keys[nb - 1]), nb - 1))
        entries.extend(chunk_entries)
    return entries, cuts


def select_from_lists(entries, cuts, K):
    """The selection the lists certify, or None."""
    listed = [(k, b) for k, b in entries if k != 0]
    if len(listed) < K:
        return None
    ks = sorted((k for k, _ in listed), reverse=True)
    T = ks[K - 1]
    if T == 0 or max(cuts) >= T:
        return None
    need_eq = K - sum(1 for k in ks if k > T)
    out, eq = [], 0
    for k, b in entries:                      # list order is ascending block order
        if k > T:
            out.append(b)
        elif k == T and k != 0:
            if eq < need_eq:
                out.append(b)
            eq += 1
    return np.array(out)


def rows(rng, n):
    kinds = ["normal", "relu", "ties", "clustered", "equal", "negative", "small_ints"]
    for t in range(n):
        kind = kinds[t % len(kinds)]
        nb = int(rng.integers(2, 5000))
        K = int(rng.choice([1, 3, 16, 128, 512]))
        if kind == "normal":
            row = rng.standard_normal(nb)
        elif kind == "relu":
            row = np.maximum(rng.standard_normal(nb), 0.0)       # many exact zeros
        elif kind == "ties":
            row = rng.integers(0, 20, nb).astype(np.float32)
        elif kind == "clustered":
            row = rng.standard_normal(nb)
            a = int(rng.integers(0, nb))
            row[a:a + max(1, nb // 10)] += 8.0
        elif kind == "equal":
            row = np.full(nb, 1.5)
        elif kind == "negative":
            row = -np.abs(rng.standard_normal(nb))
        else:
            row = rng.integers(0, 4, nb).astype(np.float32)
        yield kind, row.astype(np.float32), K


@pytest.mark.parametrize("new_block", [False, True])
def test_certified_selection_is_exact(new_block):
    rng = np.random.default_rng(20 + int(new_block))
    taken = {"lists": 0, "row": 0, "dense": 0}
    for kind, row, K in rows(rng, 1400):
        keys = order_keys(row)
        nb = len(keys)
        if nb <= K:
            taken["dense"] += 1
            continue
        entries, cuts = build_lists(keys, K, new_block)
        assert len(entries) == -(-nb // CHUNK) * list_len(nb, K)
        got = select_from_lists(entries, cuts, K)
        if got is None:
            taken["row"] += 1
            continue
        taken["lists"] += 1
        want = exact_topk(keys, K)
        assert np.array_equal(got, want), (kind, nb, K)
    assert taken["lists"] > 300 and taken["row"] > 50, taken


def test_list_order_is_ascending_blocks():
    rng = np.random.default_rng(3)
    for new_block in (False, True):
        for nb in (65, 700, 4097):
            keys = order_keys(rng.standard_normal(nb).astype(np.float32))
            entries, _ = build_lists(keys, 128, new_block)
            blocks = [b for k, b in entries if k != 0]
            assert blocks == sorted(blocks)


def test_list_len_bounds():
    # at least the chunk's expected share, at most a whole chunk; the
    # expected-share formula and the 64 cap as the kernels compute them
    for nb in (129, 1000, 2048, 8192, 32768, 131072):
        for K in (1, 128, 512, 2048):
            if nb <= K:
                continue
            kk = list_len(nb, K)
            m = -(-64 * K // nb)
            assert min(64, m) <= kk <= 64
    assert list_len(32768, 512) == 8 and list_len(8192, 512) == 15 and list_len(2048, 512) == 35


_BOUND_PROGRAM = r"""
#include <cstdio>
#include "qsa_lists.hpp"
int main() {
    long long nb;
    int K;
    while (std::scanf("%lld %d", &nb, &K) == 2) std::printf("%lld\n", (long long)qsa::list_max_entries(nb, K));
    return 0;
}
"""


def test_list_max_entries_is_the_largest_list_a_row_can_hold(tmp_path):
    # The attention kernels request, before a row's length is known, the most
    # entries any row of at most nb_max blocks can list; the library computes
    # that per value of m = ceil(64 K / nb) (the count is not monotone in nb).
    # Here the library's host function, built on its own, against the running
    # maximum of ceil(nb / 64) * list_len(nb, K) over every nb.
    import os
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = tmp_path / "bound.cpp"
    src.write_text(_BOUND_PROGRAM)
    exe = tmp_path / "bound"
    subprocess.run([hipcc, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(root, "include"),
                    "-I", os.path.join(root, "indexer_selected_sparse_amd", "csrc"), str(src), "-o", str(exe)],
                   check=True, capture_output=True, text=True, timeout=300)
    top = 140000
    pairs, want = [], []
    for K in (1, 2, 3, 7, 8, 63, 64, 100, 512, 1000, 1024, 2047, 2048):
        best, run = 0, [0] * (top + 1)
        for nb in range(1, top + 1):
            if nb > K:
                best = max(best, -(-nb // CHUNK) * list_len(nb, K))
            run[nb] = best
        nbs = set(range(1, 3001)) | set(range(1, top + 1, 61))
        for m in range(1, CHUNK + 1):
            edge = -(-CHUNK * K // m)
            nbs |= {edge - 1, edge, edge + 1}
        for nb in sorted(x for x in nbs if 1 <= x <= top):
            pairs.append(f"{nb} {K}")
            want.append(run[nb])
    out = subprocess.run([str(exe)], input="\n".join(pairs) + "\n", capture_output=True, text=True, check=True,
                         timeout=300).stdout.split()
    got = [int(x) for x in out]
    bad = [(p, g, w) for p, g, w in zip(pairs, got, want) if g != w]
    assert len(got) == len(want) and not bad, bad[:5]
