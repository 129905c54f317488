"""Pins for the CPU oracle: each test checks the oracle against something other
than itself — a library routine (torch's bf16/e4m3 casts, numpy integer
arithmetic, numpy lexsort, torch's fp64 scaled-dot-product attention), a closed
form, a brute-force enumeration, or a number the source pages print.

These run on the CPU only (no GPU, no HIP library).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import qsa_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


@pytest.fixture(scope="module")
def page():
    with open(GOLDEN) as f:
        return json.load(f)


# ------------------------------------------------------------------ codecs
def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # S.1111.111 only (E4M3FN has no infinities)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def _e4m3_test_values():
    finite = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (finite[:-1] + finite[1:]) / 2.0          # every tie between neighbours
    vals = [finite, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)]
    rng = np.random.default_rng(7)
    vals.append(rng.uniform(0, 448, 4000))
    vals.append(np.exp(rng.uniform(-25, math.log(448), 4000)))
    v = np.concatenate(vals).astype(np.float32)
    v = v[(v >= 0) & (v <= 448)]
    return np.concatenate([v, -v])


def test_e4m3_encode_matches_torch_including_every_tie():
    v = _e4m3_test_values()
    ours = oracle.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert len(bad) == 0, (v[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_bf16_round_matches_torch_including_ties():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000).astype(np.float32)
    # Exact ties: a bf16 value plus half of its ulp, both parities of the kept bit.
    base = (rng.integers(0x3800, 0x4800, 4000).astype(np.uint32) << 16)
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1e-30, 3.0e38])])
    ours = oracle.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- compress
def test_compress_groups_complete_blocks_only_and_means_exactly():
    # Row t, dim j holds 8*t + j/8: a per-row ramp with power-of-two steps, so
    # every mean is exact and reveals which rows were grouped.
    ratio, d = 4, 16
    lens = [13, 4, 3, 9]
    rows = []
    for n in lens:
        t = np.arange(n, dtype=np.float64)[:, None]
        rows.append(8.0 * t + np.arange(d)[None, :] / 8.0)
    x = np.concatenate(rows).astype(np.float32)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    kc, sc = oracle.compress(x, off, ratio, "f32")
    assert sc is None
    assert kc.shape == (sum(n // ratio for n in lens), d)
    r = 0
    for n in lens:
        for b in range(n // ratio):
            expect = 8.0 * (b * ratio + (ratio - 1) / 2.0) + np.arange(d) / 8.0
            assert np.array_equal(kc[r], expect.astype(np.float32))
            r += 1


def test_compress_constant_rows_and_bf16_store_matches_torch_cast():
    rng = np.random.default_rng(11)
    x = np.repeat(rng.standard_normal((5, 1, 32)).astype(np.float32), 4, axis=1).reshape(20, 32)
    off = np.array([0, 20], dtype=np.int64)
    kc, _ = oracle.compress(x, off, 4, "f32")
    assert np.array_equal(kc, x[::4])
    y = rng.standard_normal((40, 64)).astype(np.float32)
    off = np.array([0, 40], dtype=np.int64)
    kf, _ = oracle.compress(y, off, 4, "f32")
    kb, _ = oracle.compress(y, off, 4, "bf16")
    ref = torch.from_numpy(kf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kb, ref)
    # The fp32 mean is within one rounding of the fp64 mean per addition.
    exact = y.astype(np.float64).reshape(10, 4, 64).mean(axis=1)
    assert np.all(np.abs(kf - exact) <= 4 * 2.0 ** -24 * np.abs(y).reshape(10, 4, 64).sum(1))


def test_compress_e4m3_scale_and_codes_properties():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((64, 128)).astype(np.float32)
    y[8:12] = 0.0                         # block 2 is all zeros
    off = np.array([0, 64], dtype=np.int64)
    kf, _ = oracle.compress(y, off, 4, "f32")
    codes, scale = oracle.compress(y, off, 4, "e4m3")
    assert scale[2] == 0.0 and not codes[2].any()
    for b in range(16):
        if b == 2:
            continue
        amax = np.abs(kf[b]).max()
        # scale is max|x| / 448 (one fp32 rounding)
        assert abs(float(scale[b]) * 448.0 - amax) <= 2.0 ** -23 * amax
        dec = oracle.e4m3_decode(codes[b]).astype(np.float64)
        # the largest magnitude lands on the top code
        assert np.abs(dec).max() == 448.0
        # every code times the scale is within half an e4m3 step of the mean
        err = np.abs(dec * scale[b] - kf[b])
        assert np.all(err <= 2.0 ** -4 * np.abs(kf[b]) + 2.0 ** -10 * scale[b] + 1e-30)


# ------------------------------------------------------------------- score
def test_score_equals_integer_arithmetic_on_small_integers():
    rng = np.random.default_rng(2)
    for H, D, nb in [(4, 64, 50), (8, 128, 40), (3, 17, 9)]:
        q = rng.integers(-4, 5, (H, D))
        k = rng.integers(-4, 5, (nb, D))
        w = rng.integers(0, 4, H)
        dots = k @ q.T                                   # [nb, H] exact int64
        ref = (np.maximum(dots, 0) * w[None, :]).sum(1)
        got = oracle.score_row(q, w, k)
        assert np.array_equal(got, ref.astype(np.float32))
        # with a power-of-two block scale (e4m3 path) the score scales exactly
        sc = np.full(nb, 0.25, dtype=np.float32)
        got = oracle.score_row(q, w, k, sc)
        ref = (np.maximum(dots * 0.25, 0) * w[None, :]).sum(1)
        assert np.array_equal(got, ref.astype(np.float32))


def test_score_zero_query_gives_positive_zero_and_one_hot_weight_selects_head():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((30, 64)).astype(np.float32)
    s = oracle.score_row(np.zeros((4, 64)), rng.random(4), k)
    assert np.all(s.view(np.uint32) == 0)
    q = rng.standard_normal((4, 64)).astype(np.float32)
    for h in range(4):
        w = np.zeros(4, dtype=np.float32)
        w[h] = 1.0
        s = oracle.score_row(q, w, k).astype(np.float64)
        ref = np.maximum(k.astype(np.float64) @ q[h].astype(np.float64), 0)
        assert np.all(np.abs(s - ref) <= 64 * 2.0 ** -24 * (np.abs(k) @ np.abs(q[h])) + 1e-30)


def test_score_within_summation_bound_of_fp64():
    rng = np.random.default_rng(9)
    H, D, nb = 8, 128, 300
    q = rng.standard_normal((H, D)).astype(np.float32)
    k = rng.standard_normal((nb, D)).astype(np.float32)
    w = rng.random(H).astype(np.float32)
    s = oracle.score_row(q, w, k).astype(np.float64)
    dots = k.astype(np.float64) @ q.astype(np.float64).T
    exact = (np.maximum(dots, 0) * w.astype(np.float64)).sum(1)
    u = 2.0 ** -24
    mag = (np.abs(k).astype(np.float64) @ np.abs(q).astype(np.float64).T) @ w.astype(np.float64)
    gamma = (D + H + 2) * u / (1 - (D + H + 2) * u)
    assert np.all(np.abs(s - exact) <= gamma * mag + 1e-30)


# -------------------------------------------------------------------- topk
def _brute_topk(scores, K):
    nb = len(scores)
    if nb <= K:
        return list(range(nb)) + [-1] * (K - nb)
    better = lambda a, b: scores[a] > scores[b] or (scores[a] == scores[b] and a < b)
    found = []
    for S in itertools.combinations(range(nb), K):
        rest = set(range(nb)) - set(S)
        if all(better(a, b) for a in S for b in rest):
            found.append(list(S))
    assert len(found) == 1
    return found[0]


def test_topk_equals_brute_force_over_all_subsets():
    rng = np.random.default_rng(1)
    for trial in range(60):
        nb = int(rng.integers(1, 11))
        K = int(rng.integers(1, 9))
        scores = rng.integers(0, 4, nb).astype(np.float32)     # many ties
        if trial % 3 == 0:
            scores = rng.random(nb).astype(np.float32)
        got = oracle.topk_row(scores, K)
        assert list(got) == _brute_topk(scores, K), (scores, K)


def test_topk_matches_lexsort_at_scale():
    rng = np.random.default_rng(8)
    scores = rng.integers(0, 50, 5000).astype(np.float32)
    got = oracle.topk_row(scores, 512)
    order = np.lexsort((np.arange(5000), -scores))           # score desc, index asc
    assert np.array_equal(got, np.sort(order[:512]))


def test_topk_special_cases():
    assert list(oracle.topk_row(np.zeros(20, np.float32), 5)) == [0, 1, 2, 3, 4]
    assert list(oracle.topk_row(np.ones(3, np.float32), 5)) == [0, 1, 2, -1, -1]
    perm = np.random.default_rng(0).permutation(100).astype(np.float32)
    assert np.array_equal(oracle.topk_row(perm, 10), np.sort(np.nonzero(perm >= 90)[0]))


# ------------------------------------------------------------------ tokens
def test_token_set_membership_and_size():
    rng = np.random.default_rng(6)
    for _ in range(50):
        r = int(rng.choice([1, 2, 4, 8]))
        K = int(rng.integers(1, 9))
        L = int(rng.integers(1, 120))
        nb = L // r
        sel = np.sort(rng.choice(nb, min(K, nb), replace=False)) if nb else np.array([], int)
        idx = np.full(K, -1, np.int32)
        idx[: len(sel)] = sel
        toks = oracle.token_set(idx, r, L)
        expect = [t for t in range(L) if (t // r in set(sel.tolist())) or t >= nb * r]
        assert toks.tolist() == expect
        if nb > K:
            assert len(toks) == min(L, K * r + L % r)
        assert len(toks) <= K * r + r - 1


# --------------------------------------------------------------- attention
def _sdpa_ref(q, Kr, Vr, tokens, scale):
    Hq = q.shape[0]
    Hkv = Kr.shape[1]
    G = Hq // Hkv
    k = torch.from_numpy(Kr[tokens].astype(np.float64)).repeat_interleave(G, dim=1)   # [T,Hq,D]
    v = torch.from_numpy(Vr[tokens].astype(np.float64)).repeat_interleave(G, dim=1)
    qq = torch.from_numpy(q.astype(np.float64))[:, None, :]                           # [Hq,1,D]
    scale = float(np.float32(scale))          # the method takes the scale as an fp32 argument
    o = torch.nn.functional.scaled_dot_product_attention(
        qq, k.transpose(0, 1).contiguous(), v.transpose(0, 1).contiguous(), scale=scale)
    return o[:, 0, :].numpy()


def test_attention_matches_torch_sdpa_fp64_with_gqa():
    rng = np.random.default_rng(12)
    Hq, Hkv, D, N = 8, 2, 32, 90
    q = rng.standard_normal((Hq, D)).astype(np.float32)
    Kr = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    Vr = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    toks = np.sort(rng.choice(N, 37, replace=False))
    got = oracle.attn(q, Kr, Vr, toks, 0.17)
    ref = _sdpa_ref(q, Kr, Vr, toks, 0.17)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(13)
    Hq, Hkv, D, N = 4, 1, 16, 20
    q = rng.standard_normal((Hq, D)).astype(np.float32)
    Kr = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    Vr = np.tile(rng.standard_normal((1, Hkv, D)).astype(np.float32), (N, 1, 1))
    toks = np.arange(0, N, 3)
    assert np.allclose(oracle.attn(q, Kr, Vr, toks, 0.3), np.tile(Vr[0], (Hq, 1)), atol=1e-12)
    Vr = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    one = oracle.attn(q, Kr, Vr, [7], 0.3)
    assert np.array_equal(one, np.tile(Vr[7, 0].astype(np.float64), (Hq, 1)))
    zero_q = oracle.attn(np.zeros_like(q), Kr, Vr, toks, 0.3)
    assert np.allclose(zero_q, np.tile(Vr[toks, 0].astype(np.float64).mean(0), (Hq, 1)), atol=1e-12)


# ---------------------------------------------------------------- pipeline
def test_inert_bound_dispatch_table_from_the_pages(page):
    ib = page["inert_bound"]
    assert ib["budget"] + ib["ratio"] - 1 == ib["value"] == 2051
    tab = page["dispatch_table"]
    spec = W.VERIFY
    wl = W.small(spec, lens=[2060], n_q=[1], seed=31)
    kc, _ = oracle.compress(wl.k_idx.float().numpy(), wl.kv_offsets, 4, "bf16")
    kcv = oracle.kc_values(kc, "bf16")
    Kr, Vr = wl.K.float().numpy(), wl.V.float().numpy()
    K = 2048 // 4
    for L, dense in zip(tab["seq_len"], tab["dense"]):
        idx, _, out = oracle.run_queries(Kr, Vr, kcv, None, wl.q.float().numpy(),
                                         wl.q_idx.float().numpy(), wl.w.numpy(), [L], 4, 2048,
                                         spec.softmax_scale)
        nb = L // 4
        is_identity = list(idx[0][:min(nb, K)]) == list(range(min(nb, K)))
        toks = oracle.token_set(idx[0], 4, L)
        if dense:
            assert is_identity and len(toks) == L
            ref = oracle.dense_attn(wl.q[0].float().numpy(), Kr, Vr, L, spec.softmax_scale)
            assert np.array_equal(out[0], ref)           # bitwise: same fp64 loop, same order
        else:
            assert len(toks) == K * 4 + L % 4 < L
            assert not np.array_equal(np.sort(toks), np.arange(L))
    assert len(oracle.token_set(np.arange(K, dtype=np.int32), 4, 2051)) == \
        page["selection_width"]["value"]


def test_budget_covering_prefix_is_dense_attention():
    spec = W.TINY_DECODE
    wl = W.small(spec, lens=[300], n_q=[5], seed=2)
    kc, _ = oracle.compress(wl.k_idx.numpy(), wl.kv_offsets, 4, "f32")
    Kr, Vr = wl.K.numpy(), wl.V.numpy()
    L = wl.visible_lengths()
    for budget in (300, 512, 2048):
        _, _, out = oracle.run_queries(Kr, Vr, kc, None, wl.q.numpy(), wl.q_idx.numpy(),
                                       wl.w.numpy(), L, 4, budget, spec.softmax_scale)
        for i in range(5):
            ref = oracle.dense_attn(wl.q[i].numpy(), Kr, Vr, int(L[i]), spec.softmax_scale)
            assert np.array_equal(out[i], ref)


def test_sparse_pipeline_equals_masked_dense_attention_from_torch():
    # Selection from a brute-force top-k over the oracle's scores, attention
    # from torch's fp64 SDPA with a boolean mask: two independent routines.
    spec = W.VERIFY
    wl = W.small(spec, lens=[150, 97], n_q=[4, 3], seed=17, budget=32)
    kc, _ = oracle.compress(wl.k_idx.float().numpy(), wl.kv_offsets, 4, "bf16")
    kcv = oracle.kc_values(kc, "bf16")
    res = oracle.run_workload(wl, want_scores=True)
    K = 32 // 4
    Ls = wl.visible_lengths()
    qseq = wl.query_seq()
    blk = wl.blk_offsets()
    for i in range(wl.total_q):
        s = int(qseq[i])
        L = int(Ls[i])
        nb = L // 4
        scores = res["scores"][i]
        assert len(scores) == nb
        assert np.array_equal(scores, oracle.score_row(
            wl.q_idx[i].float().numpy(), wl.w[i].numpy(), kcv[blk[s]:blk[s] + nb]))
        order = np.lexsort((np.arange(nb), -scores))
        chosen = set(order[:K].tolist()) if nb > K else set(range(nb))
        mask = np.array([(t // 4 in chosen) or t >= nb * 4 for t in range(L)])
        a, b = int(wl.kv_offsets[s]), int(wl.kv_offsets[s + 1])
        Kr, Vr = wl.K[a:b].float().numpy(), wl.V[a:b].float().numpy()
        ref = _sdpa_ref(wl.q[i].float().numpy(), Kr, Vr, np.nonzero(mask)[0], spec.softmax_scale)
        assert np.allclose(res["out"][i], ref, rtol=1e-12, atol=1e-13)


def test_chunked_equals_single_shot_and_decode_equals_prefill_row():
    spec = W.CHUNKED_PREFILL
    wl = W.small(spec, lens=[600], n_q=[40], seed=5, budget=256)
    allq = oracle.run_workload(wl)
    first = oracle.run_workload(wl, query_ids=np.arange(0, 17))
    second = oracle.run_workload(wl, query_ids=np.arange(17, 40))
    assert np.array_equal(np.concatenate([first["idx"], second["idx"]]), allq["idx"])
    assert np.array_equal(np.concatenate([first["out"], second["out"]]), allq["out"])
    last = oracle.run_workload(wl, query_ids=[39])
    assert np.array_equal(last["idx"][0], allq["idx"][39])
    assert np.array_equal(last["out"][0], allq["out"][39])


def test_indexer_memory_sizing_matches_page(page):
    m = page["indexer_bytes_per_sequence"]
    raw = m["tokens"] * m["head_dim"] * m["bytes_per_elem"]
    blocks = m["tokens"] // m["ratio"] * m["head_dim"] * m["bytes_per_elem"]
    assert round((raw + blocks) / 1e6, 1) == m["value_mb"]
    kc, _ = oracle.compress(np.zeros((m["tokens"] // 64, 128), np.float32),
                            np.array([0, m["tokens"] // 64]), m["ratio"], "bf16")
    assert kc.nbytes == m["tokens"] // 64 // m["ratio"] * m["head_dim"] * m["bytes_per_elem"]


# ------------------------------------------------------- fp4 index plane
# E2M1 magnitudes as the OCP microscaling format lists them, codes 0..7.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_the_format_table():
    vals = oracle.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert vals[:8].tolist() == E2M1_MAGNITUDES
    assert (-vals[8:]).tolist() == E2M1_MAGNITUDES
    assert np.signbit(vals[8])                      # code 8 is -0


@pytest.mark.parametrize("x,code", [
    (0.0, 0), (0.25, 0), (0.2500001, 1), (0.5, 1), (0.7499999, 1), (0.75, 2), (1.25, 2),
    (1.2500001, 3), (1.75, 4), (2.5, 4), (2.5000002, 5), (3.5, 6), (5.0, 6), (5.0000005, 7),
    (6.0, 7), (7.9, 7), (1e30, 7), (-0.1, 8), (-0.3, 9), (-5.0, 14), (-7.0, 15),
])
def test_e2m1_encode_midpoints_and_saturation(x, code):
    # midpoints between neighbours go to the even mantissa (code bit 0);
    # past 6 the nearest value is 6
    assert int(oracle.e2m1_encode(np.array([x], dtype=np.float32))[0]) == code


def test_e2m1_encode_is_nearest_on_random_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4000) * 3).astype(np.float32)
    got = oracle.e2m1_decode(oracle.e2m1_encode(x)).astype(np.float64)
    grid = np.array(E2M1_MAGNITUDES)
    best = np.min(np.abs(np.abs(x.astype(np.float64))[:, None] - grid[None, :]), axis=1)
    assert np.all(np.abs(np.abs(got) - np.abs(x)) == best)
    nz = got != 0
    assert np.all(np.sign(got[nz]) == np.sign(x[nz]))


def _floor_log2_by_search(a: float) -> int:
    n = 0
    while 2.0 ** n > a:
        n -= 1
    while 2.0 ** (n + 1) <= a:
        n += 1
    return n


def test_e8m0_exponent_is_floor_log2_minus_two():
    rng = np.random.default_rng(4)
    vals = list(np.float32(2.0) ** rng.integers(-140, 120, 60)) + \
        list(rng.random(60).astype(np.float32) * np.float32(2.0) ** rng.integers(-130, 100, 60))
    vals += [np.float32(1.0), np.nextafter(np.float32(1.0), np.float32(0)), np.float32(6.0),
             np.float32(1e-45), np.float32(3.4e38)]
    for a in vals:
        a = np.float32(a)
        if a == 0:
            continue
        want = min(max(_floor_log2_by_search(float(a)) - 2, -127), 127)
        assert oracle.e8m0_exponent(a) == want, a
    assert oracle.e8m0_exponent(0.0) == -127


def test_fp4_value_is_code_value_times_power_of_two():
    # every (code, scale byte) a stored row can hold: the E2M1 value of the
    # format table times 2^(e - 127), exact in fp32 (e = 0 is 2^-127).  The
    # scale exponent of an fp32 group is at most floor(log2 of the largest
    # float) - 2 = 125, so bytes past 252 never occur.
    tab = oracle.fp4_value_table()
    for c in range(16):
        mag = E2M1_MAGNITUDES[c & 7]
        for e in range(253):
            want = np.float32(math.ldexp(-mag if c & 8 else mag, e - 127))
            got = tab[c, e]
            assert got.view(np.uint32) == want.view(np.uint32), (c, e, got, want)


def test_fp4_compress_hand_worked_block():
    # ratio 1, 64 dims = two groups.  Group 0 holds 4 (amax 4: floor(log2) 2,
    # X = 0, scale 1) so its other values are coded as they are; group 1 is
    # group 0 times 2^-10 (X = -10).  Values: 4, 0.25 (tie -> 0), 0.75 (tie
    # -> 1.0), 2.5 (tie -> 2), 3.5 (tie -> 4), 5.5 (-> 6), -1.3 (-> -1.5),
    # -0.2 (-> -0), then zeros.
    g0 = np.zeros(32, dtype=np.float32)
    g0[:8] = [4.0, 0.25, 0.75, 2.5, 3.5, 5.5, -1.3, -0.2]
    x = np.concatenate([g0, g0 * np.float32(2.0 ** -10)])[None, :]
    kc, sc = oracle.compress(x, np.array([0, 1], dtype=np.int64), 1, "fp4")
    assert sc.tolist() == [[127, 117]]
    want = [6, 0, 2, 4, 6, 7, 11, 8] + [0] * 24
    codes = np.empty(64, dtype=np.uint8)
    codes[0::2], codes[1::2] = kc[0] & 15, kc[0] >> 4
    assert codes[:32].tolist() == want and codes[32:].tolist() == want
    v = oracle.kc_values(kc, "fp4", sc)[0]
    assert v[:8].tolist() == [4.0, 0.0, 1.0, 2.0, 4.0, 6.0, -1.5, -0.0]
    assert np.array_equal(v[32:], v[:32] * np.float32(2.0 ** -10))


def test_fp4_compress_error_bound_and_group_scales():
    # every decoded value is within half a grid step of the mean (one step of
    # 2 * 2^X past 6 * 2^X); each 32-dim group gets its own scale
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 128)).astype(np.float32)
    x[:, 32:64] *= 1000.0
    off = np.array([0, 40], dtype=np.int64)
    kc, sc = oracle.compress(x, off, 4, "fp4")
    mean, _ = oracle.compress(x, off, 4, "f32")
    v = oracle.kc_values(kc, "fp4", sc).astype(np.float64)
    X = np.repeat(sc.astype(np.int64) - 127, 32, axis=1)
    y = np.abs(mean.astype(np.float64)) / np.ldexp(1.0, X)
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    err = np.abs(v - mean) / np.ldexp(1.0, X)
    assert np.all(err <= np.maximum(step / 2, np.where(y > 6, y - 6, 0)) + 1e-12)
    assert np.all(sc[:, 1] >= sc[:, 0] + 8)   # x1000 is about 2^10 larger


# ------------------------------------------------- recent window kept
@pytest.mark.parametrize("idx,nb,w,want", [
    ([2, 5, 9, -1], 12, 3, [2, 5, 9, 10, 11, -1, -1]),          # disjoint: union adds 3
    ([1, 10, 11, -1], 12, 2, [1, 10, 11, -1, -1, -1]),          # window already selected
    ([3, 9, 10, -1], 12, 4, [3, 8, 9, 10, 11, -1, -1, -1]),     # partly selected
    ([0, 1, 2, 3], 4, 8, [0, 1, 2, 3] + [-1] * 8),              # dense row, window past block 0
    ([-1, -1], 0, 2, [-1, -1, -1, -1]),                          # no complete block yet
])
def test_window_union_hand_cases(idx, nb, w, want):
    assert oracle.window_union(np.array(idx), nb, w).tolist() == want


# ------------------------------------------- pooled token scores
def test_pool_scores_hand_cases():
    tok = np.array([1, 5, 2, 0, 0.5, 0.25, 0.125, 0.0625, 9, 9], dtype=np.float32)
    assert oracle.pool_scores(tok, 4, "max").tolist() == [5.0, 0.5]          # the tail 9, 9 is no block
    assert oracle.pool_scores(tok, 4, "mean").tolist() == [2.0, 0.234375]
    assert oracle.pool_scores(tok, 1, "max").tolist() == tok.tolist()         # ratio 1 is the identity
    # fp32 order: 2^24 + 1 + 1 loses both ones left to right, mean then 2^22
    big = np.array([2.0 ** 24, 1, 1, 0], dtype=np.float32)
    assert oracle.pool_scores(big, 4, "mean").tolist() == [2.0 ** 22]
