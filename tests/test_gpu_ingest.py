"""Parity of qsa_ingest / qsa_ring_rewind with the ingest oracle (oracle/ingest.py).

Random histories of appends (decode-sized and prefill-sized), implicit
rollbacks (a shorter length on the next append) and explicit rollback gates
run on paged pools whose pages sit in random physical order.  After every
call, bit for bit: the per-sequence status codes, each ring slot's window,
every compressed key the oracle has written (stale ones included), the raw
keys the ring holds, and the K/V rows of every position.
"""
import numpy as np
import pytest
import torch

import indexer_selected_sparse_amd as Q
from oracle import ingest as OI

pytestmark = pytest.mark.gpu

DEV = "cuda"


def kc_torch_dtype(kind: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8, "fp4": torch.uint8}[kind]


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.float4_e2m1fn_x2, torch.float8_e8m0fnu):
        t = t.view(torch.uint8)
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def _oracle_row_bits(row: np.ndarray, kind: str) -> np.ndarray:
    if kind == "f32":
        return row.astype(np.float32).view(np.int32)
    if kind == "bf16":
        return row.astype(np.uint16).view(np.int16)
    return row.astype(np.uint8)


class Rig:
    """Paged pools, a ring with permuted slots, and one oracle per slot."""

    def __init__(self, B, max_len, page, ratio, cap, d_idx, k_dtype, kc_kind, hkv, seed):
        self.B, self.max_len, self.P, self.r, self.cap = B, max_len, page, ratio, cap
        self.d, self.k_dtype, self.kind, self.hkv = d_idx, k_dtype, kc_kind, hkv
        self.rng = np.random.default_rng(seed)
        g = torch.Generator().manual_seed(seed)
        pps = -(-max_len // page)
        self.num_pages = B * pps + 3
        table = self.rng.permutation(self.num_pages)[:B * pps].reshape(B, pps).astype(np.int32)
        self.table = table
        self.paging = Q.Paging(torch.from_numpy(table).to(DEV), self.num_pages, page)
        rows = self.num_pages * page
        brows = self.num_pages * (page // ratio)
        kct = kc_torch_dtype(kc_kind)
        # garbage everywhere a call must not write
        if kc_kind == "fp4":
            self.kc = torch.randint(0, 255, (brows, d_idx // 2), generator=g,
                                    dtype=torch.uint8).to(DEV).view(torch.float4_e2m1fn_x2)
            self.kc_scale = torch.randint(0, 255, (brows, d_idx // 32), generator=g,
                                          dtype=torch.uint8).to(DEV).view(torch.float8_e8m0fnu)
        elif kct == torch.uint8:
            self.kc = torch.randint(0, 255, (brows, d_idx), generator=g, dtype=torch.uint8).to(DEV)
            self.kc_scale = torch.randn(brows, generator=g).to(DEV)
        else:
            self.kc = torch.randn((brows, d_idx), generator=g).to(kct).to(DEV)
            self.kc_scale = None
        self.K = torch.randn((rows, hkv, 128), generator=g).to(torch.bfloat16).to(DEV) if hkv else None
        self.V = torch.randn((rows, hkv, 128), generator=g).to(torch.bfloat16).to(DEV) if hkv else None
        self.num_slots = B + 3
        self.slot_of = self.rng.permutation(self.num_slots)[:B].astype(np.int32)
        self.ring = Q.KeyRing(torch.randn((self.num_slots, cap, d_idx), generator=g).to(k_dtype).to(DEV),
                              torch.zeros((self.num_slots, 2), dtype=torch.int64, device=DEV),
                              torch.from_numpy(self.slot_of).to(DEV))
        self.orc = [OI.SlotOracle(d_idx, ratio, cap, kc_kind) for _ in range(B)]
        self.cur = [0] * B
        self.key_hist = [np.zeros((0, d_idx), np.float32) for _ in range(B)]
        self.kv_hist = [(np.zeros((0,) + ((hkv, 128) if hkv else (0,)), np.int16),) * 2 for _ in range(B)]
        self.status = torch.full((B,), -1, dtype=torch.int32, device=DEV)

    def batch(self, lens, news, one_each=False):
        """one_each: every sequence appends exactly one token, passed as a
        batch without q_offsets (the decode-step form)."""
        kv = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        qo = np.concatenate([[0], np.cumsum(news)]).astype(np.int64)
        kvt = torch.from_numpy(kv).to(DEV)
        blk = torch.zeros(self.B + 1, dtype=torch.int64, device=DEV)
        if one_each:
            assert all(n == 1 for n in news)
            return Q.Batch(kvt, blk, None, self.B, self.max_len, 1)
        return Q.Batch(kvt, blk, torch.from_numpy(qo).to(DEV), int(qo[-1]), self.max_len,
                       max(1, int(max(news))))

    def append(self, starts, news, one_each=False):
        lens = [s + n for s, n in zip(starts, news)]
        tot = int(sum(news))
        k_new = torch.randn((max(tot, 1), self.d)).to(self.k_dtype)
        kvn = None
        if self.hkv:
            kvn = (torch.randn((max(tot, 1), self.hkv, 128)).to(torch.bfloat16),
                   torch.randn((max(tot, 1), self.hkv, 128)).to(torch.bfloat16))
        b = self.batch(lens, news, one_each)
        self.status.fill_(-1)
        Q.ingest(k_new.to(DEV), self.r, b, self.ring, self.kc, self.kc_scale,
                 kv=None if kvn is None else (kvn[0].to(DEV), kvn[1].to(DEV), self.K, self.V),
                 status=self.status, paging=self.paging)
        want = []
        kf = k_new.float().numpy()
        u = 0
        for s in range(self.B):
            n = news[s]
            want.append(self.orc[s].ingest(lens[s], kf[u:u + n]))
            kh = np.zeros((lens[s], self.d), np.float32)
            kh[:starts[s]] = self.key_hist[s][:starts[s]]
            kh[starts[s]:] = kf[u:u + n]
            self.key_hist[s] = kh
            if self.hkv:
                hk, hv = self.kv_hist[s]
                nk = np.zeros((lens[s], self.hkv, 128), np.int16)
                nv = np.zeros_like(nk)
                nk[:starts[s]], nv[:starts[s]] = hk[:starts[s]], hv[:starts[s]]
                nk[starts[s]:] = _bits(kvn[0][u:u + n])
                nv[starts[s]:] = _bits(kvn[1][u:u + n])
                self.kv_hist[s] = (nk, nv)
            u += n
        self.cur = lens
        torch.cuda.synchronize()
        assert self.status.cpu().tolist() == want
        return want

    def rewind(self, lens):
        b = self.batch(lens, [0] * self.B)
        self.status.fill_(-1)
        Q.ring_rewind(b, self.r, self.ring, self.status)
        want = [self.orc[s].rewind(lens[s]) for s in range(self.B)]
        torch.cuda.synchronize()
        assert self.status.cpu().tolist() == want
        for s in range(self.B):
            if want[s] == OI.OK:
                self.cur[s] = lens[s]
        return want

    def check(self):
        win = self.ring.window.cpu().numpy()
        kc = self.kc.view(torch.uint8).cpu() if self.kind == "fp4" else self.kc.cpu()
        kcs = None if self.kc_scale is None else _bits(self.kc_scale)
        ring = _bits(self.ring.keys)
        bpp = self.P // self.r
        for s in range(self.B):
            o, sl = self.orc[s], self.slot_of[s]
            assert (win[sl, 0], win[sl, 1]) == (o.lo, o.hi), s
            for g, (row, sc) in o.kc.items():
                phys = int(self.table[s, g // bpp]) * bpp + g % bpp
                assert np.array_equal(_bits(kc[phys]), _oracle_row_bits(row, self.kind)), (s, g)
                if sc is not None and self.kind == "fp4":
                    assert np.array_equal(kcs[phys], sc), (s, g)
                elif sc is not None:
                    assert kcs[phys] == np.float32(sc).view(np.int32), (s, g)
            want = self.key_hist[s]
            for p in range(o.lo, o.hi):
                got = ring[sl, p % self.cap]
                exp = torch.from_numpy(want[p]).to(self.k_dtype)
                assert np.array_equal(got, _bits(exp)), (s, p)
            if self.hkv and self.cur[s]:
                t = np.arange(self.cur[s])
                rows = self.table[s, t // self.P].astype(np.int64) * self.P + t % self.P
                ridx = torch.from_numpy(rows).to(DEV)
                assert np.array_equal(_bits(self.K[ridx]), self.kv_hist[s][0][:self.cur[s]]), s
                assert np.array_equal(_bits(self.V[ridx]), self.kv_hist[s][1][:self.cur[s]]), s


CASES = [
    # (ratio, cap, d_idx, raw key dtype, kc kind, page, hkv)
    (4, 8, 128, torch.bfloat16, "bf16", 16, 4),
    (8, 16, 64, torch.float32, "e4m3", 32, 0),
    (4, 4, 128, torch.bfloat16, "f32", 8, 2),
    (2, 6, 128, torch.bfloat16, "bf16", 4, 1),
    (4, 12, 128, torch.bfloat16, "e4m3", 64, 8),
    (4, 8, 64, torch.bfloat16, "fp4", 16, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}_cap{c[1]}_d{c[2]}_{c[4]}_P{c[5]}_hkv{c[6]}"
                                             for c in CASES])
def test_ingest_histories_match_oracle(case):
    r, cap, d, kdt, kind, P, hkv = case
    rig = Rig(B=6, max_len=320, page=P, ratio=r, cap=cap, d_idx=d, k_dtype=kdt, kc_kind=kind, hkv=hkv,
              seed=r * 100 + cap)
    rng = rig.rng
    # prefill-sized first appends, from nothing
    rig.append([0] * rig.B, [int(x) for x in rng.integers(0, 90, rig.B)])
    rig.check()
    n_lost = 0
    for step in range(30):
        if step % 7 == 6:
            lens = [max(c - int(rng.choice([0, 1, 2, 5, 9, 13])), 0) for c in rig.cur]
            rig.rewind(lens)
            rig.check()
            continue
        starts, news = [], []
        for s in range(rig.B):
            drop = int(rng.choice([0, 0, 0, 0, 1, 3, 6, 10]))
            st = max(rig.cur[s] - drop, 0)
            n = int(rng.choice([0, 1, 1, 1, 2, 3, 5, 9, 26]))
            n = min(n, rig.max_len - st)
            starts.append(st)
            news.append(n)
        got = rig.append(starts, news)
        n_lost += sum(x == OI.LOST_KEYS for x in got)
        rig.check()
    if cap == r:
        assert n_lost > 0


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}_cap{c[1]}_d{c[2]}_{c[4]}_P{c[5]}_hkv{c[6]}"
                                             for c in CASES])
def test_decode_appends_match_oracle(case):
    """One token per sequence per call, passed without q_offsets (the
    single-token kernel), with implicit rollbacks and rollback gates."""
    r, cap, d, kdt, kind, P, hkv = case
    rig = Rig(B=7, max_len=200, page=P, ratio=r, cap=cap, d_idx=d, k_dtype=kdt, kc_kind=kind, hkv=hkv,
              seed=r * 31 + cap)
    rng = rig.rng
    rig.append([0] * rig.B, [int(x) for x in rng.integers(1, 40, rig.B)])
    n_lost = 0
    for step in range(60):
        if step % 9 == 8:
            rig.rewind([max(c - int(rng.choice([0, 1, 2, 3, 5, 9])), 1) for c in rig.cur])
            rig.check()
            continue
        starts = []
        for c in rig.cur:
            drop = int(rng.choice([0] * 8 + [1, 2, 3, 6, 11]))
            starts.append(min(max(c - drop, 0), rig.max_len - 1))
        got = rig.append(starts, [1] * rig.B, one_each=True)
        n_lost += sum(x == OI.LOST_KEYS for x in got)
        if step % 5 == 0:
            rig.check()
    rig.check()
    if cap == r and r > 1:
        assert n_lost > 0


def test_ingest_error_codes():
    r, P = 4, 16
    rig = Rig(B=4, max_len=64, page=P, ratio=r, cap=8, d_idx=128, k_dtype=torch.bfloat16, kc_kind="bf16",
              hkv=0, seed=3)
    rig.append([0] * 4, [10, 10, 10, 10])
    rig.check()
    kc_before = rig.kc.clone()
    win_before = rig.ring.window.clone()
    # slot out of range for sequence 1, beyond the block table for sequence 2,
    # more new tokens than the length for sequence 3: nothing of theirs written
    slots = rig.ring.slots.clone()
    slots[1] = rig.num_slots
    ring = Q.KeyRing(rig.ring.keys, rig.ring.window, slots)
    lens, news = [12, 12, 4 * P + 1, 2], [2, 2, 2, 5]
    kv = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    qo = np.concatenate([[0], np.cumsum(news)]).astype(np.int64)
    b = Q.Batch(torch.from_numpy(kv).to(DEV), torch.zeros(5, dtype=torch.int64, device=DEV),
                torch.from_numpy(qo).to(DEV), int(qo[-1]), 4 * P, 5)
    k_new = torch.randn((int(qo[-1]), 128)).to(torch.bfloat16).to(DEV)
    st = torch.full((4,), -1, dtype=torch.int32, device=DEV)
    Q.ingest(k_new, r, b, ring, rig.kc, None, status=st, paging=rig.paging)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [Q.INGEST_OK, Q.INGEST_BAD_SLOT, Q.INGEST_TOO_LONG, Q.INGEST_TOO_LONG]
    w0, w1 = win_before.cpu().numpy(), rig.ring.window.cpu().numpy()
    for s in (1, 2, 3):
        sl = rig.slot_of[s]
        assert (w0[sl] == w1[sl]).all()
    # sequence 0 completed block 2 (positions 8..11); no other block changed
    changed = (rig.kc != kc_before).any(dim=1).nonzero().flatten().cpu().tolist()
    phys0 = int(rig.table[0, 2 // (P // r)]) * (P // r) + 2 % (P // r)
    assert set(changed) <= {phys0}


@pytest.mark.parametrize("kind", ["bf16", "e4m3"])
@pytest.mark.parametrize("kdt,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 128),
                                   (torch.float32, 64)], ids=["bf16_d128", "bf16_d64", "f32_d128", "f32_d64"])
def test_contiguous_prefill_ingest_equals_compress(kind, kdt, d):
    """One append per sequence from length 0 on the contiguous layout: the
    compressed keys equal qsa_compress_keys over the same keys, bit for bit,
    and the ring ends with the last `cap` keys of every sequence.  Ratio 4
    takes the kernels' compile-time-ratio paths, for bf16 and fp32 raw keys
    of 64 and 128 dims (one and two values per lane)."""
    r, cap = 4, 8
    lens = [37, 4, 3, 130, 0, 64, 1031]
    g = torch.Generator().manual_seed(5)
    k_all = torch.randn((sum(lens), d), generator=g).to(kdt).to(DEV)
    b = Q.Batch.from_lengths(lens, lens, ratio=r, device=DEV)
    nb = sum(n // r for n in lens)
    kct = kc_torch_dtype(kind)
    ref = torch.zeros((nb, d), dtype=kct, device=DEV)
    got = torch.full((nb, d), 7, dtype=kct, device=DEV)
    rs = torch.zeros(nb, device=DEV) if kind == "e4m3" else None
    gs = torch.full((nb,), 5.0, device=DEV) if kind == "e4m3" else None
    Q.compress_keys(k_all, r, b, ref, rs)
    ring = Q.KeyRing.empty(len(lens), cap, d, dtype=kdt)
    st = torch.full((len(lens),), -1, dtype=torch.int32, device=DEV)
    Q.ingest(k_all, r, b, ring, got, gs, status=st)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [Q.INGEST_OK] * len(lens)
    assert torch.equal(_t_bits(got), _t_bits(ref))
    if rs is not None:
        assert torch.equal(gs.view(torch.int32), rs.view(torch.int32))
    off = np.concatenate([[0], np.cumsum(lens)])
    win = ring.window.cpu().numpy()
    for s, n in enumerate(lens):
        assert tuple(win[s]) == (max(n - cap, 0), n)
        for p in range(max(n - cap, 0), n):
            assert torch.equal(ring.keys[s, p % cap], k_all[off[s] + p])


def _t_bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.uint8)


def test_decode_loop_on_ingested_caches_equals_compressed_caches():
    """Prefill-sized appends, then decode appends one token at a time; the
    paged kc pool then equals qsa_compress_keys_paged over a full raw-key
    pool of the same history, and a decode step on it selects and attends
    identically."""
    r, cap, d, P, hkv, hq = 4, 8, 128, 64, 4, 32
    B = 5
    rig = Rig(B=B, max_len=3000, page=P, ratio=r, cap=cap, d_idx=d, k_dtype=torch.bfloat16, kc_kind="bf16",
              hkv=hkv, seed=17)
    lens0 = [2900, 2100, 2049, 2500, 2999 - 13]
    rig.append([0] * B, lens0)
    for _ in range(13):
        rig.append(list(rig.cur), [1] * B)
    rig.check()
    # the same history as a full raw-key pool, compressed in one pass
    rows = rig.num_pages * P
    kpool = torch.zeros((rows, d), dtype=torch.bfloat16)
    for s in range(B):
        t = np.arange(rig.cur[s])
        pr = rig.table[s, t // P].astype(np.int64) * P + t % P
        kpool[torch.from_numpy(pr)] = torch.from_numpy(rig.key_hist[s]).to(torch.bfloat16)
    kpool = kpool.to(DEV)
    b = Q.Batch.from_lengths(rig.cur, None, ratio=r, device=DEV)
    kc_ref = rig.kc.clone()
    Q.compress_keys(kpool, r, b, kc_ref, None, paging=rig.paging)
    torch.cuda.synchronize()
    for s in range(B):
        nb = rig.cur[s] // r
        g = np.arange(nb)
        bpp = P // r
        pr = torch.from_numpy(rig.table[s, g // bpp].astype(np.int64) * bpp + g % bpp).to(DEV)
        assert torch.equal(_t_bits(rig.kc[pr]), _t_bits(kc_ref[pr])), s
    # one decode step on the ingested caches (K/V were appended by ingest too)
    budget = 2048
    gq = torch.Generator().manual_seed(2)
    q = torch.randn((B, hq, 128), generator=gq).to(torch.bfloat16).to(DEV)
    q_idx = torch.randn((B, 8, d), generator=gq).to(torch.bfloat16).to(DEV)
    w = torch.rand((B, 8), generator=gq).to(DEV)
    ld = -(-max(rig.cur) // r)
    outs = []
    for kc in (rig.kc, kc_ref):
        scores = torch.zeros((B, ld), device=DEV)
        idx = torch.full((B, budget // r), -7, dtype=torch.int32, device=DEV)
        out = torch.zeros((B, hq, 128), dtype=torch.bfloat16, device=DEV)
        Q.index_score(q_idx, w, kc, None, r, b, scores, paging=rig.paging)
        nws = Q.topk_workspace_size(b, budget, r, None)
        tws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
        Q.topk_blocks(scores, budget, r, b, idx, ws=tws if nws else None)
        aws = torch.empty(Q.attn_workspace_size(q, rig.K, rig.V, 0.08838834764831845, budget, r, b),
                          dtype=torch.uint8, device=DEV)
        Q.sparse_attn_decode(q, rig.K, rig.V, 0.08838834764831845, idx, budget, r, b, out, aws,
                             paging=rig.paging)
        torch.cuda.synchronize()
        outs.append((idx.clone(), out.clone()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


@pytest.mark.parametrize("paged", [0, 64])
def test_decode_step_with_ingest_equals_step_without(paged):
    """attach_ingest() + a step that first re-appends every sequence's newest
    token gives the same selection and output as the plain step, eagerly and
    on every replay of a captured HIP graph."""
    import dataclasses

    import qsa_workloads as W
    from indexer_selected_sparse_amd import pipeline
    sp = dataclasses.replace(W.LONG_DECODE, budget=512)     # e4m3 compressed keys
    wl = W.make(sp, lens=[4001, 2222, 517, 1024, 8], seed=5)

    def problem():
        dp = pipeline.upload(wl, DEV, decode=True)
        dp.compress()
        return pipeline.page(dp, wl.lens, paged, seed=1) if paged else dp

    ref = problem()
    ref.step()
    dp = pipeline.attach_ingest(problem(), wl)
    for _ in range(2):
        dp.idx.fill_(-7)
        dp.out.zero_()
        dp.step()
        torch.cuda.synchronize()
        assert torch.equal(dp.idx, ref.idx)
        assert torch.equal(dp.out.view(torch.int16), ref.out.view(torch.int16))
        assert (dp.ing.status == Q.INGEST_OK).all()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dp.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dp.step()
    for _ in range(3):
        dp.idx.fill_(-7)
        dp.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dp.idx, ref.idx)
        assert torch.equal(dp.out.view(torch.int16), ref.out.view(torch.int16))
