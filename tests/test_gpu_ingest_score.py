"""qsa_ingest_index_score (the decode step's append and canonical scores in
one launch) against the two calls it replaces, qsa_ingest followed by
qsa_index_score, on two copies of the same state.  Random histories of
one-token appends with implicit rollbacks (blocks whose older keys the ring
lost), sequences pointed at an invalid ring slot, every compressed-key
format, both raw-key dtypes, paged and contiguous caches.  After every step,
bit for bit: scores, compressed keys and scales, ring keys and windows,
statuses and K/V rows.  (The two calls themselves are checked against the
oracle in test_gpu_ingest.py and the parity tests; the fused launch alone is
also checked against the ingest oracle and the score oracle below.)

The same histories also drive the two-launch step with ingest:
qsa_ingest_index_score_lists must leave every state tensor as
qsa_ingest_index_score does, and the selection and attention from its lists
must equal the whole-row top-k and the plain decode attention bit for bit,
on rows whose newest token completes a block with lost keys or an invalid
slot too."""
import numpy as np
import pytest
import torch

import indexer_selected_sparse_amd as Q
from tests.parity import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda"


def _bits(t):
    if t.dtype in (torch.float4_e2m1fn_x2, torch.float8_e8m0fnu):
        t = t.view(torch.uint8)
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


class State:
    def __init__(self, B, max_len, r, cap, d, H, k_dtype, kind, hkv, paged, seed, kv_dtype=torch.bfloat16):
        g = torch.Generator().manual_seed(seed)
        rng = np.random.default_rng(seed)
        self.B, self.max_len, self.r, self.d, self.H = B, max_len, r, d, H
        self.paged = paged
        if paged:
            P = max(16, 2 * r)
            pps = -(-max_len // P)
            num_pages = B * pps + 3
            table = rng.permutation(num_pages)[:B * pps].reshape(B, pps).astype(np.int32)
            self.paging = Q.Paging(torch.from_numpy(table).to(DEV), num_pages, P)
            rows, brows = num_pages * P, num_pages * (P // r)
        else:
            self.paging = None
            rows, brows = B * max_len, B * (max_len // r)
        if kind == "fp4":
            self.kc = torch.randint(0, 255, (brows, d // 2), generator=g, dtype=torch.uint8).to(DEV) \
                .view(torch.float4_e2m1fn_x2)
            self.kc_scale = torch.randint(100, 140, (brows, d // 32), generator=g, dtype=torch.uint8).to(DEV) \
                .view(torch.float8_e8m0fnu)
        elif kind == "e4m3":
            self.kc = torch.randint(0, 126, (brows, d), generator=g, dtype=torch.uint8).to(DEV)
            self.kc_scale = torch.rand(brows, generator=g).to(DEV)
        else:
            self.kc = torch.randn((brows, d), generator=g).to(torch.bfloat16).to(DEV)
            self.kc_scale = None
        self.K = torch.randn((rows, hkv, 128), generator=g).to(kv_dtype).to(DEV) if hkv else None
        self.V = torch.randn((rows, hkv, 128), generator=g).to(kv_dtype).to(DEV) if hkv else None
        self.kv_dtype = kv_dtype
        self.num_slots = B + 2
        self.ring = Q.KeyRing(torch.randn((self.num_slots, cap, d), generator=g).to(k_dtype).to(DEV),
                              torch.zeros((self.num_slots, 2), dtype=torch.int64, device=DEV),
                              torch.zeros(B, dtype=torch.int32, device=DEV))
        self.status = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        self.ld = -(-max_len // r) + 3
        self.scores = torch.full((B, self.ld), float("nan"), device=DEV)

    def clone(self):
        c = object.__new__(State)
        c.__dict__.update(self.__dict__)
        for n in ("kc", "kc_scale", "K", "V", "status", "scores"):
            t = getattr(self, n)
            setattr(c, n, None if t is None else t.clone())
        c.ring = Q.KeyRing(self.ring.keys.clone(), self.ring.window.clone(), self.ring.slots.clone())
        return c

    def batch(self, lens):
        kv = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)).to(DEV)
        blk = torch.from_numpy(np.concatenate([[0], np.cumsum([n // self.r for n in lens])]).astype(np.int64)).to(DEV)
        return Q.Batch(kv, blk, None, self.B, self.max_len, 1)

    def tensors(self):
        out = {"kc": self.kc, "K": self.K, "V": self.V, "status": self.status, "scores": self.scores,
               "ring": self.ring.keys, "window": self.ring.window}
        if self.kc_scale is not None:
            out["kc_scale"] = self.kc_scale
        return {k: v for k, v in out.items() if v is not None}


BF, F32 = torch.bfloat16, torch.float32
CASES = [  # (kind, k dtype, d, H, ratio, capacity, hkv, paged, K/V dtype)
    ("bf16", BF, 128, 8, 4, 8, 2, True, BF),
    ("e4m3", F32, 128, 16, 4, 12, 2, True, BF),
    ("fp4", BF, 128, 8, 4, 8, 0, True, BF),
    ("fp4", F32, 64, 4, 8, 16, 2, False, BF),
    ("e4m3", BF, 64, 1, 4, 4, 0, False, BF),
    ("bf16", F32, 64, 2, 16, 32, 1, False, BF),
    ("fp4", BF, 64, 16, 16, 16, 2, True, BF),
    ("bf16", BF, 128, 8, 4, 8, 16, True, F32),    # 8 KB K/V rows: copied, not held in registers
    ("e4m3", BF, 128, 8, 4, 8, 4, False, F32),    # 2 KB rows in registers
]


@pytest.mark.parametrize("kind,k_dtype,d,H,r,cap,hkv,paged,kv_dtype", CASES,
                         ids=[f"{c[0]}-{str(c[1])[6:]}-d{c[2]}-h{c[3]}-r{c[4]}-{'paged' if c[7] else 'flat'}"
                              f"-kv{c[6]}x{str(c[8])[6:]}" for c in CASES])
def test_fused_equals_ingest_then_score(kind, k_dtype, d, H, r, cap, hkv, paged, kv_dtype):
    B, max_len = 6, 240
    seed = 17 * d + 3 * r + H + (1 if paged else 0) + hkv
    rng = np.random.default_rng(seed)
    a = State(B, max_len, r, cap, d, H, k_dtype, kind, hkv, paged, seed, kv_dtype)
    b = a.clone()
    slot_of = rng.permutation(a.num_slots)[:B].astype(np.int32)
    lens = [int(x) for x in rng.integers(1, 120, B)]
    g = torch.Generator().manual_seed(seed)
    n_stored = n_lost = n_bad = 0
    for step in range(48):
        for s in range(B):
            u = rng.random()
            # rates scale as 1/ratio, so that larger blocks still complete with all their keys
            if u < 0.4 / r and lens[s] > 2 * r:       # implicit rollback: a shorter N on this append
                lens[s] -= int(rng.integers(1, 2 * r))
            lens[s] = min(lens[s] + 1, max_len)
        slots = slot_of.copy()
        bad = rng.random(B) < 0.24 / r
        slots[bad] = -1
        n_bad += int(bad.sum())
        for st in (a, b):
            st.ring.slots.copy_(torch.from_numpy(slots))
        batch = a.batch(lens)
        k_new = torch.randn((B, d), generator=g).to(k_dtype).to(DEV)
        q_idx = torch.randn((B, H, d), generator=g).to(torch.bfloat16).to(DEV)
        w = torch.rand((B, H), generator=g).to(DEV)
        kvn = None
        if hkv:
            kvn = (torch.randn((B, hkv, 128), generator=g).to(kv_dtype).to(DEV),
                   torch.randn((B, hkv, 128), generator=g).to(kv_dtype).to(DEV))
        # the two calls
        Q.ingest(k_new, r, batch, a.ring, a.kc, a.kc_scale,
                 kv=None if kvn is None else (kvn[0], kvn[1], a.K, a.V), status=a.status, paging=a.paging)
        Q.index_score(q_idx, w, a.kc, a.kc_scale, r, batch, a.scores, paging=a.paging)
        # one launch
        Q.ingest_index_score(k_new, r, batch, b.ring, q_idx, w, b.kc, b.kc_scale, b.scores,
                             kv=None if kvn is None else (kvn[0], kvn[1], b.K, b.V), status=b.status,
                             paging=b.paging)
        torch.cuda.synchronize()
        ta, tb = a.tensors(), b.tensors()
        for name in ta:
            assert np.array_equal(_bits(ta[name]), _bits(tb[name])), (step, name)
        st = a.status.cpu().numpy()
        done = np.array([n % r == 0 for n in lens])
        n_stored += int(((st == Q.INGEST_OK) & done).sum())
        n_lost += int((st == Q.INGEST_LOST_KEYS).sum())
    # the histories reached every path of the fused kernel
    assert n_stored > 0 and n_lost > 0 and n_bad > 0


LIST_CASES = [c for c in CASES if c[6] > 0]


@pytest.mark.parametrize("kind,k_dtype,d,H,r,cap,hkv,paged,kv_dtype", LIST_CASES,
                         ids=[f"{c[0]}-{str(c[1])[6:]}-d{c[2]}-h{c[3]}-r{c[4]}-{'paged' if c[7] else 'flat'}"
                              f"-kv{c[6]}x{str(c[8])[6:]}" for c in LIST_CASES])
def test_ingest_step_lists_on_histories(kind, k_dtype, d, H, r, cap, hkv, paged, kv_dtype):
    # qsa_ingest_index_score_lists against qsa_ingest_index_score on the same
    # histories (every state tensor bit for bit), then the selection and
    # attention from its lists (qsa_sparse_attn_decode_lists) against the
    # whole-row top-k and qsa_sparse_attn_decode on the other copy's scores.
    # Rows whose newest token completes a block take their last list entry
    # from the append's score, including blocks scored from the stored row
    # (lost keys, invalid slots).
    B, max_len, budget = 6, 240, 4 * r
    seed = 31 * d + 5 * r + H + (1 if paged else 0) + hkv
    rng = np.random.default_rng(seed)
    a = State(B, max_len, r, cap, d, H, k_dtype, kind, hkv, paged, seed, kv_dtype)
    b = a.clone()
    slot_of = rng.permutation(a.num_slots)[:B].astype(np.int32)
    lens = [int(x) for x in rng.integers(1, 120, B)]
    g = torch.Generator().manual_seed(seed)
    hq = 2 * hkv
    scale = 1.0 / np.sqrt(128.0)
    K_ = budget // r
    n_slot = 0
    for step in range(40):
        for s in range(B):
            if rng.random() < 0.4 / r and lens[s] > 2 * r:
                lens[s] -= int(rng.integers(1, 2 * r))
            lens[s] = min(lens[s] + 1, max_len)
        slots = slot_of.copy()
        slots[rng.random(B) < 0.24 / r] = -1
        for st in (a, b):
            st.ring.slots.copy_(torch.from_numpy(slots))
        batch = a.batch(lens)
        k_new = torch.randn((B, d), generator=g).to(k_dtype).to(DEV)
        q_idx = torch.randn((B, H, d), generator=g).to(torch.bfloat16).to(DEV)
        w = torch.rand((B, H), generator=g).to(DEV)
        kvn = (torch.randn((B, hkv, 128), generator=g).to(kv_dtype).to(DEV),
               torch.randn((B, hkv, 128), generator=g).to(kv_dtype).to(DEV))
        q = torch.randn((B, hq, 128), generator=g).to(kv_dtype).to(DEV)
        ws = torch.empty(max(1, Q.decode_step_workspace_size(q, a.K, a.V, scale, budget, r, batch)),
                         dtype=torch.uint8, device=DEV)
        Q.ingest_index_score(k_new, r, batch, a.ring, q_idx, w, a.kc, a.kc_scale, a.scores,
                             kv=(kvn[0], kvn[1], a.K, a.V), status=a.status, paging=a.paging)
        Q.ingest_index_score_lists(k_new, b.ring, q_idx, w, b.kc, b.kc_scale, q, b.K, b.V, scale, budget, r, batch,
                                   b.scores, ws, kv=(kvn[0], kvn[1], b.K, b.V), status=b.status, paging=b.paging)
        torch.cuda.synchronize()
        ta, tb = a.tensors(), b.tensors()
        for name in ta:
            assert np.array_equal(_bits(ta[name]), _bits(tb[name])), (step, name)
        idx_a = torch.full((B, K_), -9, dtype=torch.int32, device=DEV)
        idx_b = torch.full((B, K_), -9, dtype=torch.int32, device=DEV)
        out_a = torch.zeros_like(q)
        out_b = torch.zeros_like(q)
        tws = Q.topk_workspace_size(batch, budget, r, None)
        Q.topk_blocks(a.scores, budget, r, batch, idx_a, ws=torch.empty(max(1, tws), dtype=torch.uint8, device=DEV))
        aws = Q.attn_workspace_size(q, a.K, a.V, scale, budget, r, batch)
        Q.sparse_attn_decode(q, a.K, a.V, scale, idx_a, budget, r, batch, out_a,
                             torch.empty(max(1, aws), dtype=torch.uint8, device=DEV), paging=a.paging)
        Q.sparse_attn_decode_lists(q, b.K, b.V, scale, budget, r, batch, b.scores, idx_b, out_b, ws,
                                   paging=b.paging)
        torch.cuda.synchronize()
        assert torch.equal(idx_a, idx_b), (step, "selection")
        assert np.array_equal(_bits(out_a), _bits(out_b)), (step, "outputs")
        n_slot += sum(1 for n in lens if n % r == 0 and n // r > K_)
    assert n_slot > 0


# ---------------------------------------------------------------------------
# The fused launch on its own against the oracles: the ingest oracle
# (oracle/ingest.py) for statuses, windows, ring rows, completed compressed
# keys and K/V rows, and the canonical-score oracle for every score of every
# row, computed from the compressed keys the row then holds.
from oracle import ingest as OI  # noqa: E402
import oracle as O  # noqa: E402

ORACLE_CASES = [  # (kind, k dtype, d, H, ratio, capacity, hkv, paged, B)
    ("bf16", BF, 128, 8, 4, 8, 2, True, 6),
    ("e4m3", F32, 128, 16, 4, 12, 2, True, 6),
    ("fp4", BF, 64, 4, 8, 16, 1, True, 5),
    ("e4m3", BF, 64, 2, 4, 8, 1, False, 1),
]


def _kind_name(kind):
    return {"bf16": "bf16", "e4m3": "e4m3", "fp4": "fp4"}[kind]


@pytest.mark.parametrize("kind,k_dtype,d,H,r,cap,hkv,paged,B", ORACLE_CASES,
                         ids=[f"{c[0]}-d{c[2]}-h{c[3]}-r{c[4]}-{'paged' if c[7] else 'flat'}" for c in ORACLE_CASES])
def test_fused_against_oracles(kind, k_dtype, d, H, r, cap, hkv, paged, B):
    max_len = 200
    seed = 1000 + 7 * d + r + H + B
    rng = np.random.default_rng(seed)
    st = State(B, max_len, r, cap, d, H, k_dtype, kind, hkv, paged, seed)
    slot_of = rng.permutation(st.num_slots)[:B].astype(np.int32)
    orc = {int(sl): OI.SlotOracle(d, r, cap, _kind_name(kind)) for sl in slot_of}
    lens = [0] * B
    g = torch.Generator().manual_seed(seed)
    seen = {"ok_block": 0, "lost": 0, "bad": 0}
    P = st.paging.page_size if paged else None
    tbl = st.paging.block_table.cpu().numpy() if paged else None

    def blk_row(s, b):
        if paged:
            per = P // r
            return int(tbl[s, b // per]) * per + b % per
        return b                       # B == 1: sequence 0's blocks start at row 0

    def tok_row(s, t):
        return int(tbl[s, t // P]) * P + t % P if paged else t

    for step in range(40):
        for s in range(B):
            if rng.random() < 0.35 / r and lens[s] > 2 * r:
                lens[s] -= int(rng.integers(1, 2 * r))
            lens[s] = min(lens[s] + 1, max_len)
        slots = slot_of.copy()
        bad = rng.random(B) < 0.2 / r
        slots[bad] = -1
        st.ring.slots.copy_(torch.from_numpy(slots))
        batch = st.batch(lens)
        k_new = torch.randn((B, d), generator=g).to(k_dtype)
        q_idx = torch.randn((B, H, d), generator=g).to(torch.bfloat16)
        w = torch.rand((B, H), generator=g)
        kvn = None
        if hkv:
            kvn = (torch.randn((B, hkv, 128), generator=g).to(BF), torch.randn((B, hkv, 128), generator=g).to(BF))
        st.status.fill_(-1)
        Q.ingest_index_score(k_new.to(DEV), r, batch, st.ring, q_idx.to(DEV), w.to(DEV), st.kc, st.kc_scale,
                             st.scores, kv=None if kvn is None else (kvn[0].to(DEV), kvn[1].to(DEV), st.K, st.V),
                             status=st.status, paging=st.paging)
        torch.cuda.synchronize()
        status = st.status.cpu().numpy()
        kc_host = _bits(st.kc)
        sc_host = None if st.kc_scale is None else _bits(st.kc_scale)
        win = st.ring.window.cpu().numpy()
        scores = st.scores.cpu().numpy()
        kf = k_new.float().numpy()
        for s in range(B):
            N = lens[s]
            if bad[s]:
                assert status[s] == OI.BAD_SLOT, (step, s, status[s])
                seen["bad"] += 1
            else:
                o = orc[int(slots[s])]
                want = o.ingest(N, kf[s:s + 1])
                assert status[s] == want, (step, s, status[s], want)
                assert win[slots[s]].tolist() == [o.lo, o.hi], (step, s, win[slots[s]], o.lo, o.hi)
                ring_keys = _bits(st.ring.keys[int(slots[s])])
                for p_, row in o.ring_positions().items():
                    want_row = o.hist[p_]
                    got_row = ring_keys[row]
                    exp_bits = (torch.from_numpy(want_row).to(k_dtype).view(torch.int16).numpy()
                                if k_dtype == BF else want_row.view(np.int32))
                    assert np.array_equal(got_row, exp_bits), (step, s, p_)
                if N % r == 0 and want == OI.OK:
                    b = N // r - 1
                    row_o, sc_o = o.kc[b]
                    got = kc_host[blk_row(s, b)]
                    exp = (row_o.astype(np.uint16).view(np.int16) if kind == "bf16" else row_o.astype(np.uint8))
                    assert np.array_equal(got, exp), (step, s, "completed block key")
                    if kind == "e4m3":
                        assert sc_host[blk_row(s, b)] == np.float32(sc_o).view(np.int32), (step, s, "scale")
                    elif kind == "fp4":
                        assert np.array_equal(sc_host[blk_row(s, b)], sc_o.astype(np.uint8)), (step, s, "scale")
                    seen["ok_block"] += 1
                seen["lost"] += int(want == OI.LOST_KEYS)
                if hkv:
                    kr = _bits(st.K[tok_row(s, N - 1)])
                    assert np.array_equal(kr, _bits(kvn[0][s])), (step, s, "K row")
            # every score of the row from the compressed keys it now holds
            nb = N // r
            if nb == 0:
                continue
            rows = np.array([blk_row(s, b) for b in range(nb)])
            if kind == "bf16":
                kv_ = O.kc_values(kc_host[rows].view(np.uint16), "bf16")
                dscale = None
            elif kind == "e4m3":
                kv_ = O.kc_values(kc_host[rows], "e4m3")
                dscale = sc_host[rows].view(np.float32)
            else:
                kv_ = O.kc_values(kc_host[rows], "fp4", sc_host[rows])
                dscale = None
            ref = O.score_row(q_idx[s].float().numpy(), w[s].numpy(), kv_, dscale)
            got = scores[s, :nb]
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (step, s, "scores")
    assert seen["ok_block"] > 0 and seen["lost"] > 0 and seen["bad"] > 0, seen
