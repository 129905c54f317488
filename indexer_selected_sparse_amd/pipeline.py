"""Device-side driver of one pass of the method: buffers plus the four C-ABI
calls (compress once; then score -> top-k -> sparse attention per step).

Allocation and argument marshalling only; every step runs in libqsa's HIP
kernels.  Inputs are the varlen-packed tensors described in include/qsa.h.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

import numpy as np

from . import (INGEST_OK, MAX_LAYERS, QSA_POOL_MAX, QSA_POOL_MEAN, QSA_SCORE_CANONICAL, QSA_SCORE_MFMA,
               Batch, KeyRing, Paging, attn_layers_workspace_size, attn_workspace_size, compress_keys,
               decode_step, decode_step_workspace_size, index_score, index_score_lists, index_score_topk, ingest,
               ingest_index_score, ingest_index_score_lists, pool_scores, score_topk_workspace_size, sparse_attn_decode_lists,
               sparse_attn_decode, sparse_attn_decode_layers, sparse_attn_prefill, topk_blocks, topk_workspace_size)

_KC_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8,
             "fp4": torch.float4_e2m1fn_x2}


def alloc_kc(rows: int, d_idx: int, kind: str, device):
    """Compressed-key storage of `rows` blocks: (kc, kc_scale).  fp4 rows are
    d_idx/2 bytes of E2M1 pairs with d_idx/32 E8M0 scale bytes; e4m3 rows have
    one fp32 scale; the others none."""
    if kind == "fp4":
        kc = torch.empty((rows, d_idx // 2), dtype=torch.uint8, device=device).view(torch.float4_e2m1fn_x2)
        sc = torch.empty((rows, d_idx // 32), dtype=torch.uint8, device=device).view(torch.float8_e8m0fnu)
        return kc, sc
    kc = torch.empty((rows, d_idx), dtype=_KC_TORCH[kind], device=device)
    return kc, (torch.empty(rows, dtype=torch.float32, device=device) if kind == "e4m3" else None)


@dataclass
class IngestState:
    """What a decode step appends: each sequence's newest token (position
    N_s - 1), its raw indexer key into the ring, its K/V rows into the caches."""
    ring: KeyRing
    k_new: torch.Tensor                 # [B, d_idx] raw indexer keys
    k_row: torch.Tensor                 # [B, hkv, d]
    v_row: torch.Tensor                 # [B, hkv, d]
    status: torch.Tensor                # int32 [B]


@dataclass
class DeviceProblem:
    batch: Batch
    ratio: int
    budget: int
    softmax_scale: float
    K: torch.Tensor
    V: torch.Tensor
    k_idx: torch.Tensor
    q: torch.Tensor
    q_idx: torch.Tensor
    w: torch.Tensor
    kc: torch.Tensor
    kc_scale: Optional[torch.Tensor]
    scores: torch.Tensor
    idx: torch.Tensor
    out: torch.Tensor
    attn_ws: Optional[torch.Tensor]
    topk_ws: Optional[torch.Tensor]        # certified (matrix-core scores) selection
    topk_ws_canon: Optional[torch.Tensor]  # selection from canonical scores
    decode: bool
    paging: Optional[Paging] = None        # K, V, k_idx, kc (+ scale) are page pools
    ing: Optional[IngestState] = None      # set by attach_ingest()
    local_blocks: int = 0                  # recent complete blocks always kept (set_local_blocks())
    token_pool: Optional[int] = None       # QSA_POOL_*: block scores pooled from token scores
    tok_scores: Optional[torch.Tensor] = None
    fuse_ingest: bool = True               # append + canonical scores in one launch when possible
    sel_ws: Optional[torch.Tensor] = None  # qsa_index_score_topk workspace
    fuse_select: bool = True               # canonical scores and their top-k in one call when possible
    step_ws: Optional[torch.Tensor] = None # qsa_decode_step workspace
    fuse_step: bool = True                 # decode: scores, selection and attention as qsa_decode_step

    @property
    def blocks_per_query(self) -> int:
        return self.budget // self.ratio

    def compress(self, stream=None) -> None:
        compress_keys(self.k_idx, self.ratio, self.batch, self.kc, self.kc_scale, stream=stream,
                      paging=self.paging)

    def ingest(self, stream=None) -> None:
        """Append every sequence's newest token (qsa_ingest, one token per
        sequence): ring commit, the block it completes, its K/V rows."""
        st = self.ing
        ingest(st.k_new, self.ratio, self.batch, st.ring, self.kc, self.kc_scale,
               kv=(st.k_row, st.v_row, self.K, self.V), status=st.status, stream=stream,
               paging=self.paging)

    def ingest_fusable(self, mode: int = QSA_SCORE_CANONICAL) -> bool:
        """Whether the append and the scores can run as one qsa_ingest_index_score
        launch: a decode batch, canonical scores on compressed keys, a bf16
        query and bf16 / e4m3 / fp4 keys."""
        return (self.fuse_ingest and self.ing is not None and self.batch.q_offsets is None
                and mode == QSA_SCORE_CANONICAL and self.token_pool is None
                and self.q_idx.dtype == torch.bfloat16 and self.kc.dtype != torch.float32)

    def ingest_step_fusable(self, mode: int = QSA_SCORE_CANONICAL) -> bool:
        """Whether a decode step with the append can run as
        qsa_ingest_index_score_lists + qsa_sparse_attn_decode_lists."""
        return (self.fuse_step and self.ingest_fusable(mode) and self.step_ws is not None
                and self.local_blocks == 0)

    def ingest_score_lists(self, stream=None) -> None:
        """qsa_ingest_index_score_lists: the append, the scores and the candidate
        lists; attend_lists() selects and attends."""
        st = self.ing
        ingest_index_score_lists(st.k_new, st.ring, self.q_idx, self.w, self.kc, self.kc_scale, self.q, self.K,
                                 self.V, self.softmax_scale, self.budget, self.ratio, self.batch, self.scores,
                                 self.step_ws, kv=(st.k_row, st.v_row, self.K, self.V), status=st.status,
                                 stream=stream, paging=self.paging)

    def ingest_score(self, stream=None) -> None:
        """qsa_ingest_index_score: ingest() and score() in one launch."""
        st = self.ing
        ingest_index_score(st.k_new, self.ratio, self.batch, st.ring, self.q_idx, self.w, self.kc,
                           self.kc_scale, self.scores, kv=(st.k_row, st.v_row, self.K, self.V),
                           status=st.status, stream=stream, paging=self.paging)

    def score(self, mode: int = QSA_SCORE_CANONICAL, stream=None) -> None:
        if self.token_pool is not None:
            # every token scored on its raw key (ratio 1: kc rows are k_idx rows),
            # then each block of `ratio` tokens pooled
            bt = self.batch
            tb = Batch(bt.kv_offsets, bt.kv_offsets, bt.q_offsets, bt.total_q, bt.max_kv_len,
                       bt.max_q_per_seq)
            index_score(self.q_idx, self.w, self.k_idx, None, 1, tb, self.tok_scores, stream=stream,
                        paging=self.paging)
            pool_scores(self.tok_scores, self.ratio, self.token_pool, bt, self.scores, stream=stream)
            return
        index_score(self.q_idx, self.w, self.kc, self.kc_scale, self.ratio, self.batch, self.scores,
                    mode=mode, stream=stream, paging=self.paging)

    def select_fusable(self, mode: int = QSA_SCORE_CANONICAL) -> bool:
        """Whether scores and selection can run as one qsa_index_score_topk
        call (canonical scores on compressed keys, no window)."""
        return (self.fuse_select and mode == QSA_SCORE_CANONICAL and self.token_pool is None
                and self.local_blocks == 0)

    def score_topk(self, stream=None) -> None:
        """qsa_index_score_topk: score() and topk() in one call."""
        index_score_topk(self.q_idx, self.w, self.kc, self.kc_scale, self.budget, self.ratio, self.batch,
                         self.scores, self.idx, self.sel_ws, stream=stream, paging=self.paging)

    def step_fusable(self, mode: int = QSA_SCORE_CANONICAL) -> bool:
        """Whether a decode step can run as qsa_decode_step (decode batch,
        canonical scores on compressed keys, no window, no fused append)."""
        return (self.decode and self.fuse_step and self.select_fusable(mode) and not self.ingest_fusable(mode)
                and self.ing is None and self.step_ws is not None)

    def decode_step(self, stream=None) -> None:
        """qsa_decode_step: scores, selection and sparse attention."""
        decode_step(self.q_idx, self.w, self.kc, self.kc_scale, self.q, self.K, self.V, self.softmax_scale,
                    self.budget, self.ratio, self.batch, self.scores, self.idx, self.out, self.step_ws,
                    stream=stream, paging=self.paging)

    def score_lists(self, stream=None) -> None:
        """qsa_index_score_lists: the scorer half of decode_step()."""
        index_score_lists(self.q_idx, self.w, self.kc, self.kc_scale, self.q, self.K, self.V, self.softmax_scale,
                          self.budget, self.ratio, self.batch, self.scores, self.step_ws, stream=stream,
                          paging=self.paging)

    def attend_lists(self, stream=None) -> None:
        """qsa_sparse_attn_decode_lists: the selection + attention half of decode_step()."""
        sparse_attn_decode_lists(self.q, self.K, self.V, self.softmax_scale, self.budget, self.ratio, self.batch,
                                 self.scores, self.idx, self.out, self.step_ws, stream=stream, paging=self.paging)

    def topk(self, certified: bool = False, stream=None) -> None:
        recheck = (self.q_idx, self.w, self.kc, self.kc_scale) if certified else None
        topk_blocks(self.scores, self.budget, self.ratio, self.batch, self.idx, recheck=recheck,
                    ws=self.topk_ws if certified else self.topk_ws_canon, stream=stream,
                    local_blocks=self.local_blocks)

    def attend(self, stream=None) -> None:
        fn = sparse_attn_decode if self.decode else sparse_attn_prefill
        fn(self.q, self.K, self.V, self.softmax_scale, self.idx, self.budget + self.local_blocks * self.ratio,
           self.ratio, self.batch, self.out, self.attn_ws, stream=stream, paging=self.paging)

    def step(self, mfma: bool = False, stream=None) -> None:
        """One pass of the hot path: [ingest ->] score -> top-k -> sparse attention."""
        mode = QSA_SCORE_MFMA if mfma else QSA_SCORE_CANONICAL
        if self.step_fusable(mode):
            self.decode_step(stream=stream)
            return
        if self.ingest_step_fusable(mode):
            self.ingest_score_lists(stream=stream)
            self.attend_lists(stream=stream)
            return
        if self.ingest_fusable(mode):
            self.ingest_score(stream=stream)
            self.topk(certified=mfma, stream=stream)
        else:
            if self.ing is not None:
                self.ingest(stream=stream)
            if self.select_fusable(mode):
                self.score_topk(stream=stream)
            else:
                self.score(mode, stream=stream)
                self.topk(certified=mfma, stream=stream)
        self.attend(stream=stream)


def upload(wl, device: str = "cuda", decode: Optional[bool] = None, mfma_ws: bool = False) -> DeviceProblem:
    """Copy a `qsa_workloads.Workload` to the device and allocate outputs."""
    sp = wl.spec
    if decode is None:
        decode = all(n == 1 for n in wl.n_q)
    q_lens = None if decode else wl.n_q
    batch = Batch.from_lengths(wl.lens, q_lens, ratio=sp.ratio, device=device)
    nb_tot = int(sum(n // sp.ratio for n in wl.lens))
    d_idx = sp.d_idx
    kc, kc_scale = alloc_kc(max(nb_tot, 1), d_idx, sp.kc_dtype, device)
    ld = max(1, (max(wl.lens) + sp.ratio - 1) // sp.ratio)
    tq = wl.total_q
    K = wl.K.to(device)
    V = wl.V.to(device)
    q = wl.q.to(device)
    dp = DeviceProblem(
        batch=batch, ratio=sp.ratio, budget=sp.budget, softmax_scale=sp.softmax_scale,
        K=K, V=V, k_idx=wl.k_idx.to(device), q=q, q_idx=wl.q_idx.to(device), w=wl.w.to(device),
        kc=kc, kc_scale=kc_scale,
        scores=torch.zeros((max(tq, 1), ld), dtype=torch.float32, device=device),
        idx=torch.full((max(tq, 1), sp.budget // sp.ratio), -7, dtype=torch.int32, device=device),
        out=torch.zeros((max(tq, 1), sp.hq, sp.d), dtype=q.dtype, device=device),
        attn_ws=None, topk_ws=None, topk_ws_canon=None, decode=decode)
    nws = attn_workspace_size(q, K, V, sp.softmax_scale, sp.budget, sp.ratio, batch)
    if nws:
        dp.attn_ws = torch.empty(nws, dtype=torch.uint8, device=device)
    cws = topk_workspace_size(batch, sp.budget, sp.ratio, None)
    if cws:
        dp.topk_ws_canon = torch.empty(cws, dtype=torch.uint8, device=device)
    sws = score_topk_workspace_size(batch, sp.budget, sp.ratio)
    if sws:
        dp.sel_ws = torch.empty(sws, dtype=torch.uint8, device=device)
    if decode:
        dws = decode_step_workspace_size(q, K, V, sp.softmax_scale, sp.budget, sp.ratio, batch)
        dp.step_ws = torch.empty(max(dws, 1), dtype=torch.uint8, device=device)
    if mfma_ws:
        tws = topk_workspace_size(batch, sp.budget, sp.ratio,
                                  (dp.q_idx, dp.w, dp.kc, dp.kc_scale))
        if tws:
            dp.topk_ws = torch.empty(tws, dtype=torch.uint8, device=device)
    return dp


def page(dp: DeviceProblem, lens, page_size: int, seed: int = 0, extra_pages: int = 0) -> DeviceProblem:
    """A copy of `dp` whose K, V, k_idx and compressed keys live in page pools:
    the pages of every sequence at random physical pages (seeded), plus
    `extra_pages` unused pages.  `lens` are the sequences' token counts; the
    compressed keys are copied from dp.kc, so compress `dp` first (or call
    compress() on the result)."""
    P, r = int(page_size), dp.ratio
    lens = [int(n) for n in lens]
    npg = [(n + P - 1) // P for n in lens]
    num_pages = sum(npg) + int(extra_pages)
    rng = np.random.default_rng(seed)
    phys = rng.permutation(num_pages)[:sum(npg)]
    table = np.zeros((len(lens), max(1, max(npg))), dtype=np.int32)
    tok_rows, blk_rows, u = [], [], 0
    for s_, (n, m) in enumerate(zip(lens, npg)):
        table[s_, :m] = phys[u:u + m]
        u += m
        t = np.arange(n)
        tok_rows.append(table[s_, t // P].astype(np.int64) * P + t % P)
        b = np.arange(n // r)
        blk_rows.append(table[s_, b // (P // r)].astype(np.int64) * (P // r) + b % (P // r))
    dev = dp.K.device
    tok = torch.from_numpy(np.concatenate(tok_rows)).to(dev)
    blk = torch.from_numpy(np.concatenate(blk_rows)).to(dev)

    def pool(t: torch.Tensor, rows: int, idx: torch.Tensor) -> torch.Tensor:
        if t.dtype in (torch.float4_e2m1fn_x2, torch.float8_e8m0fnu):   # byte formats
            return pool(t.view(torch.uint8), rows, idx).view(t.dtype)
        p = torch.zeros((rows,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
        p.index_copy_(0, idx, t[:idx.numel()])
        return p

    out = DeviceProblem(**{**dp.__dict__})
    out.K = pool(dp.K, num_pages * P, tok)
    out.V = pool(dp.V, num_pages * P, tok)
    out.k_idx = pool(dp.k_idx, num_pages * P, tok)
    out.kc = pool(dp.kc, num_pages * (P // r), blk)
    out.kc_scale = None if dp.kc_scale is None else pool(dp.kc_scale, num_pages * (P // r), blk)
    out.paging = Paging(torch.from_numpy(table).to(dev), num_pages, P)
    return out


def attach_ingest(dp: DeviceProblem, wl, capacity: Optional[int] = None) -> DeviceProblem:
    """Give a decode problem a raw-key ring (`capacity` tokens per sequence,
    default 2*ratio), filled by one prefill-sized qsa_ingest of every token
    (which also rewrites kc exactly as compress() does), and the rows its
    steps re-append: the newest token of each sequence (its raw key and K/V
    rows, equal to what the caches already hold, so outputs are unchanged)."""
    if not dp.decode:
        raise ValueError("attach_ingest: decode problems only")
    r = dp.ratio
    cap = int(capacity or 2 * r)
    dev = dp.kc.device
    lens = [int(n) for n in wl.lens]
    B = len(lens)
    ring = KeyRing.empty(B, cap, wl.k_idx.shape[-1], dtype=wl.k_idx.dtype, device=dev)
    status = torch.full((B,), -1, dtype=torch.int32, device=dev)
    every = Batch.from_lengths(lens, lens, ratio=r, device=dev)
    ingest(wl.k_idx.to(dev), r, every, ring, dp.kc, dp.kc_scale, status=status, paging=dp.paging)
    torch.cuda.synchronize()
    if not bool((status == INGEST_OK).all()):
        raise RuntimeError(f"attach_ingest: ingest status {status.tolist()}")
    last = torch.tensor(np.cumsum(lens) - 1, dtype=torch.int64)
    dp.ing = IngestState(ring, wl.k_idx[last].to(dev).contiguous(), wl.K[last].to(dev).contiguous(),
                         wl.V[last].to(dev).contiguous(), status)
    return dp


def set_local_blocks(dp: DeviceProblem, local_blocks: int) -> DeviceProblem:
    """Keep the last `local_blocks` complete blocks of every query besides its
    top-k selection (qsa_topk_blocks_local): widens idx to budget/ratio +
    local_blocks entries and sizes the attention workspace for it."""
    dp.local_blocks = int(local_blocks)
    K2 = dp.budget // dp.ratio + dp.local_blocks
    dp.idx = torch.full((dp.idx.shape[0], K2), -7, dtype=torch.int32, device=dp.idx.device)
    nws = attn_workspace_size(dp.q, dp.K, dp.V, dp.softmax_scale, K2 * dp.ratio, dp.ratio, dp.batch)
    dp.attn_ws = torch.empty(nws, dtype=torch.uint8, device=dp.idx.device) if nws else None
    return dp


def set_token_pool(dp: DeviceProblem, mode: int) -> DeviceProblem:
    """Select blocks from pooled token scores instead of compressed keys
    (canonical token scores on the raw indexer keys, then qsa_pool_scores
    with QSA_POOL_MAX or QSA_POOL_MEAN, then the usual block top-k)."""
    if mode not in (QSA_POOL_MAX, QSA_POOL_MEAN):
        raise ValueError("mode must be QSA_POOL_MAX or QSA_POOL_MEAN")
    dp.token_pool = mode
    rows = dp.scores.shape[0]
    dp.tok_scores = torch.zeros((rows, max(1, dp.batch.max_kv_len)), dtype=torch.float32,
                                device=dp.scores.device)
    return dp


@dataclass
class LayerStack:
    """A decode step over several attention layers whose indexers are either
    full or shared (the first "llama.cpp vs Atlas" report, section (a)3: a
    shared layer reuses the top-k of the previous full layer).  Layer l is
    full when l % full_every == 0; a shared layer skips scoring and top-k and
    attends its own K/V with the selection of the last full layer before it.
    With `fused`, the decode attention of a full layer and the shared layers
    after it runs as one qsa_sparse_attn_decode_layers launch (up to
    MAX_LAYERS layers each; outputs bit-identical to per-layer calls)."""
    layers: List[DeviceProblem]
    full_every: int = 1
    fused: bool = True
    full: List[bool] = field(default_factory=list)
    groups: List[List[DeviceProblem]] = field(default_factory=list)
    heads: List[DeviceProblem] = field(default_factory=list)
    group_ws: Optional[torch.Tensor] = None

    def __post_init__(self):
        if self.full_every < 1:
            raise ValueError("full_every must be >= 1")
        if any(dp.ing is not None for dp in self.layers):
            raise ValueError("LayerStack runs score, top-k and attention only; append each layer's new tokens "
                             "(qsa_ingest) before its step")
        self.full = [l % self.full_every == 0 for l in range(len(self.layers))]
        src = None
        for dp, f in zip(self.layers, self.full):
            if f:
                src = dp
                self.groups.append([dp])
                self.heads.append(dp)
            else:   # a shared layer reads (and never writes) the full layer's selection
                if dp.idx.shape != src.idx.shape:
                    raise ValueError("shared layers need the full layer's selection width")
                dp.idx = src.idx
                if len(self.groups[-1]) == MAX_LAYERS:
                    self.groups.append([dp])
                else:
                    self.groups[-1].append(dp)
        if self.fused:
            need = max([self._group_ws_bytes(g) for g in self.groups] + [0])
            if need:
                self.group_ws = torch.empty(need, dtype=torch.uint8, device=self.layers[0].idx.device)

    def _fusable(self, g: List[DeviceProblem]) -> bool:
        h = g[0]
        if len(g) < 2 or not all(dp.decode for dp in g):
            return False
        same_pg = all((dp.paging is None) == (h.paging is None) for dp in g) and (
            h.paging is None or all(dp.paging.block_table.data_ptr() == h.paging.block_table.data_ptr()
                                    and dp.paging.num_pages == h.paging.num_pages
                                    and dp.paging.page_size == h.paging.page_size for dp in g))
        return same_pg and all(dp.budget + dp.local_blocks * dp.ratio == h.budget + h.local_blocks * h.ratio
                               and dp.ratio == h.ratio and dp.q.shape == h.q.shape and dp.K.shape[1:] == h.K.shape[1:]
                               and dp.q.dtype == h.q.dtype for dp in g)

    def _group_ws_bytes(self, g: List[DeviceProblem]) -> int:
        if not self._fusable(g):
            return 0
        h = g[0]
        return attn_layers_workspace_size(h.q, h.K, h.V, h.softmax_scale, len(g),
                                          h.budget + h.local_blocks * h.ratio, h.ratio, h.batch)

    def step(self, stream=None) -> None:
        for g in self.groups:
            h = g[0]
            full = any(h is x for x in self.heads)
            if full and len(g) == 1 and h.step_fusable():
                h.decode_step(stream=stream)     # a full layer alone: qsa_decode_step
                continue
            if full:                              # a full layer: its own selection first
                if h.select_fusable():
                    h.score_topk(stream=stream)
                else:
                    h.score(stream=stream)
                    h.topk(stream=stream)
            if self.fused and self._fusable(g):
                sparse_attn_decode_layers([(dp.q, dp.K, dp.V, dp.softmax_scale) for dp in g], h.idx,
                                          h.budget + h.local_blocks * h.ratio, h.ratio, h.batch,
                                          [dp.out for dp in g], self.group_ws, stream=stream, paging=h.paging)
            else:
                for dp in g:
                    dp.attend(stream=stream)
