"""Device-side driver of one pass of the method: buffers plus the four C-ABI
calls (compress once; then score -> top-k -> sparse attention per step).

Allocation and argument marshalling only; every step runs in libqsa's HIP
kernels.  Inputs are the varlen-packed tensors described in include/qsa.h.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import (QSA_SCORE_CANONICAL, QSA_SCORE_MFMA, Batch, attn_workspace_size, compress_keys,
               index_score, sparse_attn_decode, sparse_attn_prefill, topk_blocks,
               topk_workspace_size)

_KC_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}


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

    @property
    def blocks_per_query(self) -> int:
        return self.budget // self.ratio

    def compress(self, stream=None) -> None:
        compress_keys(self.k_idx, self.ratio, self.batch, self.kc, self.kc_scale, stream=stream)

    def score(self, mode: int = QSA_SCORE_CANONICAL, stream=None) -> None:
        index_score(self.q_idx, self.w, self.kc, self.kc_scale, self.ratio, self.batch, self.scores,
                    mode=mode, stream=stream)

    def topk(self, certified: bool = False, stream=None) -> None:
        recheck = (self.q_idx, self.w, self.kc, self.kc_scale) if certified else None
        topk_blocks(self.scores, self.budget, self.ratio, self.batch, self.idx, recheck=recheck,
                    ws=self.topk_ws if certified else self.topk_ws_canon, stream=stream)

    def attend(self, stream=None) -> None:
        fn = sparse_attn_decode if self.decode else sparse_attn_prefill
        fn(self.q, self.K, self.V, self.softmax_scale, self.idx, self.budget, self.ratio,
           self.batch, self.out, self.attn_ws, stream=stream)

    def step(self, mfma: bool = False, stream=None) -> None:
        """One pass of the hot path: score -> top-k -> sparse attention."""
        self.score(QSA_SCORE_MFMA if mfma else QSA_SCORE_CANONICAL, stream=stream)
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
    kc = torch.empty((max(nb_tot, 1), d_idx), dtype=_KC_TORCH[sp.kc_dtype], device=device)
    kc_scale = torch.empty(max(nb_tot, 1), dtype=torch.float32, device=device) \
        if sp.kc_dtype == "e4m3" else None
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
    if mfma_ws:
        tws = topk_workspace_size(batch, sp.budget, sp.ratio,
                                  (dp.q_idx, dp.w, dp.kc, dp.kc_scale))
        if tws:
            dp.topk_ws = torch.empty(tws, dtype=torch.uint8, device=device)
    return dp
