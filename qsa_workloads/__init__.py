"""Seeded synthetic inputs for indexer-selected sparse attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no pooling, scoring, selection or attention).  Both the
CPU oracle and the HIP path consume what it returns.

Workloads follow the five configurations of the method's headline evaluation
(tiny decode, batched decode, long-context decode with an e4m3 index plane,
chunked prefill, speculative verify across the inert bound).  No public dataset
is involved: every tensor is N(0,1) (weights U[0,1)) drawn from numpy's PCG64
with a fixed seed, then rounded to the storage dtype with round-to-nearest-even
(torch's cast).

Draw order for a workload (fixed, so that a seed pins every value):
  1. sequence lengths (only where they are random),
  2. for each sequence in order: K_s, V_s ~ N(0,1) of shape (N_s, Hkv, D),
     then k_idx_s ~ N(0,1) of shape (N_s, D_idx),
  3. q (sum n_q, Hq, D), then q_idx (sum n_q, H_idx, D_idx), both N(0,1),
  4. w ~ U[0,1) of shape (sum n_q, H_idx).

Layouts are row-major and varlen-packed with int64 offsets [B+1]:
  K, V: [sum N_s, Hkv, D]; k_idx: [sum N_s, D_idx];
  q: [sum n_q, Hq, D]; q_idx: [sum n_q, H_idx, D_idx]; w: [sum n_q, H_idx].
Sequence s holds N_s tokens; its n_q,s queries are its last n_q,s tokens.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Spec:
    """Shape and dtype description of one workload (no tensors)."""
    name: str
    seed: int
    lens: Optional[List[int]]          # N_s per sequence (None: drawn)
    n_q: int                           # queries per sequence (last n_q tokens)
    hq: int
    hkv: int
    d: int
    kv_dtype: str                      # "f32" | "bf16" (q, K, V, out)
    h_idx: int
    d_idx: int
    idx_dtype: str                     # "f32" | "bf16" (q_idx, k_idx)
    kc_dtype: str                      # "f32" | "bf16" | "e4m3" (compressed keys)
    ratio: int = 4
    budget: int = 2048
    len_range: Optional[tuple] = None  # (lo, hi) inclusive, drawn per sequence
    len_extra: int = 0                 # N_s = drawn + len_extra
    num_seqs: int = 1

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt(D) rounded to fp32.
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The five configurations.  Sizes, head counts and dtypes are those the
# method's evaluation names; seeds are 0..4 in order.
TINY_DECODE = Spec("tiny_decode_4096_f32", 0, [4096], 1, 8, 1, 128, "f32", 4, 64, "f32", "f32")
BATCHED_DECODE = Spec("batched_decode_32seq_8k-32k", 1, None, 1, 32, 4, 128, "bf16", 8, 128, "bf16", "bf16",
          len_range=(8192, 32768), num_seqs=32)
LONG_DECODE = Spec("long_decode_8x131072_e4m3", 2, [131072] * 8, 1, 64, 8, 128, "bf16", 8, 128, "bf16", "e4m3",
          num_seqs=8)
CHUNKED_PREFILL = Spec("chunked_prefill_8193q_on_32768", 3, [40961], 8193, 32, 4, 128, "bf16", 8, 128, "bf16", "bf16")
VERIFY = Spec("verify_16x4q_inert_boundary", 4, None, 4, 16, 2, 128, "bf16", 4, 64, "bf16", "bf16",
          len_range=(2040, 2060), len_extra=4, num_seqs=16)

CONFIGS = {"tiny_decode": TINY_DECODE, "batched_decode": BATCHED_DECODE, "long_decode": LONG_DECODE,
           "chunked_prefill": CHUNKED_PREFILL, "verify": VERIFY}


@dataclasses.dataclass
class Workload:
    spec: Spec
    lens: List[int]
    n_q: List[int]
    kv_offsets: np.ndarray      # int64 [B+1]
    q_offsets: np.ndarray       # int64 [B+1]
    K: torch.Tensor             # [sum N, Hkv, D] (kv dtype, CPU)
    V: torch.Tensor
    k_idx: torch.Tensor         # [sum N, D_idx] (idx dtype)
    q: torch.Tensor             # [sum n_q, Hq, D]
    q_idx: torch.Tensor         # [sum n_q, H_idx, D_idx]
    w: torch.Tensor             # [sum n_q, H_idx] f32

    @property
    def num_seqs(self) -> int:
        return len(self.lens)

    @property
    def total_q(self) -> int:
        return int(self.q_offsets[-1])

    def blk_offsets(self) -> np.ndarray:
        r = self.spec.ratio
        nb = np.array([n // r for n in self.lens], dtype=np.int64)
        return np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)

    def visible_lengths(self) -> np.ndarray:
        """L of every query: its own position + 1 (its key is already appended)."""
        out = []
        for n, nq in zip(self.lens, self.n_q):
            out.extend(range(n - nq + 1, n + 1))
        return np.asarray(out, dtype=np.int64)

    def query_seq(self) -> np.ndarray:
        return np.repeat(np.arange(self.num_seqs), self.n_q).astype(np.int64)


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(_TORCH_DTYPE[dtype]) if dtype != "f32" else t.clone()


def make(spec: Spec, lens: Optional[List[int]] = None, n_q: Optional[List[int]] = None,
         seed: Optional[int] = None) -> Workload:
    """Draw one workload.  `lens`/`n_q`/`seed` override the spec (small cases)."""
    rng = np.random.Generator(np.random.PCG64(spec.seed if seed is None else seed))
    if lens is None:
        if spec.lens is not None:
            lens = list(spec.lens)
        else:
            lo, hi = spec.len_range
            lens = [int(x) + spec.len_extra for x in rng.integers(lo, hi + 1, spec.num_seqs)]
    lens = [int(x) for x in lens]
    if n_q is None:
        n_q = [min(spec.n_q, n) for n in lens]
    assert len(n_q) == len(lens) and all(0 <= a <= b for a, b in zip(n_q, lens))

    Ks, Vs, kis = [], [], []
    for n in lens:
        Ks.append(_cast(rng.standard_normal((n, spec.hkv, spec.d), dtype=np.float32), spec.kv_dtype))
        Vs.append(_cast(rng.standard_normal((n, spec.hkv, spec.d), dtype=np.float32), spec.kv_dtype))
        kis.append(_cast(rng.standard_normal((n, spec.d_idx), dtype=np.float32), spec.idx_dtype))
    tq = int(sum(n_q))
    q = _cast(rng.standard_normal((tq, spec.hq, spec.d), dtype=np.float32), spec.kv_dtype)
    q_idx = _cast(rng.standard_normal((tq, spec.h_idx, spec.d_idx), dtype=np.float32), spec.idx_dtype)
    w = torch.from_numpy(rng.random((tq, spec.h_idx), dtype=np.float32))

    kv_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q_off = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int64)
    cat = (lambda xs, shape: torch.cat(xs) if xs else torch.zeros(shape))
    return Workload(spec, lens, list(n_q), kv_off, q_off,
                    cat(Ks, (0, spec.hkv, spec.d)), cat(Vs, (0, spec.hkv, spec.d)),
                    cat(kis, (0, spec.d_idx)), q, q_idx, w)


def small(spec: Spec, lens: List[int], n_q: Optional[List[int]] = None, seed: int = 123,
          **overrides) -> Workload:
    """A shrunken workload with the same dtypes/heads as `spec` (parity tests)."""
    sp = dataclasses.replace(spec, **overrides) if overrides else spec
    return make(sp, lens=lens, n_q=n_q, seed=seed)
