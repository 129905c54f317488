"""Oracle of the per-step ingest and the rollback gate — TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this module; the product path never does.

What it models ("Agentic shootout" page, "Flash-Next support: vLLM vs
Atlas", section (a)6: one compressed key per completed group of `ratio`
tokens, raw keys of the open group held in a per-request circular buffer of
whole groups; "Atlas Flash-Next defect investigations" page, Defect 1 and
fix plan PR-F: a rollback lowers the length, the indexer state must follow
it or the rollback is declined):

- a sequence's history: the raw indexer key of every position 0 .. N-1 it
  currently holds (an append of n keys at length N leaves positions
  < N - n as they were and sets N - n .. N - 1);
- the compressed key of each block completed by an append: the mean of the
  block's raw keys, computed by the pinned `oracle.compress` on that block
  alone;
- the ring slot's window {lo, hi} of positions whose raw keys the ring still
  holds, with the rules of the library's contract: an append ending at N
  with first position start uses lo' = min(lo, start) when start <= hi, else
  start (positions were skipped); a block whose old keys fall below lo' is
  not compressed and the append reports LOST_KEYS; afterwards the window is
  {max(lo', N - capacity), N}.  The rollback gate to length N succeeds iff
  N <= hi and min(lo, N) <= ratio * floor(N / ratio), and then sets the
  window to {min(lo, N), N}.

Pure Python over small cases; the block mean is the C oracle's.  Pinned in
`tests/test_ingest_oracle.py` against a literal ring of tagged rows (each row
remembers the position it was last written for).
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from . import compress as _compress

OK, LOST_KEYS, BAD_SLOT, TOO_LONG, DECLINED = 0, 1, 2, 3, 4


class SlotOracle:
    """One ring slot and the sequence that uses it."""

    def __init__(self, d: int, ratio: int, capacity: int, kind: str):
        self.d, self.r, self.cap, self.kind = d, ratio, capacity, kind
        self.lo, self.hi = 0, 0
        self.hist = np.full((0, d), np.nan, dtype=np.float32)  # NaN = never written
        # block -> (stored row, scale(s) or None) as last written by an append:
        # one fp32 scale for e4m3, the d/32 E8M0 bytes for fp4
        self.kc: Dict[int, Tuple[np.ndarray, Optional[np.ndarray]]] = {}

    def _block(self, rows: np.ndarray):
        kc, sc = _compress(rows, np.array([0, self.r], dtype=np.int64), self.r, self.kind)
        return kc[0].copy(), (None if sc is None else np.array(sc[0]).copy())

    def ingest(self, N: int, new_keys: np.ndarray) -> int:
        """Append the rows of `new_keys` as positions N - n .. N - 1."""
        new_keys = np.asarray(new_keys, dtype=np.float32).reshape(-1, self.d)
        n = new_keys.shape[0]
        start = N - n
        if n < 0 or start < 0:
            return TOO_LONG
        lo_eff = min(self.lo, start) if start <= self.hi else start
        status = OK
        r = self.r
        for g in range(start // r, N // r):           # blocks this append completes
            b0 = g * r
            if b0 < start and lo_eff > b0:
                status = LOST_KEYS
                continue
            rows = np.empty((r, self.d), dtype=np.float32)
            for j in range(r):
                p = b0 + j
                rows[j] = new_keys[p - start] if p >= start else self.hist[p]
            self.kc[g] = self._block(rows)
        hist = np.full((N, self.d), np.nan, dtype=np.float32)
        keep = min(start, self.hist.shape[0])
        hist[:keep] = self.hist[:keep]
        hist[start:N] = new_keys
        self.hist = hist
        self.lo, self.hi = max(lo_eff, N - self.cap), N
        return status

    def rewind(self, N: int) -> int:
        lo2 = min(self.lo, N)
        if 0 <= N <= self.hi and lo2 <= (N // self.r) * self.r:
            self.lo, self.hi = lo2, N
            return OK
        return DECLINED

    def ring_positions(self):
        """Positions whose raw keys the ring holds, and where: {pos: row}."""
        return {p: p % self.cap for p in range(self.lo, self.hi)}
