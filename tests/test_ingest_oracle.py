"""Pins for the ingest / rollback oracle (oracle/ingest.py), CPU only.

The oracle tracks each ring slot as a window of positions {lo, hi}.  Here it
is checked against things other than itself:

- a literal ring: `capacity` rows, each remembering the position it was last
  written for, read before it is written, exactly as the buffer of the pages'
  engine would behave; on every history that appends positions in order
  (with any rollbacks) both must report the same status for every append and
  rollback, and compress the same blocks from the same rows;
- hand-worked cases whose statuses, windows and block means are worked out
  in the comments below;
- invariants: appending keys in pieces equals appending them at once, and a
  rollback followed by re-appending the same keys changes nothing.
"""
import numpy as np
import pytest

import oracle
from oracle import ingest as OI


class TagRing:
    """A literal ring of `cap` rows tagged with the position each holds."""

    def __init__(self, d, r, cap, kind):
        self.d, self.r, self.cap, self.kind = d, r, cap, kind
        self.tags = [-1] * cap
        self.rows = np.zeros((cap, d), dtype=np.float32)
        self.kc = {}

    def _held(self, p):
        return self.tags[p % self.cap] == p

    def ingest(self, N, keys):
        n = len(keys)
        start = N - n
        status = OI.OK
        for g in range(start // self.r, N // self.r):
            rows = []
            for p in range(g * self.r, (g + 1) * self.r):
                if p >= start:
                    rows.append(keys[p - start])
                elif self._held(p):
                    rows.append(self.rows[p % self.cap].copy())
                else:
                    rows = None
                    break
            if rows is None:
                status = OI.LOST_KEYS
                continue
            kc, sc = oracle.compress(np.stack(rows), np.array([0, self.r], dtype=np.int64), self.r,
                                     self.kind)
            self.kc[g] = (kc[0].copy(), None if sc is None else np.array(sc[0]).copy())
        for p in range(start, N):                     # writes after every read
            self.tags[p % self.cap] = p
            self.rows[p % self.cap] = keys[p - start]
        return status

    def can_rewind(self, N):
        return all(self._held(p) for p in range((N // self.r) * self.r, N))


def _same_blocks(a, b):
    assert a.keys() == b.keys()
    for g in a:
        assert np.array_equal(a[g][0], b[g][0]), g
        assert (a[g][1] is None) == (b[g][1] is None), g
        if a[g][1] is not None:
            assert np.array_equal(a[g][1], b[g][1]), g


CONFIGS = [  # (ratio, capacity, d, kind)
    (4, 4, 8, "bf16"), (4, 8, 8, "f32"), (4, 12, 8, "e4m3"), (2, 6, 4, "bf16"),
    (8, 8, 4, "f32"), (1, 1, 4, "f32"), (1, 3, 4, "bf16"), (4, 16, 8, "e4m3"), (4, 8, 64, "fp4"),
]


@pytest.mark.parametrize("r,cap,d,kind", CONFIGS)
def test_window_oracle_matches_literal_ring(r, cap, d, kind):
    rng = np.random.default_rng(1000 * r + cap)
    orc, tag = OI.SlotOracle(d, r, cap, kind), TagRing(d, r, cap, kind)
    cur = 0
    n_lost = n_declined = 0
    for _ in range(400):
        if rng.random() < 0.15 and cur > 0:           # explicit rollback gate
            N = cur - int(rng.choice([1, 2, 3, 5, 9, 17]))
            N = max(N, 0)
            want = OI.OK if tag.can_rewind(N) else OI.DECLINED
            got = orc.rewind(N)
            assert got == want, (N, cur)
            if got == OI.OK:
                cur = N
            else:
                n_declined += 1
            continue
        drop = int(rng.choice([0, 0, 0, 0, 1, 2, 3, 5, 7, 11, 16]))
        start = max(cur - drop, 0)                    # an implicit rollback when drop > 0
        n = int(rng.choice([0, 1, 1, 1, 2, 3, 4, 5, 8, 13, 33]))
        keys = rng.standard_normal((n, d)).astype(np.float32)
        N = start + n
        st_t = tag.ingest(N, keys)
        st_o = orc.ingest(N, keys)
        assert st_o == st_t, (start, N)
        n_lost += st_o == OI.LOST_KEYS
        _same_blocks(orc.kc, tag.kc)
        assert orc.hi == N and orc.lo >= max(N - cap, 0)
        # the window never claims a key the literal ring no longer holds
        assert all(tag._held(p) for p in range(orc.lo, orc.hi))
        cur = N
    if r > 1 and cap < 3 * r:  # small rings must actually lose keys and decline rollbacks
        assert n_lost > 0 and n_declined > 0


def _const_rows(values, d=4):
    return np.repeat(np.asarray(values, dtype=np.float32)[:, None], d, axis=1)


def test_hand_worked_cases():
    d = 4
    # ratio 4, capacity 4.  12 keys (value = position) fill blocks 0..2; the
    # ring keeps positions 8..11.  A rollback to 7 needs positions 4..6 for
    # the open block 1: gone, so declined.  Appending one key at position 7
    # anyway (an implicit rollback) completes block 1 without them: LOST_KEYS,
    # and block 1 keeps its old mean (4+5+6+7)/4 = 5.5.
    o = OI.SlotOracle(d, 4, 4, "f32")
    assert o.ingest(12, _const_rows(range(12))) == OI.OK
    assert (o.lo, o.hi) == (8, 12)
    assert [float(o.kc[g][0][0]) for g in range(3)] == [1.5, 5.5, 9.5]
    assert o.rewind(7) == OI.DECLINED and (o.lo, o.hi) == (8, 12)
    assert o.ingest(8, _const_rows([107])) == OI.LOST_KEYS
    assert float(o.kc[1][0][0]) == 5.5
    assert (o.lo, o.hi) == (7, 8)          # lo' = min(8, 7) = 7; max(7, 8 - 4) = 7

    # ratio 4, capacity 8: the ring keeps 4..11, so a rollback to 9 is
    # accepted (block 2 needs position 8 only).  Re-appending 9..11 with
    # values 109..111 gives block 2 = (8 + 109 + 110 + 111)/4 = 84.5.
    o = OI.SlotOracle(d, 4, 8, "f32")
    assert o.ingest(12, _const_rows(range(12))) == OI.OK
    assert (o.lo, o.hi) == (4, 12)
    assert o.rewind(9) == OI.OK and (o.lo, o.hi) == (4, 9)
    assert o.ingest(12, _const_rows([109, 110, 111])) == OI.OK
    assert float(o.kc[2][0][0]) == 84.5 and float(o.kc[1][0][0]) == 5.5

    # skipped positions: after 0..3, an append of 6..7 (4 and 5 never
    # written) cannot complete block 1.
    o = OI.SlotOracle(d, 4, 8, "f32")
    assert o.ingest(4, _const_rows(range(4))) == OI.OK
    assert o.ingest(8, _const_rows([6, 7])) == OI.LOST_KEYS
    assert 1 not in o.kc and (o.lo, o.hi) == (6, 8)

    # an append longer than the ring: 2 keys, then 10 more through a ring of
    # 4.  Block 0 = (0 + 1 + 102 + 103)/4 = 51.5 reads 0 and 1 from the ring
    # before they are overwritten; blocks 1, 2 come from the new keys.
    o = OI.SlotOracle(d, 4, 4, "f32")
    assert o.ingest(2, _const_rows([0, 1])) == OI.OK
    assert 0 not in o.kc
    assert o.ingest(12, _const_rows(range(102, 112))) == OI.OK
    assert [float(o.kc[g][0][0]) for g in range(3)] == [51.5, 105.5, 109.5]
    assert (o.lo, o.hi) == (8, 12)

    # e4m3: block mean (1, -2, 0.5, 3) -> scale 3/448, codes of mean/scale.
    o = OI.SlotOracle(4, 1, 1, "e4m3")
    assert o.ingest(1, np.array([[1, -2, 0.5, 3]], dtype=np.float32)) == OI.OK
    row, scale = o.kc[0]
    assert scale == np.float32(3) / np.float32(448)
    assert row[3] == 0x7E   # 448: the largest finite E4M3FN code


@pytest.mark.parametrize("r,cap,kind", [(4, 4, "bf16"), (4, 8, "e4m3"), (2, 2, "f32")])
def test_piecewise_append_equals_one_append(r, cap, kind):
    rng = np.random.default_rng(7)
    d = 8
    keys = rng.standard_normal((97, d)).astype(np.float32)
    whole = OI.SlotOracle(d, r, cap, kind)
    assert whole.ingest(97, keys) == OI.OK
    parts = OI.SlotOracle(d, r, cap, kind)
    N = 0
    while N < 97:
        n = min(int(rng.integers(0, 9)), 97 - N)
        assert parts.ingest(N + n, keys[N:N + n]) == OI.OK
        N += n
    _same_blocks(whole.kc, parts.kc)
    assert (whole.lo, whole.hi) == (parts.lo, parts.hi)


@pytest.mark.parametrize("explicit", [True, False])
def test_rollback_then_same_keys_changes_nothing(explicit):
    rng = np.random.default_rng(11)
    d, r, cap = 8, 4, 12
    keys = rng.standard_normal((80, d)).astype(np.float32)
    ref = OI.SlotOracle(d, r, cap, "bf16")
    assert ref.ingest(80, keys) == OI.OK
    o = OI.SlotOracle(d, r, cap, "bf16")
    assert o.ingest(60, keys[:60]) == OI.OK
    for drop in (1, 3, 8, 9):                 # every depth the ring can follow (cap - r + 1 = 9)
        N = o.hi - drop
        if explicit:
            assert o.rewind(N) == OI.OK
        wrong = rng.standard_normal((drop + 2, d)).astype(np.float32)
        assert o.ingest(N + drop + 2, wrong) == OI.OK   # a branch that is then rolled back
        N2 = N + drop + 2 - (drop + 2)
        if explicit:
            assert o.rewind(N2) == OI.OK
        assert o.ingest(N2 + drop + 2, keys[N2:N2 + drop + 2]) == OI.OK
    assert o.ingest(80, keys[o.hi:80]) == OI.OK
    _same_blocks(ref.kc, o.kc)
