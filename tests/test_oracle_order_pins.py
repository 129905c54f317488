"""Pins on the oracle's fp32 evaluation order.

The canonical score and the block mean decide integers (the selection, the
stored key bits), so the oracle fixes one fp32 order for them: block means sum
the rows of a block left to right from +0; a score sums, per indexer head,
rounded products left to right over d from +0, multiplies by the e4m3 block
scale once after the dot, applies ReLU, and then sums rounded w_h * r_h left
to right over heads from +0, never with a fused multiply-add.  (The method's
pages fix no order: the plain left-to-right one is the reading taken, and the
kernels follow it.)

Every input below is hand-worked so that the left-to-right result differs
from the reversed order, a pairwise (tree) order, the exact (fp64) value and a
fused multiply-add, and the expected value is derived by hand in the comment
next to it.  The mutation tests then rebuild the oracle from its source with
one of those changes planted (on the CPU, in a temporary directory) and check
that the pins reject every such build.

CPU only.
"""
from __future__ import annotations

import ctypes
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "qsa_oracle.c")
FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", "-std=c99"]
P = ctypes.c_void_p
F32 = np.float32
TWO24 = 2.0 ** 24


def _bind(lib):
    lib.qo_compress.restype = ctypes.c_int
    lib.qo_compress.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    lib.qo_score_row.restype = ctypes.c_int
    lib.qo_score_row.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P]
    return lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _score(lib, q, w, k, scale=None):
    q = np.ascontiguousarray(q, dtype=F32)
    w = np.ascontiguousarray(w, dtype=F32)
    k = np.ascontiguousarray(np.atleast_2d(k), dtype=F32)
    sc = None if scale is None else np.ascontiguousarray(np.atleast_1d(scale), dtype=F32)
    H, D = q.shape
    out = np.zeros(k.shape[0], dtype=F32)
    assert lib.qo_score_row(_ptr(q), _ptr(w), _ptr(k), _ptr(sc), k.shape[0], H, D, _ptr(out)) == 0
    return out


def _mean_f32(lib, rows, ratio):
    x = np.ascontiguousarray(rows, dtype=F32)
    off = np.array([0, x.shape[0]], dtype=np.int64)
    blk = np.array([0, x.shape[0] // ratio], dtype=np.int64)
    out = np.zeros((x.shape[0] // ratio, x.shape[1]), dtype=F32)
    assert lib.qo_compress(_ptr(x), _ptr(off), _ptr(blk), 1, x.shape[1], ratio, 0, _ptr(out), None) == 0
    return out


# ------------------------------------------------------------- the pins
# Each pin returns a list of failure messages (empty = pinned value holds),
# so the same checks can be run against planted-mistake builds.

def pin_block_mean_order(lib):
    bad = []
    # ratio 4, rows 2^24, 1, 1, 2 in dim 0 (bf16-exact raw keys):
    #   left to right: 2^24+1 -> 2^24 (tie, even), +1 -> 2^24, +2 -> 2^24+2; /4 = 2^22 + 0.5
    #   reversed: 2+1+1 = 4, +2^24 = 2^24+4 -> 2^22+1; pairwise (2^24+1)+(1+2) -> 2^24+4
    #   -> 2^22+1; exact (2^24+4)/4 = 2^22+1.
    # dim 1 holds the same multiset in another row order (1, 2^24, 1, 2):
    #   left to right: 1+2^24 -> 2^24, +1 -> 2^24, +2 -> 2^24+2 -> 2^22+0.5 again.
    rows = np.zeros((4, 64), dtype=F32)
    rows[:, 0] = [TWO24, 1, 1, 2]
    rows[:, 1] = [1, TWO24, 1, 2]
    m = _mean_f32(lib, rows, 4)[0]
    if m[0] != F32(2.0 ** 22 + 0.5) or m[1] != F32(2.0 ** 22 + 0.5):
        bad.append(f"ratio-4 block mean {m[0]!r}, {m[1]!r}, expected 4194304.5 twice")
    # ratio 8, rows 2^24 then seven 1s:
    #   left to right: every +1 ties back to 2^24 -> 2^24; /8 = 2^21
    #   pairwise: 2^24, 2, 2, 2 -> 2^24+6 -> 2^21 + 0.75; reversed: 7 + 2^24 -> 2^24+8 -> 2^21+1;
    #   exact: 2^21 + 0.875.
    rows = np.zeros((8, 64), dtype=F32)
    rows[:, 5] = [TWO24] + [1] * 7
    m = _mean_f32(lib, rows, 8)[0]
    if m[5] != F32(2.0 ** 21):
        bad.append(f"ratio-8 block mean {m[5]!r}, expected 2097152.0")
    return bad


def pin_dot_order(lib):
    bad = []
    # D = 64, bf16-exact operands, products 2^24 then 63 products of 1
    # (q = [2^12, 1, ...], k = [2^12, 1, ...]):
    #   left to right: each +1 ties back to 2^24 -> 2^24
    #   reversed: 63 + 2^24 = 2^24+63 -> 2^24+64; pairwise -> 2^24+62; exact 2^24+63.
    q = np.zeros((4, 64), dtype=F32)
    q[1] = 1.0
    q[1, 0] = 2.0 ** 12
    k = np.ones(64, dtype=F32)
    k[0] = 2.0 ** 12
    s = _score(lib, q, [0, 1, 0, 0], k)[0]
    if s != F32(TWO24):
        bad.append(f"dot of 2^24 and 63 ones {s!r}, expected 16777216.0")
    # The ones first, then 2^24 (products 1 x 63, then 2^24 at d = 63):
    #   left to right: 63, then 63 + 2^24 -> 2^24+64 (tie between +62 and +64, even)
    q = np.zeros((1, 64), dtype=F32)
    q[0] = 1.0
    q[0, 63] = 2.0 ** 12
    k = np.ones(64, dtype=F32)
    k[63] = 2.0 ** 12
    s = _score(lib, q, [1], k)[0]
    if s != F32(TWO24 + 64):
        bad.append(f"dot of 63 ones then 2^24 {s!r}, expected 16777280.0")
    return bad


def pin_dot_no_fma(lib):
    bad = []
    # fp32 operands (the tiny decode workload's dtype): products
    #   p0 = -1 * (1 + 2^-11) = -(1 + 2^-11)       exact
    #   p1 = (1 + 2^-12)^2 = 1 + 2^-11 + 2^-24      rounds to 1 + 2^-11 (tie, even)
    # rounded product then sum: -(1+2^-11) + (1+2^-11) = +0 -> ReLU +0 -> score +0;
    # a fused multiply-add at d = 1 would keep 2^-24 and give a score of 2^-24.
    a = F32(1 + 2.0 ** -12)
    q = np.zeros((1, 64), dtype=F32)
    q[0, 0], q[0, 1] = -1.0, a
    k = np.zeros(64, dtype=F32)
    k[0], k[1] = F32(1 + 2.0 ** -11), a
    s = _score(lib, q, [1], k)[0]
    if s.view(np.uint32) != 0:
        bad.append(f"rounded-product dot gave {s!r}, expected +0 (a fused multiply-add gives 2^-24)")
    return bad


def pin_head_sum_order(lib):
    bad = []
    # H = 4, w = 1, head dots r = 2^24, 1, 1, 2 (one key row k = e0, q_h = r_h e0):
    #   left to right: 2^24 -> +1 -> 2^24 -> +1 -> 2^24 -> +2 -> 2^24+2
    #   reversed: 2+1+1 = 4 -> 2^24+4; pairwise (2^24+1) + (1+2) -> 2^24+4; exact 2^24+4.
    q = np.zeros((4, 64), dtype=F32)
    q[:, 0] = [TWO24, 1, 1, 2]
    k = np.zeros(64, dtype=F32)
    k[0] = 1.0
    s = _score(lib, q, [1, 1, 1, 1], k)[0]
    if s != F32(TWO24 + 2):
        bad.append(f"head sum of 2^24, 1, 1, 2 {s!r}, expected 16777218.0")
    return bad


def pin_head_sum_no_fma(lib):
    bad = []
    # H = 2, key row k = [1, 1, 0, ...], bf16-exact query rows:
    #   head 0: q = [1, 2^-11] -> r0 = 1 + 2^-11, w0 = -1 -> term -(1 + 2^-11)  exact
    #   head 1: q = [1, 2^-12] -> r1 = 1 + 2^-12, w1 = 1 + 2^-12
    #           w1 * r1 = 1 + 2^-11 + 2^-24 rounds to 1 + 2^-11 (tie, even)
    # rounded product then sum: +0; a fused multiply-add for head 1 gives 2^-24.
    q = np.zeros((2, 64), dtype=F32)
    q[0, 0], q[0, 1] = 1.0, 2.0 ** -11
    q[1, 0], q[1, 1] = 1.0, 2.0 ** -12
    k = np.zeros(64, dtype=F32)
    k[0] = k[1] = 1.0
    s = _score(lib, q, [-1.0, 1 + 2.0 ** -12], k)[0]
    if s.view(np.uint32) != 0:
        bad.append(f"head sum gave {s!r}, expected +0 (a fused multiply-add gives 2^-24)")
    return bad


def pin_scale_after_dot(lib):
    bad = []
    # e4m3 path: q = [2^16, 1, 1, 1] (bf16), key codes [256, 1, 1, 1], block scale 0.75:
    #   dot over codes, left to right: 2^24, then +1 three times (ties back) -> 2^24
    #   times the scale once: 2^24 * 0.75 = 12582912 (exact)
    #   scaling every product instead: 12582912 + 0.75 -> 12582913 -> ... -> 12582915.
    q = np.zeros((1, 64), dtype=F32)
    q[0, :4] = [2.0 ** 16, 1, 1, 1]
    k = np.zeros(64, dtype=F32)
    k[:4] = [256, 1, 1, 1]
    s = _score(lib, q, [1], k, scale=0.75)[0]
    if s != F32(12582912.0):
        bad.append(f"scaled dot {s!r}, expected 12582912.0")
    return bad


PINS = [pin_block_mean_order, pin_dot_order, pin_dot_no_fma, pin_head_sum_order,
        pin_head_sum_no_fma, pin_scale_after_dot]


@pytest.fixture(scope="module")
def olib():
    return _bind(oracle.lib())


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_holds_pin(olib, pin):
    assert pin(olib) == []


def test_python_binding_agrees_on_the_pinned_values():
    # the marshalling layer used by every other test reaches the same values
    q = np.zeros((4, 64), dtype=F32)
    q[:, 0] = [TWO24, 1, 1, 2]
    k = np.zeros((1, 64), dtype=F32)
    k[0, 0] = 1.0
    assert oracle.score_row(q, np.ones(4), k)[0] == F32(TWO24 + 2)
    rows = np.zeros((4, 64), dtype=F32)
    rows[:, 0] = [TWO24, 1, 1, 2]
    kc, _ = oracle.compress(rows, np.array([0, 4]), 4, "f32")
    assert kc[0, 0] == F32(2.0 ** 22 + 0.5)


# -------------------------------------------------------- planted mistakes
# (pattern in the oracle source, replacement, pin that must catch it)
MUTATIONS = [
    ("block mean summed in reverse row order",
     r"for \(int t = 0; t < ratio; \+\+t\) acc = acc \+ rows",
     "for (int t = ratio - 1; t >= 0; --t) acc = acc + rows", pin_block_mean_order),
    ("block mean summed pairwise",
     r"for \(int t = 0; t < ratio; \+\+t\) acc = acc \+ rows\[\(int64_t\)t \* d \+ j\];",
     "{ float pr[64]; int n = ratio; for (int t = 0; t < n; ++t) pr[t] = rows[(int64_t)t * d + j]; "
     "while (n > 1) { for (int t = 0; t < n / 2; ++t) pr[t] = pr[2 * t] + pr[2 * t + 1]; n /= 2; } "
     "acc = pr[0]; }", pin_block_mean_order),
    ("dot summed in reverse d order",
     r"for \(int j = 0; j < D; \+\+j\) \{\n(\s*)float p = q",
     r"for (int j = D - 1; j >= 0; --j) {\n\1float p = q", pin_dot_order),
    ("dot accumulated in double",
     r"float dot = 0\.0f;\n(\s*)for \(int j = 0; j < D; \+\+j\) \{\n(\s*)float p = q\[\(int64_t\)h \* D \+ j\] \* k\[j\];\n(\s*)dot = dot \+ p;",
     r"double dd = 0.0;\n\1for (int j = 0; j < D; ++j) {\n\2dd += (double)q[(int64_t)h * D + j] * k[j];\n\3}\n\3float dot = (float)dd; {",
     pin_dot_order),
    ("heads summed in reverse order",
     r"for \(int h = 0; h < H; \+\+h\) \{\n(\s*)float dot = 0\.0f;",
     r"for (int h = H - 1; h >= 0; --h) {\n\1float dot = 0.0f;", pin_head_sum_order),
    ("scale applied to every product",
     r"float p = q\[\(int64_t\)h \* D \+ j\] \* k\[j\];",
     "float p = q[(int64_t)h * D + j] * k[j]; if (has_scale) p = p * scale;", pin_scale_after_dot),
]


def _build_variant(tmp, name, src_text, extra_flags=()):
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *FLAGS, *extra_flags, c, "-o", so, "-lm"], check=True, capture_output=True)
    return _bind(ctypes.CDLL(so))


@pytest.fixture(scope="module")
def tmpdir_mut():
    d = tempfile.mkdtemp(prefix="qsa_oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("what,pat,rep,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_order_change_is_caught(tmpdir_mut, what, pat, rep, pin):
    src = open(SRC).read()
    mutated, n = re.subn(pat, rep, src)
    assert n == 1, f"mutation '{what}' did not apply to the oracle source"
    lib = _build_variant(tmpdir_mut, re.sub(r"\W+", "_", what), mutated)
    assert pin(lib) != [], f"the pin did not notice: {what}"


def test_planted_contraction_is_caught(tmpdir_mut):
    # the same source built to fuse multiply-adds (x86-64 FMA, contraction on)
    probe = subprocess.run(["gcc", "-mfma", "-x", "c", "-E", "-"], input="", capture_output=True, text=True)
    if probe.returncode != 0:
        pytest.skip("gcc cannot target FMA here")
    flags = [f for f in FLAGS if f != "-ffp-contract=off"]
    c = os.path.join(tmpdir_mut, "contract.c")
    so = os.path.join(tmpdir_mut, "contract.so")
    shutil.copy(SRC, c)
    subprocess.run(["gcc", *flags, "-mfma", "-ffp-contract=fast", c, "-o", so, "-lm"], check=True,
                   capture_output=True)
    lib = _bind(ctypes.CDLL(so))
    caught = pin_dot_no_fma(lib) + pin_head_sum_no_fma(lib)
    assert caught != [], "a contracting build passed the no-fused-multiply-add pins"
