"""CPU oracle for indexer-selected sparse attention — TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and it never imports them.

The arithmetic lives in `qsa_oracle.c` (plain C, fp32 canonical scores, fp64
attention); this module builds it with gcc and marshals numpy arrays.

Pins: every function here is checked by `tests/test_oracle_pins.py` against
things other than itself (library routines, closed forms, brute force).
The method as a whole has no printed worked example on its source pages:
end-to-end values are pinned only through those internal pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqsa_oracle.so")
_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
          "-std=c99", "-Wall", "-Wextra"]

KIND = {"f32": 0, "bf16": 1, "e4m3": 2, "fp4": 3}


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    cmd = ["gcc", *_FLAGS, _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.qo_bf16_round.restype = ctypes.c_uint16
        L.qo_bf16_round.argtypes = [ctypes.c_float]
        L.qo_bf16_to_f32.restype = ctypes.c_float
        L.qo_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.qo_e4m3_decode.restype = ctypes.c_float
        L.qo_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.qo_e4m3_encode.restype = ctypes.c_uint8
        L.qo_e4m3_encode.argtypes = [ctypes.c_float]
        L.qo_e2m1_decode.restype = ctypes.c_float
        L.qo_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.qo_e2m1_encode.restype = ctypes.c_uint8
        L.qo_e2m1_encode.argtypes = [ctypes.c_float]
        L.qo_e8m0_exponent.restype = i32
        L.qo_e8m0_exponent.argtypes = [ctypes.c_float]
        L.qo_fp4_value.restype = ctypes.c_float
        L.qo_fp4_value.argtypes = [ctypes.c_uint8, ctypes.c_uint8]
        L.qo_compress.restype = i32
        L.qo_compress.argtypes = [P, P, P, i32, i32, i32, i32, P, P]
        L.qo_score_row.restype = i32
        L.qo_score_row.argtypes = [P, P, P, P, i64, i32, i32, P]
        L.qo_topk_row.restype = i32
        L.qo_topk_row.argtypes = [P, i64, i32, P]
        L.qo_token_set.restype = i64
        L.qo_token_set.argtypes = [P, i32, i32, i64, P]
        L.qo_attn.restype = i32
        L.qo_attn.argtypes = [P, P, P, P, i64, i32, i32, i32, ctypes.c_float, P]
        L.qo_dense_attn.restype = i32
        L.qo_dense_attn.argtypes = [P, P, P, i64, i32, i32, i32, ctypes.c_float, P]
        L.qo_run_queries.restype = i32
        L.qo_run_queries.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P, i64,
                                     i32, i32, ctypes.c_float, P, P, i64, P, i32]
        L.qo_max_threads.restype = i32
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


# ------------------------------------------------------------------ codecs
def bf16_round_bits(x) -> np.ndarray:
    x = _f32(x).ravel()
    f = lib().qo_bf16_round
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def e4m3_decode(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().qo_e4m3_decode(c) for c in range(256)], dtype=np.float32)
    return table[codes]


def e2m1_decode(codes) -> np.ndarray:
    """Values of 4-bit E2M1 codes (one code per array element)."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().qo_e2m1_decode(c) for c in range(16)], dtype=np.float32)
    return table[codes & 15]


def e2m1_encode(x) -> np.ndarray:
    x = _f32(x)
    f = lib().qo_e2m1_encode
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


_FP4_TABLE = None


def fp4_value_table() -> np.ndarray:
    """[16, 256] float32: the exact value of E2M1 code c under E8M0 scale
    byte e (qo_fp4_value: code value times 2^(e - 127))."""
    global _FP4_TABLE
    if _FP4_TABLE is None:
        f = lib().qo_fp4_value
        _FP4_TABLE = np.array([[f(c, e) for e in range(256)] for c in range(16)], dtype=np.float32)
    return _FP4_TABLE


def e8m0_exponent(amax: float) -> int:
    return int(lib().qo_e8m0_exponent(float(amax)))


def e4m3_encode(x) -> np.ndarray:
    x = _f32(x)
    f = lib().qo_e4m3_encode
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


# ---------------------------------------------------------------- compress
def compress(k_idx, kv_offsets, ratio: int, kind: str):
    """Mean-pool complete blocks.  Returns (kc, scale): kc is float32 for
    "f32", uint16 bf16 bits for "bf16", uint8 codes for "e4m3" (scale: a
    float32 array), and for "fp4" uint8 [nb, d/2] bytes of two E2M1 codes
    (dim 2j in the low nibble of byte j) with uint8 [nb, d/32] E8M0 scale
    bytes; scale is None for "f32" and "bf16"."""
    x = _f32(k_idx)
    kv_off = np.ascontiguousarray(kv_offsets, dtype=np.int64)
    B = len(kv_off) - 1
    d = x.shape[1]
    nb = (np.diff(kv_off) // ratio).astype(np.int64)
    blk_off = np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)
    tot = int(blk_off[-1])
    dt = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8, "fp4": np.uint8}[kind]
    out = np.zeros((tot, d // 2 if kind == "fp4" else d), dtype=dt)
    scale = None
    if kind == "e4m3":
        scale = np.zeros(tot, dtype=np.float32)
    elif kind == "fp4":
        scale = np.zeros((tot, d // 32), dtype=np.uint8)
    rc = lib().qo_compress(_p(x), _p(kv_off), _p(blk_off), B, d, ratio, KIND[kind], _p(out),
                           _p(scale))
    _check(rc, "compress")
    return out, scale


def kc_values(kc, kind: str, scale=None) -> np.ndarray:
    """Exact fp32 values of stored compressed keys: the code values for e4m3
    (its per-block scale multiplies the dot afterwards); for fp4 each value
    is code value * 2^(E - 127) of its 32-dim group, exact in fp32."""
    if kind == "f32":
        return _f32(kc)
    if kind == "bf16":
        return bf16_bits_to_f32(kc)
    if kind == "fp4":
        kc = np.asarray(kc, dtype=np.uint8)
        nb, half = kc.shape
        codes = np.empty((nb, 2 * half), dtype=np.uint8)
        codes[:, 0::2] = kc & 15
        codes[:, 1::2] = kc >> 4
        exps = np.repeat(np.asarray(scale, dtype=np.uint8), 32, axis=1)
        return fp4_value_table()[codes, exps]
    return e4m3_decode(kc)


def score_scale(kc_scale, kind: str):
    """The per-block scale that multiplies the dot (e4m3 only; fp4 scales are
    folded into the key values by kc_values)."""
    return kc_scale if kind == "e4m3" else None


# ------------------------------------------------------------------- score
def score_row(q, w, kc_vals, kc_scale=None) -> np.ndarray:
    q = _f32(q)
    w = _f32(w)
    kc = _f32(kc_vals)
    H, D = q.shape
    nb = kc.shape[0]
    sc = None if kc_scale is None else _f32(kc_scale)
    out = np.zeros(nb, dtype=np.float32)
    _check(lib().qo_score_row(_p(q), _p(w), _p(kc), _p(sc), nb, H, D, _p(out)), "score")
    return out


def pool_scores(tok, ratio: int, mode: str) -> np.ndarray:
    """Block scores from token scores (the second "vLLM vs Atlas" report,
    section (a)3, block pooling): one per complete block, "max" of its
    tokens' scores, or "mean": their fp32 sum left to right from +0, times
    1/ratio (exact for a power of two)."""
    tok = _f32(tok)
    nb = len(tok) // ratio
    out = np.zeros(nb, dtype=np.float32)
    inv = np.float32(1.0) / np.float32(ratio)
    for b in range(nb):
        seg = tok[b * ratio:(b + 1) * ratio]
        if mode == "max":
            out[b] = max(seg)
        else:
            acc = np.float32(0.0)
            for v in seg:
                acc = np.float32(acc + v)
            out[b] = np.float32(acc * inv)
    return out


def topk_row(scores, K: int) -> np.ndarray:
    s = _f32(scores)
    out = np.zeros(K, dtype=np.int32)
    _check(lib().qo_topk_row(_p(s), len(s), K, _p(out)), "topk")
    return out


def window_union(idx, nb: int, local_blocks: int) -> np.ndarray:
    """A top-k row (ascending, -1 padded) with the last min(local_blocks, nb)
    complete blocks added: the ascending union, -1 padded to
    len(idx) + local_blocks entries (the second "llama.cpp vs Atlas"
    report, section (d), phase 3, item 6: the most recent tokens are kept as
    a union with the top-k set, here in whole blocks)."""
    keep = {int(b) for b in idx if b >= 0}
    keep |= set(range(max(nb - local_blocks, 0), nb))
    out = np.full(len(idx) + local_blocks, -1, dtype=np.int32)
    srt = sorted(keep)
    out[:len(srt)] = srt
    return out


def token_set(idx, ratio: int, L: int) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    K = len(idx)
    buf = np.zeros(K * ratio + ratio, dtype=np.int64)
    n = lib().qo_token_set(_p(idx), K, ratio, L, _p(buf))
    if n < 0:
        raise ValueError("oracle token_set rejected its arguments")
    return buf[:n].copy()


def attn(q, Kr, Vr, tokens, scale: float) -> np.ndarray:
    q = _f32(q)
    Kr = _f32(Kr)
    Vr = _f32(Vr)
    tok = np.ascontiguousarray(tokens, dtype=np.int64)
    Hq, D = q.shape
    Hkv = Kr.shape[1]
    out = np.zeros((Hq, D), dtype=np.float64)
    _check(lib().qo_attn(_p(q), _p(Kr), _p(Vr), _p(tok), len(tok), Hq, Hkv, D, scale, _p(out)),
           "attn")
    return out


def dense_attn(q, Kr, Vr, L: int, scale: float) -> np.ndarray:
    q = _f32(q)
    Kr = _f32(Kr)
    Vr = _f32(Vr)
    Hq, D = q.shape
    out = np.zeros((Hq, D), dtype=np.float64)
    _check(lib().qo_dense_attn(_p(q), _p(Kr), _p(Vr), L, Hq, Kr.shape[1], D, scale, _p(out)),
           "dense_attn")
    return out


def run_queries(Kr, Vr, kc_vals, kc_scale, q, q_idx, w, L, ratio: int, budget: int,
                scale: float, want_scores: bool = False, want_out: bool = True,
                n_threads: Optional[int] = None):
    """The whole method for some queries of one sequence (see qo_run_queries).
    Returns (idx [n,K] int32, scores [n, nb_seq] or None, out [n,Hq,D] f64 or None)."""
    Kr = _f32(Kr)
    Vr = _f32(Vr)
    kc = _f32(kc_vals)
    sc = None if kc_scale is None else _f32(kc_scale)
    q = _f32(q)
    q_idx = _f32(q_idx)
    w = _f32(w)
    L = np.ascontiguousarray(L, dtype=np.int64)
    n = len(L)
    N, Hkv, D = Kr.shape
    Hq = q.shape[1]
    H_idx, D_idx = q_idx.shape[1], q_idx.shape[2]
    K = budget // ratio
    nb_seq = N // ratio
    idx = np.zeros((n, K), dtype=np.int32)
    scores = np.zeros((n, max(nb_seq, 1)), dtype=np.float32) if want_scores else None
    out = np.zeros((n, Hq, D), dtype=np.float64) if want_out else None
    nt = n_threads or os.cpu_count() or 1
    rc = lib().qo_run_queries(_p(Kr), _p(Vr), _p(kc), _p(sc), N, Hq, Hkv, D, H_idx, D_idx,
                              _p(q), _p(q_idx), _p(w), _p(L), n, ratio, budget, scale, _p(idx),
                              _p(scores), max(nb_seq, 1), _p(out), nt)
    _check(rc, "run_queries")
    return idx, scores, out


def run_workload(wl, query_ids=None, want_scores=False, want_out=True, n_threads=None):
    """Run the oracle on a `qsa_workloads.Workload` (all queries, or the given
    global query indices).  Returns dict with kc (stored form), kc_scale,
    idx, scores (list of per-query arrays), out."""
    sp = wl.spec
    kc, kc_scale = compress(wl.k_idx.float().numpy(), wl.kv_offsets, sp.ratio, sp.kc_dtype)
    kcv = kc_values(kc, sp.kc_dtype, kc_scale)
    dot_scale = score_scale(kc_scale, sp.kc_dtype)
    blk = wl.blk_offsets()
    Ls = wl.visible_lengths()
    qseq = wl.query_seq()
    if query_ids is None:
        query_ids = np.arange(wl.total_q)
    query_ids = np.asarray(query_ids, dtype=np.int64)
    K = sp.budget // sp.ratio
    idx_all = np.zeros((len(query_ids), K), dtype=np.int32)
    out_all = np.zeros((len(query_ids), sp.hq, sp.d), dtype=np.float64) if want_out else None
    scores_all = [None] * len(query_ids)
    for s in range(wl.num_seqs):
        sel = np.nonzero(qseq[query_ids] == s)[0]
        if len(sel) == 0:
            continue
        gq = query_ids[sel]
        a, b = int(wl.kv_offsets[s]), int(wl.kv_offsets[s + 1])
        Kr = wl.K[a:b].float().numpy()
        Vr = wl.V[a:b].float().numpy()
        ka, kb = int(blk[s]), int(blk[s + 1])
        idx, scores, out = run_queries(
            Kr, Vr, kcv[ka:kb], None if dot_scale is None else dot_scale[ka:kb],
            wl.q[gq].float().numpy(), wl.q_idx[gq].float().numpy(), wl.w[gq].numpy(), Ls[gq],
            sp.ratio, sp.budget, sp.softmax_scale, want_scores=want_scores, want_out=want_out,
            n_threads=n_threads)
        idx_all[sel] = idx
        if want_out:
            out_all[sel] = out
        if want_scores:
            for j, i in enumerate(sel):
                scores_all[i] = scores[j, : int(Ls[gq[j]]) // sp.ratio].copy()
    return {"kc": kc, "kc_scale": kc_scale, "idx": idx_all, "out": out_all,
            "scores": scores_all if want_scores else None}


def max_threads() -> int:
    return int(lib().qo_max_threads())
