"""C-ABI checks that need no GPU: the library loads, exports every entry point
that include/qsa.h declares, and rejects bad arguments on the host with the
documented status codes before touching a device (all pointers below are
never dereferenced)."""
import ctypes
import json
import os
import re

import pytest

import indexer_selected_sparse_amd as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a non-null address that validation never dereferences


def header_functions():
    txt = open(os.path.join(ROOT, "include", "qsa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_\w+)\s*\(", txt)))


def _header_prototypes():
    """name -> parameter count of every function qsa.h declares."""
    txt = open(os.path.join(ROOT, "include", "qsa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(qsa_\w+)\s*\(([^)]*)\)\s*;", txt):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_declares_every_signature():
    # ctypes passes an undeclared integer argument as a 32-bit int; a 64-bit
    # parameter (a leading dimension, a byte count) would then carry garbage
    # in its upper half, so every function must have its argument types
    L = Q.lib()
    protos = _header_prototypes()
    assert set(protos) == set(Q.EXPORTS)
    for name, n in protos.items():
        f = getattr(L, name)
        if n == 0:
            continue
        assert f.argtypes is not None, f"{name}: no argtypes in the binding"
        assert len(f.argtypes) == n, f"{name}: {len(f.argtypes)} argtypes for {n} parameters"


def test_library_exports_every_declared_function():
    L = Q.lib()
    names = header_functions()
    assert len(names) == 30, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in qsa.h but not exported"
    assert set(names) == set(Q.EXPORTS)
    out = os.popen(f"nm -D --defined-only {Q.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_versions_and_inert_bound():
    assert Q.lib().qsa_abi_version() == 3
    assert "gfx950" in Q.version()
    with open(os.path.join(ROOT, "tests", "golden", "page_constants.json")) as f:
        page = json.load(f)
    ib = page["inert_bound"]
    assert Q.inert_bound(ib["budget"], ib["ratio"]) == ib["value"] == 2051
    assert Q.inert_bound(8192, 4) == 8195
    assert Q.inert_bound(0, 4) == -1 and Q.inert_bound(2048, 0) == -1


def _batch(**kw):
    d = dict(num_seqs=2, max_q_per_seq=1, total_q=2, max_kv_len=4096, kv_offsets=FAKE,
             blk_offsets=FAKE, q_offsets=None)
    d.update(kw)
    return Q._Batch(**d)


def _ix(**kw):
    d = dict(q_idx=FAKE, w=FAKE, kc=FAKE, kc_scale=None, q_dtype=Q.QSA_BF16,
             kc_dtype=Q.QSA_BF16, h_idx=8, d_idx=128)
    d.update(kw)
    return Q._Indexer(**d)


def _attn(**kw):
    d = dict(q=FAKE, k=FAKE, v=FAKE, dtype=Q.QSA_BF16, hq=32, hkv=4, d=128,
             softmax_scale=0.0883883)
    d.update(kw)
    return Q._Attn(**d)


def _err():
    return Q.lib().qsa_last_error().decode()


P = ctypes.c_void_p


def score(ix=None, ratio=4, b=None, scores=FAKE, ld=1024, flags=0):
    ix = ix or _ix()
    b = b or _batch()
    return Q.lib().qsa_index_score(ctypes.byref(ix), ratio, ctypes.byref(b), P(scores), ld, flags, None)


def topk(scores=FAKE, ld=1024, recheck=None, budget=2048, ratio=4, b=None, idx=FAKE, ws=None, nws=0):
    b = b or _batch()
    return Q.lib().qsa_topk_blocks(P(scores), ld, None if recheck is None else ctypes.byref(recheck),
                                   budget, ratio, ctypes.byref(b), P(idx), P(ws), nws, None)


def topk_local(local_blocks, budget=2048, ratio=4):
    b = _batch()
    return Q.lib().qsa_topk_blocks_local(P(FAKE), 1024, None, budget, ratio, local_blocks, ctypes.byref(b),
                                         P(FAKE), None, 0, None)


def decode(a=None, idx=FAKE, budget=2048, ratio=4, b=None, out=FAKE, ws=FAKE, nws=1 << 30):
    a = a or _attn()
    b = b or _batch()
    return Q.lib().qsa_sparse_attn_decode(ctypes.byref(a), P(idx), budget, ratio, ctypes.byref(b),
                                          P(out), P(ws), nws, None)


def prefill(a=None, idx=FAKE, budget=2048, ratio=4, b=None, out=FAKE, ws=None, nws=0):
    a = a or _attn()
    b = b or _batch()
    return Q.lib().qsa_sparse_attn_prefill(ctypes.byref(a), P(idx), budget, ratio,
                                           ctypes.byref(b), P(out), P(ws), nws, None)


def compress(k=FAKE, kdt=Q.QSA_BF16, d=128, ratio=4, b=None, kc=FAKE, kcdt=Q.QSA_BF16, scale=None):
    b = b or _batch()
    return Q.lib().qsa_compress_keys(P(k), kdt, d, ratio, ctypes.byref(b), None, P(kc), kcdt,
                                     P(scale), None)


def _pg(**kw):
    d = dict(block_table=FAKE, max_pages=64, num_pages=128, page_size=64)
    d.update(kw)
    return Q._PagedKV(**d)


def _ref(x):
    return None if x is None else ctypes.byref(x)


def score_paged(pg="default", flags=0, b=None):
    ix, b = _ix(), b or _batch(blk_offsets=None)
    pg = _pg() if pg == "default" else pg
    return Q.lib().qsa_index_score_paged(ctypes.byref(ix), 4, ctypes.byref(b), P(FAKE), 1024, flags,
                                         _ref(pg), None)


def decode_paged(pg="default"):
    a, b = _attn(), _batch(blk_offsets=None)
    pg = _pg() if pg == "default" else pg
    return Q.lib().qsa_sparse_attn_decode_paged(ctypes.byref(a), P(FAKE), 2048, 4, ctypes.byref(b),
                                                P(FAKE), P(FAKE), 1 << 30, _ref(pg), None)


def compress_paged(pg="default"):
    b = _batch(blk_offsets=None)
    pg = _pg() if pg == "default" else pg
    return Q.lib().qsa_compress_keys_paged(P(FAKE), Q.QSA_BF16, 128, 4, ctypes.byref(b), None, P(FAKE),
                                           Q.QSA_BF16, None, _ref(pg), None)


def _ring(**kw):
    d = dict(keys=FAKE, window=FAKE, slots=None, num_slots=2, capacity=8)
    d.update(kw)
    return Q._KeyRing(**d)


def _kv(**kw):
    d = dict(k_new=FAKE, v_new=FAKE, k=FAKE, v=FAKE, dtype=Q.QSA_BF16, hkv=4, d=128)
    d.update(kw)
    return Q._KvAppend(**d)


def ingest(ring="default", kv=None, kdt=Q.QSA_BF16, d=128, ratio=4, kcdt=Q.QSA_BF16, scale=None, pg=None,
           b=None, k_new=FAKE):
    b = b or _batch()
    ring = _ring() if ring == "default" else ring
    return Q.lib().qsa_ingest(P(k_new), kdt, d, ratio, ctypes.byref(b), _ref(ring), P(FAKE), kcdt, P(scale),
                              _ref(kv), None, _ref(pg), None)


def rewind(ring="default", ratio=4, b=None):
    b = b or _batch()
    ring = _ring() if ring == "default" else ring
    return Q.lib().qsa_ring_rewind(ctypes.byref(b), ratio, _ref(ring), None, None)


def decode_layers(layers=None, n=None, outs="default", ws=FAKE, nws=1 << 30, b=None, idx=FAKE):
    layers = [_attn(), _attn()] if layers is None else layers
    n = len(layers) if n is None else n
    arr = (Q._Attn * max(len(layers), 1))(*layers)
    if outs == "default":
        outs = [FAKE] * max(len(layers), 1)
    optrs = None if outs is None else (ctypes.c_void_p * len(outs))(*outs)
    b = b or _batch()
    return Q.lib().qsa_sparse_attn_decode_layers(arr, n, P(idx), 2048, 4, ctypes.byref(b), optrs, P(ws), nws,
                                                 None, None)


def ingest_score(b=None, ix=None, scores=FAKE, ld=1024, kdt=Q.QSA_BF16):
    b = b or _batch()
    ix = ix or _ix()
    ring = _ring()
    return Q.lib().qsa_ingest_index_score(P(FAKE), kdt, 4, ctypes.byref(b), ctypes.byref(ring), None, None,
                                          ctypes.byref(ix), P(scores), ld, None, None)


def score_topk(b=None, ix=None, scores=FAKE, ld=1024, idx=FAKE, ws=FAKE, nws=1 << 30):
    b = b or _batch()
    ix = ix or _ix()
    return Q.lib().qsa_index_score_topk(ctypes.byref(ix), 2048, 4, ctypes.byref(b), P(scores), ld, P(idx), P(ws),
                                        nws, None, None)


def decode_step(b=None, ix=None, a=None, scores=FAKE, ld=1024, idx=FAKE, out=FAKE, ws=FAKE, nws=1 << 30):
    b = b or _batch()
    ix = ix or _ix()
    a = a or _attn()
    return Q.lib().qsa_decode_step(ctypes.byref(ix), ctypes.byref(a), 2048, 4, ctypes.byref(b), P(scores), ld,
                                   P(idx), P(out), P(ws), nws, None, None)


def attend_lists(b=None, a=None, scores=FAKE, ld=1024, idx=FAKE, out=FAKE, ws=FAKE, nws=1 << 30):
    b = b or _batch()
    a = a or _attn()
    return Q.lib().qsa_sparse_attn_decode_lists(ctypes.byref(a), 2048, 4, ctypes.byref(b), P(scores), ld, P(idx),
                                                P(out), P(ws), nws, None, None)


def ingest_lists(b=None, ix=None, a=None, scores=FAKE, ld=1024, ws=FAKE, nws=1 << 30):
    b = b or _batch()
    ix = ix or _ix()
    a = a or _attn()
    ring = _ring()
    return Q.lib().qsa_ingest_index_score_lists(P(FAKE), Q.QSA_BF16, ctypes.byref(ring), None, None,
                                                ctypes.byref(ix), ctypes.byref(a), 2048, 4, ctypes.byref(b),
                                                P(scores), ld, P(ws), nws, None, None)


INV, UNS, WS = Q.QSA_ERR_INVALID_ARGUMENT, Q.QSA_ERR_UNSUPPORTED, Q.QSA_ERR_WORKSPACE

CASES = [
    # (name, thunk, expected status, fragment of the message)
    ("compress null k_idx", lambda: compress(k=None), INV, "k_idx"),
    ("compress ratio 3", lambda: compress(ratio=3), UNS, "ratio=3"),
    ("compress ratio 128", lambda: compress(ratio=128), UNS, "ratio=128"),
    ("compress d_idx 96", lambda: compress(d=96), UNS, "d_idx=96"),
    ("compress e4m3 without scale", lambda: compress(kcdt=Q.QSA_FP8_E4M3), INV, "kc_scale"),
    ("compress num_seqs 0", lambda: compress(b=_batch(num_seqs=0)), INV, "num_seqs"),
    ("compress missing blk_offsets", lambda: compress(b=_batch(blk_offsets=None)), INV, "blk_offsets"),
    ("score bad flags", lambda: score(flags=7), INV, "flags"),
    ("score h_idx 3", lambda: score(ix=_ix(h_idx=3)), UNS, "h_idx=3"),
    ("score d_idx 32", lambda: score(ix=_ix(d_idx=32)), UNS, "d_idx=32"),
    ("score scale without e4m3", lambda: score(ix=_ix(kc_scale=FAKE)), INV, "kc_scale"),
    ("score q fp8", lambda: score(ix=_ix(q_dtype=Q.QSA_FP8_E4M3)), UNS, "q_dtype"),
    ("score ld too small", lambda: score(ld=1023), INV, "ld_scores"),
    ("score mfma f32", lambda: score(ix=_ix(q_dtype=Q.QSA_F32), flags=1), UNS, "MFMA"),
    ("score total_q mismatch", lambda: score(b=_batch(total_q=3)), INV, "total_q"),
    ("score too many blocks", lambda: score(b=_batch(max_kv_len=4 * 131073), ld=131073), UNS, "131072"),
    ("topk budget not multiple", lambda: topk(budget=2047), UNS, "budget=2047"),
    ("topk K too large", lambda: topk(budget=4 * 4096), UNS, "budget/ratio=4096"),
    ("topk null idx", lambda: topk(idx=None), INV, "idx"),
    ("topk null scores", lambda: topk(scores=None), INV, "scores"),
    ("topk recheck row too long", lambda: topk(recheck=_ix(), b=_batch(max_kv_len=4 * 40000), ld=40000),
     UNS, "re-checked"),
    ("topk recheck workspace missing", lambda: topk(recheck=_ix()), WS, "workspace"),
    ("decode hq not multiple", lambda: decode(a=_attn(hq=30)), INV, "attn.hq=30"),
    ("decode group 32", lambda: decode(a=_attn(hq=64, hkv=2)), UNS, "hq/attn.hkv=32"),
    ("decode d 64", lambda: decode(a=_attn(d=64)), UNS, "attn.d=64"),
    ("decode fp8", lambda: decode(a=_attn(dtype=Q.QSA_FP8_E4M3)), UNS, "attn.dtype"),
    ("decode bad scale", lambda: decode(a=_attn(softmax_scale=0.0)), INV, "softmax_scale"),
    ("decode null out", lambda: decode(out=None), INV, "out"),
    ("decode workspace missing", lambda: decode(ws=None, nws=0), WS, "workspace"),
    ("decode workspace small", lambda: decode(nws=16), WS, "workspace"),
    ("decode multi-query batch", lambda: decode(b=_batch(q_offsets=FAKE, max_q_per_seq=4, total_q=8)),
     INV, "prefill"),
    ("prefill null idx", lambda: prefill(idx=None), INV, "idx"),
    ("paged score null descriptor", lambda: score_paged(pg=None), INV, "paging descriptor"),
    ("paged score null table", lambda: score_paged(pg=_pg(block_table=None)), INV, "block_table"),
    ("paged score page 48", lambda: score_paged(pg=_pg(page_size=48)), INV, "page_size=48"),
    ("paged score page below ratio", lambda: score_paged(pg=_pg(page_size=2)), INV, "page_size=2"),
    ("paged score too few pages", lambda: score_paged(pg=_pg(max_pages=63)), INV, "max_pages=63"),
    ("paged score mfma", lambda: score_paged(flags=1), UNS, "paged"),
    ("paged pool too large", lambda: score_paged(pg=_pg(num_pages=1 << 26)), UNS, "2^31"),
    ("paged decode no pages", lambda: decode_paged(pg=_pg(num_pages=0)), INV, "num_pages=0"),
    ("paged decode null descriptor", lambda: decode_paged(pg=None), INV, "paging descriptor"),
    ("paged compress null table", lambda: compress_paged(pg=_pg(block_table=None)),
     INV, "block_table"),
    ("ingest null ring", lambda: ingest(ring=None), INV, "ring is NULL"),
    ("ingest null ring keys", lambda: ingest(ring=_ring(keys=None)), INV, "ring.keys"),
    ("ingest null window", lambda: ingest(ring=_ring(window=None)), INV, "ring.window"),
    ("ingest capacity below ratio", lambda: ingest(ring=_ring(capacity=2)), INV, "ring.capacity=2"),
    ("ingest capacity not whole blocks", lambda: ingest(ring=_ring(capacity=10)), INV, "ring.capacity=10"),
    ("ingest too few slots", lambda: ingest(ring=_ring(num_slots=1)), INV, "ring.num_slots=1"),
    ("ingest null k_new", lambda: ingest(k_new=None), INV, "k_new"),
    ("ingest e4m3 without scale", lambda: ingest(kcdt=Q.QSA_FP8_E4M3), INV, "kc_scale"),
    ("ingest ratio 3", lambda: ingest(ratio=3), UNS, "ratio=3"),
    ("ingest d_idx 32", lambda: ingest(d=32), UNS, "d_idx=32"),
    ("ingest kv null", lambda: ingest(kv=_kv(v=None)), INV, "kv.k_new/v_new/k/v"),
    ("ingest kv d 64", lambda: ingest(kv=_kv(d=64)), UNS, "kv.d=64"),
    ("ingest kv fp8", lambda: ingest(kv=_kv(dtype=Q.QSA_FP8_E4M3)), UNS, "kv.dtype"),
    ("ingest contiguous needs blk_offsets", lambda: ingest(b=_batch(blk_offsets=None)), INV, "blk_offsets"),
    ("ingest paged page 48", lambda: ingest(pg=_pg(page_size=48), b=_batch(blk_offsets=None)), INV,
     "page_size=48"),
    ("score fp4 with f32 query", lambda: score(ix=_ix(q_dtype=Q.QSA_F32, kc_dtype=Q.QSA_FP4_E2M1,
                                                       kc_scale=FAKE)), UNS, "bf16 q_idx"),
    ("score fp4 without scales", lambda: score(ix=_ix(kc_dtype=Q.QSA_FP4_E2M1)), INV, "needs scales"),
    ("compress fp4 without scales", lambda: compress(kcdt=Q.QSA_FP4_E2M1), INV, "needs scales"),
    ("topk recheck fp4", lambda: topk(recheck=_ix(kc_dtype=Q.QSA_FP4_E2M1, kc_scale=FAKE)), UNS, "fp4"),
    ("topk local negative", lambda: topk_local(-1), UNS, "local_blocks=-1"),
    ("topk local too wide", lambda: topk_local(1537), UNS, "local_blocks=1537"),
    ("pool bad mode", lambda: Q.lib().qsa_pool_scores(P(FAKE), 4096, 4, 2, ctypes.byref(_batch()), P(FAKE),
                                                     1024, None), INV, "mode=2"),
    ("pool ld_tok small", lambda: Q.lib().qsa_pool_scores(P(FAKE), 4095, 4, 0, ctypes.byref(_batch()), P(FAKE),
                                                          1024, None), INV, "ld_tok=4095"),
    ("layers zero", lambda: decode_layers(n=0), INV, "n_layers=0"),
    ("layers nine", lambda: decode_layers(layers=[_attn()] * 9), INV, "n_layers=9"),
    ("layers null outs", lambda: decode_layers(outs=None), INV, "outs is NULL"),
    ("layers null out entry", lambda: decode_layers(outs=[FAKE, 0]), INV, "outs[1]"),
    ("layers shape mismatch", lambda: decode_layers(layers=[_attn(), _attn(hkv=8)]), INV, "layers[1]"),
    ("layers bad layer", lambda: decode_layers(layers=[_attn(), _attn(d=64)]), UNS, "attn.d=64"),
    ("layers workspace small", lambda: decode_layers(nws=16), WS, "qsa_attn_layers_workspace_size"),
    ("layers multi-query batch",
     lambda: decode_layers(b=_batch(q_offsets=FAKE, max_q_per_seq=4, total_q=8)), INV, "one query"),
    ("ingest+score multi-query batch", lambda: ingest_score(b=_batch(q_offsets=FAKE, max_q_per_seq=4, total_q=8)),
     INV, "q_offsets must be NULL"),
    ("ingest+score f32 keys", lambda: ingest_score(ix=_ix(kc_dtype=Q.QSA_F32)), UNS, "bf16, e4m3 or fp4"),
    ("ingest+score f32 query", lambda: ingest_score(ix=_ix(q_dtype=Q.QSA_F32)), UNS, "bf16 q_idx"),
    ("ingest+score null scores", lambda: ingest_score(scores=None), INV, "scores is NULL"),
    ("ingest+score ld small", lambda: ingest_score(ld=1023), INV, "ld_scores=1023"),
    ("ingest+score raw key fp8", lambda: ingest_score(kdt=Q.QSA_FP8_E4M3), UNS, "k_dtype"),
    ("score+select null idx", lambda: score_topk(idx=None), INV, "idx is NULL"),
    ("score+select workspace small", lambda: score_topk(nws=16), WS, "qsa_score_topk_workspace_size"),
    ("decode step null scores", lambda: decode_step(scores=None), INV, "scores is NULL"),
    ("decode step ld small", lambda: decode_step(ld=1023), INV, "ld_scores=1023"),
    ("decode step workspace small", lambda: decode_step(nws=16), WS, "qsa_decode_step_workspace_size"),
    ("decode step workspace misaligned", lambda: decode_step(ws=FAKE + 4), INV, "16-byte aligned"),
    ("decode step multi-query batch",
     lambda: decode_step(b=_batch(q_offsets=FAKE, max_q_per_seq=4, total_q=8)), INV, "one query"),
    ("attend lists workspace small", lambda: attend_lists(nws=16), WS, "qsa_decode_step_workspace_size"),
    ("ingest step multi-query batch",
     lambda: ingest_lists(b=_batch(q_offsets=FAKE, max_q_per_seq=4, total_q=8)), INV, "q_offsets must be NULL"),
    ("ingest step f32 keys", lambda: ingest_lists(ix=_ix(kc_dtype=Q.QSA_F32)), UNS, "bf16, e4m3 or fp4"),
    ("ingest step workspace small", lambda: ingest_lists(nws=16), WS, "qsa_decode_step_workspace_size"),
    ("ingest step workspace misaligned", lambda: ingest_lists(ws=FAKE + 4), INV, "16-byte aligned"),
    ("rewind null ring", lambda: rewind(ring=None), INV, "ring is NULL"),
    ("rewind ratio 0", lambda: rewind(ratio=0), UNS, "ratio=0"),
]


@pytest.mark.parametrize("name,thunk,status,frag", CASES, ids=[c[0] for c in CASES])
def test_validation_rejects_before_launch(name, thunk, status, frag):
    assert thunk() == status
    assert frag in _err(), _err()


def test_workspace_sizes():
    b = _batch(total_q=32, num_seqs=32)
    a = _attn()
    n = Q.lib().qsa_attn_workspace_size(ctypes.byref(b), ctypes.byref(a), 2048, 4)
    # decode cuts K=512 into 16 parts: 16 partials of (m, l) + 128 outputs
    # per query head
    assert n >= 32 * 32 * 16 * 130 * 4
    # canonical scores: a few-row batch keeps per-row lists (header, K "in"
    # indices, candidate keys and indices); large batches need none
    n = Q.lib().qsa_topk_workspace_size(ctypes.byref(b), 2048, 4, None)
    assert n >= 32 * (512 * 4 + 2 * 1024 * 4)
    big = _batch(total_q=4096, num_seqs=4096)
    assert Q.lib().qsa_topk_workspace_size(ctypes.byref(big), 2048, 4, None) == 0
    # re-checked top-k: one fp32 key-norm maximum per 256 blocks per sequence
    ix = _ix()
    n = Q.lib().qsa_topk_workspace_size(ctypes.byref(b), 2048, 4, ctypes.byref(ix))
    assert n >= 32 * (1024 // 256) * 4
    assert Q.lib().qsa_attn_workspace_size(ctypes.byref(b), ctypes.byref(a), 2047, 4) == 0
    # layered decode: one 256-byte aligned single-layer slice per layer
    one = Q.lib().qsa_attn_workspace_size(ctypes.byref(b), ctypes.byref(a), 2048, 4)
    n4 = Q.lib().qsa_attn_layers_workspace_size(ctypes.byref(b), ctypes.byref(a), 4, 2048, 4)
    assert n4 == 4 * ((one + 255) // 256 * 256)
    assert Q.lib().qsa_attn_layers_workspace_size(ctypes.byref(b), ctypes.byref(a), 9, 2048, 4) == 0


# ------------------------------------------------ forced launch failure hook
HOOK = "QSA_TEST_FORCE_LAUNCH_ERROR"
VALID_CALLS = [
    ("compress", lambda: compress()),
    ("compress paged", lambda: compress_paged()),
    ("score", lambda: score()),
    ("score paged", lambda: score_paged()),
    ("topk", lambda: topk(b=_batch(total_q=4096, num_seqs=4096))),
    ("topk local", lambda: Q.lib().qsa_topk_blocks_local(P(FAKE), 1024, None, 2048, 4, 8,
                                                         ctypes.byref(_batch(total_q=4096, num_seqs=4096)),
                                                         P(FAKE), None, 0, None)),
    ("decode", lambda: decode()),
    ("decode paged", lambda: decode_paged()),
    ("prefill", lambda: prefill()),
    ("decode layers", lambda: decode_layers()),
    ("ingest", lambda: ingest()),
    ("ingest + score", lambda: ingest_score()),
    ("rewind", lambda: rewind()),
    ("pool", lambda: Q.lib().qsa_pool_scores(P(FAKE), 4096, 4, 0, ctypes.byref(_batch()), P(FAKE), 1024, None)),
]


@pytest.mark.parametrize("name,thunk", VALID_CALLS, ids=[c[0] for c in VALID_CALLS])
def test_forced_launch_failure_returns_hip_error(monkeypatch, name, thunk):
    # host validation passes, then the hook fails the launch without touching
    # a device (the pointers are fake)
    monkeypatch.setenv(HOOK, "1")
    assert thunk() == Q.QSA_ERR_HIP
    assert HOOK in _err() and "launch failed" in _err()


def test_forced_launch_failure_does_not_hide_validation(monkeypatch):
    monkeypatch.setenv(HOOK, "1")
    assert compress(ratio=3) == UNS and "ratio=3" in _err()
    assert decode(nws=16) == WS
    monkeypatch.setenv(HOOK, "0")
    assert compress(ratio=5) == UNS


def test_binding_raises_qsa_error_with_the_status(monkeypatch):
    import torch
    monkeypatch.setenv(HOOK, "1")
    with pytest.raises(Q.QsaError) as e:
        Q._check(score())
    assert e.value.status == Q.QSA_ERR_HIP and HOOK in e.value.message
    assert Q.QSA_ERR_DEVICE_ASSERT == 5
    del torch


def test_static_decode_rejects_batches_past_its_array(monkeypatch):
    a = _attn()
    b = _batch(total_q=4096, num_seqs=4096)
    st = Q.lib().qsa_sparse_attn_decode_static(ctypes.byref(a), P(FAKE), 2048, 4, ctypes.byref(b), P(FAKE), None)
    assert st == Q.QSA_ERR_WORKSPACE and "static array" in _err()
    assert Q.lib().qsa_sparse_attn_decode_static(ctypes.byref(_attn(hq=30)), P(FAKE), 2048, 4,
                                                 ctypes.byref(_batch()), P(FAKE), None) == INV
    assert Q.lib().qsa_sparse_attn_decode_static(ctypes.byref(a), P(FAKE), 2048, 4, ctypes.byref(_batch()), None,
                                                 None) == INV
    monkeypatch.setenv(HOOK, "1")
    assert Q.lib().qsa_sparse_attn_decode_static(ctypes.byref(a), P(FAKE), 2048, 4, ctypes.byref(_batch()),
                                                 P(FAKE), None) == Q.QSA_ERR_HIP
