"""Python binding of libqsa (indexer-selected sparse attention on MI355X).

Argument marshalling only: every step of the method runs in the HIP kernels of
`libqsa.so` behind the C ABI declared in `include/qsa.h`.  PyTorch provides
device memory and streams.  There is no CPU fallback: if the library is not
built or fails to load, every call raises.

Entry points mirror the C names:
    inert_bound, version,
    compress_keys, index_score, topk_workspace_size, topk_blocks,
    attn_workspace_size, sparse_attn_decode, sparse_attn_prefill.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_OK, QSA_ERR_INVALID_ARGUMENT, QSA_ERR_UNSUPPORTED, QSA_ERR_WORKSPACE, QSA_ERR_HIP, QSA_ERR_DEVICE_ASSERT = range(6)
ABI_VERSION = 3   # QSA_ABI_VERSION of include/qsa.h
QSA_F32, QSA_BF16, QSA_FP8_E4M3, QSA_FP4_E2M1 = 0, 1, 2, 3
QSA_SCORE_CANONICAL, QSA_SCORE_MFMA = 0, 1
QSA_POOL_MAX, QSA_POOL_MEAN = 0, 1

EXPORTS = (
    "qsa_inert_bound", "qsa_last_error", "qsa_version", "qsa_abi_version",
    "qsa_compress_keys", "qsa_index_score", "qsa_topk_workspace_size", "qsa_topk_blocks",
    "qsa_attn_workspace_size", "qsa_sparse_attn_decode", "qsa_sparse_attn_prefill",
    "qsa_compress_keys_paged", "qsa_index_score_paged", "qsa_sparse_attn_decode_paged",
    "qsa_sparse_attn_prefill_paged", "qsa_ingest", "qsa_ring_rewind", "qsa_topk_blocks_local",
    "qsa_pool_scores", "qsa_attn_layers_workspace_size", "qsa_sparse_attn_decode_layers",
    "qsa_ingest_index_score", "qsa_sparse_attn_decode_static", "qsa_score_topk_workspace_size",
    "qsa_index_score_topk", "qsa_decode_step_workspace_size", "qsa_decode_step", "qsa_index_score_lists",
    "qsa_sparse_attn_decode_lists", "qsa_ingest_index_score_lists",
)

MAX_LAYERS = 8   # QSA_MAX_LAYERS

# per-sequence codes written by qsa_ingest / qsa_ring_rewind
INGEST_OK, INGEST_LOST_KEYS, INGEST_BAD_SLOT, INGEST_TOO_LONG, REWIND_DECLINED = range(5)


class QsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"qsa status {status}: {message}")
        self.status = status
        self.message = message


class _Batch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("max_q_per_seq", ctypes.c_int32),
                ("total_q", ctypes.c_int64), ("max_kv_len", ctypes.c_int64),
                ("kv_offsets", ctypes.c_void_p), ("blk_offsets", ctypes.c_void_p),
                ("q_offsets", ctypes.c_void_p)]


class _Indexer(ctypes.Structure):
    _fields_ = [("q_idx", ctypes.c_void_p), ("w", ctypes.c_void_p), ("kc", ctypes.c_void_p),
                ("kc_scale", ctypes.c_void_p), ("q_dtype", ctypes.c_int32),
                ("kc_dtype", ctypes.c_int32), ("h_idx", ctypes.c_int32), ("d_idx", ctypes.c_int32)]


class _Attn(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("dtype", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class _PagedKV(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int64),
                ("num_pages", ctypes.c_int64), ("page_size", ctypes.c_int32)]


class _KeyRing(ctypes.Structure):
    _fields_ = [("keys", ctypes.c_void_p), ("window", ctypes.c_void_p), ("slots", ctypes.c_void_p),
                ("num_slots", ctypes.c_int64), ("capacity", ctypes.c_int32)]


class _KvAppend(ctypes.Structure):
    _fields_ = [("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32)]


_lib = None


def lib():
    """Load libqsa.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libqsa.so is not built ({LIB_PATH}); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.qsa_inert_bound.restype = i32
        L.qsa_inert_bound.argtypes = [i32, i32]
        L.qsa_last_error.restype = ctypes.c_char_p
        L.qsa_version.restype = ctypes.c_char_p
        L.qsa_abi_version.restype = i32
        L.qsa_compress_keys.restype = i32
        L.qsa_compress_keys.argtypes = [P, i32, i32, i32, P, P, P, i32, P, P]
        L.qsa_index_score.restype = i32
        L.qsa_index_score.argtypes = [P, i32, P, P, i64, ctypes.c_uint32, P]
        L.qsa_topk_workspace_size.restype = sz
        L.qsa_topk_workspace_size.argtypes = [P, i32, i32, P]
        L.qsa_topk_blocks.restype = i32
        L.qsa_topk_blocks.argtypes = [P, i64, P, i32, i32, P, P, P, sz, P]
        L.qsa_attn_workspace_size.restype = sz
        L.qsa_attn_workspace_size.argtypes = [P, P, i32, i32]
        for f in (L.qsa_sparse_attn_decode, L.qsa_sparse_attn_prefill):
            f.restype = i32
            f.argtypes = [P, P, i32, i32, P, P, P, sz, P]
        L.qsa_compress_keys_paged.restype = i32
        L.qsa_compress_keys_paged.argtypes = [P, i32, i32, i32, P, P, P, i32, P, P, P]
        L.qsa_index_score_paged.restype = i32
        L.qsa_index_score_paged.argtypes = [P, i32, P, P, i64, ctypes.c_uint32, P, P]
        for f in (L.qsa_sparse_attn_decode_paged, L.qsa_sparse_attn_prefill_paged):
            f.restype = i32
            f.argtypes = [P, P, i32, i32, P, P, P, sz, P, P]
        L.qsa_topk_blocks_local.restype = i32
        L.qsa_topk_blocks_local.argtypes = [P, i64, P, i32, i32, i32, P, P, P, sz, P]
        L.qsa_pool_scores.restype = i32
        L.qsa_pool_scores.argtypes = [P, i64, i32, i32, P, P, i64, P]
        L.qsa_attn_layers_workspace_size.restype = sz
        L.qsa_attn_layers_workspace_size.argtypes = [P, P, i32, i32, i32]
        L.qsa_sparse_attn_decode_layers.restype = i32
        L.qsa_sparse_attn_decode_layers.argtypes = [P, i32, P, i32, i32, P, P, P, sz, P, P]
        L.qsa_ingest.restype = i32
        L.qsa_ingest.argtypes = [P, i32, i32, i32, P, P, P, i32, P, P, P, P, P]
        L.qsa_ingest_index_score.restype = i32
        L.qsa_ingest_index_score.argtypes = [P, i32, i32, P, P, P, P, P, P, i64, P, P]
        L.qsa_score_topk_workspace_size.restype = sz
        L.qsa_score_topk_workspace_size.argtypes = [P, i32, i32]
        L.qsa_index_score_topk.restype = i32
        L.qsa_index_score_topk.argtypes = [P, i32, i32, P, P, i64, P, P, sz, P, P]
        L.qsa_decode_step_workspace_size.restype = sz
        L.qsa_decode_step_workspace_size.argtypes = [P, P, i32, i32]
        L.qsa_decode_step.restype = i32
        L.qsa_decode_step.argtypes = [P, P, i32, i32, P, P, i64, P, P, P, sz, P, P]
        L.qsa_index_score_lists.restype = i32
        L.qsa_index_score_lists.argtypes = [P, P, i32, i32, P, P, i64, P, sz, P, P]
        L.qsa_sparse_attn_decode_lists.restype = i32
        L.qsa_sparse_attn_decode_lists.argtypes = [P, i32, i32, P, P, i64, P, P, P, sz, P, P]
        L.qsa_ingest_index_score_lists.restype = i32
        L.qsa_ingest_index_score_lists.argtypes = [P, i32, P, P, P, P, P, i32, i32, P, P, i64, P, sz, P, P]
        L.qsa_sparse_attn_decode_static.restype = i32
        L.qsa_sparse_attn_decode_static.argtypes = [P, P, i32, i32, P, P, P]
        L.qsa_ring_rewind.restype = i32
        L.qsa_ring_rewind.argtypes = [P, i32, P, P, P]
        _lib = L
    return _lib


def _check(status: int):
    if status != QSA_OK:
        raise QsaError(status, lib().qsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return QSA_F32
    if t.dtype == torch.bfloat16:
        return QSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return QSA_FP8_E4M3
    if t.dtype == torch.float4_e2m1fn_x2:
        return QSA_FP4_E2M1
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------------ batch
@dataclass
class Batch:
    """A varlen batch: device int64 offsets plus host bounds (C qsa_batch)."""
    kv_offsets: torch.Tensor            # device int64 [B+1]
    blk_offsets: torch.Tensor           # device int64 [B+1]
    q_offsets: Optional[torch.Tensor]   # device int64 [B+1] or None (decode)
    total_q: int
    max_kv_len: int
    max_q_per_seq: int

    @property
    def num_seqs(self) -> int:
        return self.kv_offsets.numel() - 1

    @staticmethod
    def from_lengths(kv_lens, q_lens=None, ratio: int = 4, device="cuda") -> "Batch":
        kv_lens = [int(x) for x in kv_lens]
        kv = [0]
        bl = [0]
        for n in kv_lens:
            kv.append(kv[-1] + n)
            bl.append(bl[-1] + n // ratio)
        qo = None
        total_q, max_q = len(kv_lens), 1
        if q_lens is not None:
            q_lens = [int(x) for x in q_lens]
            acc = [0]
            for n in q_lens:
                acc.append(acc[-1] + n)
            qo = torch.tensor(acc, dtype=torch.int64, device=device)
            total_q, max_q = acc[-1], max(q_lens) if q_lens else 1
        return Batch(torch.tensor(kv, dtype=torch.int64, device=device),
                     torch.tensor(bl, dtype=torch.int64, device=device), qo, total_q,
                     max(kv_lens) if kv_lens else 0, max(max_q, 1))

    def _c(self) -> _Batch:
        return _Batch(self.num_seqs, self.max_q_per_seq, self.total_q, self.max_kv_len,
                      self.kv_offsets.data_ptr(), self.blk_offsets.data_ptr(),
                      None if self.q_offsets is None else self.q_offsets.data_ptr())


@dataclass
class Paging:
    """Paged caches (C qsa_paged_kv): page j of sequence s is physical page
    block_table[s, j]; every pool holds num_pages pages (page_size token rows
    of K, V, k_idx; page_size/ratio rows of kc, kc_scale)."""
    block_table: torch.Tensor           # device int32 [num_seqs, max_pages]
    num_pages: int
    page_size: int

    def _c(self) -> _PagedKV:
        _dev(self.block_table, "block_table")
        if self.block_table.dtype != torch.int32 or self.block_table.dim() != 2:
            raise TypeError("block_table must be a 2-D int32 tensor")
        return _PagedKV(self.block_table.data_ptr(), self.block_table.shape[1], int(self.num_pages),
                        int(self.page_size))


@dataclass
class KeyRing:
    """Raw indexer keys of the last `capacity` positions per ring slot (C
    qsa_key_ring).  keys [num_slots, capacity, d_idx] (dtype of the raw keys);
    window int64 [num_slots, 2] = {lo, hi} (a fresh slot is {0, 0}); slots:
    int32 [num_seqs] slot of each sequence, or None for slot s."""
    keys: torch.Tensor
    window: torch.Tensor
    slots: Optional[torch.Tensor] = None

    @staticmethod
    def empty(num_slots: int, capacity: int, d_idx: int, dtype=torch.bfloat16, device="cuda"):
        return KeyRing(torch.zeros((num_slots, capacity, d_idx), dtype=dtype, device=device),
                       torch.zeros((num_slots, 2), dtype=torch.int64, device=device))

    def _c(self) -> _KeyRing:
        _dev(self.keys, "ring.keys")
        _dev(self.window, "ring.window")
        if self.window.dtype != torch.int64 or tuple(self.window.shape) != (self.keys.shape[0], 2):
            raise TypeError("ring.window must be int64 [num_slots, 2]")
        if self.slots is not None:
            _dev(self.slots, "ring.slots")
            if self.slots.dtype != torch.int32:
                raise TypeError("ring.slots must be int32")
        return _KeyRing(self.keys.data_ptr(), self.window.data_ptr(), _ptr(self.slots),
                        self.keys.shape[0], self.keys.shape[1])


# -------------------------------------------------------------- functions
def inert_bound(budget: int, ratio: int) -> int:
    return int(lib().qsa_inert_bound(budget, ratio))


def version() -> str:
    return lib().qsa_version().decode()


def compress_keys(k_idx: torch.Tensor, ratio: int, batch: Batch, kc: torch.Tensor,
                  kc_scale: Optional[torch.Tensor] = None, first_block: Optional[torch.Tensor] = None,
                  stream=None, paging: Optional[Paging] = None) -> None:
    """qsa_compress_keys (qsa_compress_keys_paged with `paging`): writes kc (f32,
    bf16, or uint8 e4m3 codes) [+ kc_scale]."""
    _dev(k_idx, "k_idx")
    _dev(kc, "kc")
    kcd = QSA_FP8_E4M3 if kc.dtype == torch.uint8 else _dtype_code(kc)
    b = batch._c()
    if paging is None:
        _check(lib().qsa_compress_keys(_ptr(k_idx), _dtype_code(k_idx), k_idx.shape[-1], ratio,
                                       ctypes.byref(b), _ptr(first_block), _ptr(kc), kcd,
                                       _ptr(kc_scale), _stream(stream)))
    else:
        pg = paging._c()
        _check(lib().qsa_compress_keys_paged(_ptr(k_idx), _dtype_code(k_idx), k_idx.shape[-1], ratio,
                                             ctypes.byref(b), _ptr(first_block), _ptr(kc), kcd,
                                             _ptr(kc_scale), ctypes.byref(pg), _stream(stream)))


def _indexer(q_idx, w, kc, kc_scale) -> _Indexer:
    for t, n in ((q_idx, "q_idx"), (w, "w"), (kc, "kc")):
        _dev(t, n)
    if w.dtype != torch.float32:
        raise TypeError("w must be float32")
    kcd = QSA_FP8_E4M3 if kc.dtype == torch.uint8 else _dtype_code(kc)
    return _Indexer(q_idx.data_ptr(), w.data_ptr(), kc.data_ptr(),
                    None if kc_scale is None else kc_scale.data_ptr(), _dtype_code(q_idx), kcd,
                    q_idx.shape[1], q_idx.shape[2])


def index_score(q_idx, w, kc, kc_scale, ratio: int, batch: Batch, scores: torch.Tensor,
                mode: int = QSA_SCORE_CANONICAL, stream=None, paging: Optional[Paging] = None) -> None:
    """qsa_index_score (qsa_index_score_paged with `paging`) into scores [total_q, ld]."""
    _dev(scores, "scores")
    ix = _indexer(q_idx, w, kc, kc_scale)
    b = batch._c()
    if paging is None:
        _check(lib().qsa_index_score(ctypes.byref(ix), ratio, ctypes.byref(b), _ptr(scores),
                                     scores.shape[1], mode, _stream(stream)))
    else:
        pg = paging._c()
        _check(lib().qsa_index_score_paged(ctypes.byref(ix), ratio, ctypes.byref(b), _ptr(scores),
                                           scores.shape[1], mode, ctypes.byref(pg), _stream(stream)))


def score_topk_workspace_size(batch: Batch, budget: int, ratio: int) -> int:
    b = batch._c()
    return int(lib().qsa_score_topk_workspace_size(ctypes.byref(b), budget, ratio))


def index_score_topk(q_idx, w, kc, kc_scale, budget: int, ratio: int, batch: Batch, scores: torch.Tensor,
                     idx: torch.Tensor, ws: Optional[torch.Tensor], stream=None,
                     paging: Optional[Paging] = None) -> None:
    """qsa_index_score_topk: canonical scores and their block top-k in one call."""
    _dev(scores, "scores")
    _dev(idx, "idx")
    ix = _indexer(q_idx, w, kc, kc_scale)
    b = batch._c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    pg = None if paging is None else ctypes.byref(paging._c())
    _check(lib().qsa_index_score_topk(ctypes.byref(ix), budget, ratio, ctypes.byref(b), _ptr(scores),
                                      scores.shape[1], _ptr(idx), _ptr(ws), nbytes, pg, _stream(stream)))


def decode_step_workspace_size(q, k, v, softmax_scale, budget: int, ratio: int, batch: Batch) -> int:
    a = _attn(q, k, v, softmax_scale)
    b = batch._c()
    return int(lib().qsa_decode_step_workspace_size(ctypes.byref(b), ctypes.byref(a), budget, ratio))


def decode_step(q_idx, w, kc, kc_scale, q, k, v, softmax_scale, budget: int, ratio: int, batch: Batch,
                scores: torch.Tensor, idx: torch.Tensor, out: torch.Tensor, ws: Optional[torch.Tensor],
                stream=None, paging: Optional[Paging] = None) -> None:
    """qsa_decode_step: scores, selection and sparse attention of a decode batch."""
    for t, n in ((scores, "scores"), (idx, "idx"), (out, "out")):
        _dev(t, n)
    ix = _indexer(q_idx, w, kc, kc_scale)
    a = _attn(q, k, v, softmax_scale)
    b = batch._c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    pg = None if paging is None else ctypes.byref(paging._c())
    _check(lib().qsa_decode_step(ctypes.byref(ix), ctypes.byref(a), budget, ratio, ctypes.byref(b), _ptr(scores),
                                 scores.shape[1], _ptr(idx), _ptr(out), _ptr(ws), nbytes, pg, _stream(stream)))


def index_score_lists(q_idx, w, kc, kc_scale, q, k, v, softmax_scale, budget: int, ratio: int, batch: Batch,
                      scores: torch.Tensor, ws: Optional[torch.Tensor], stream=None,
                      paging: Optional[Paging] = None) -> None:
    """qsa_index_score_lists: the scorer half of qsa_decode_step."""
    _dev(scores, "scores")
    ix = _indexer(q_idx, w, kc, kc_scale)
    a = _attn(q, k, v, softmax_scale)
    b = batch._c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    pg = None if paging is None else ctypes.byref(paging._c())
    _check(lib().qsa_index_score_lists(ctypes.byref(ix), ctypes.byref(a), budget, ratio, ctypes.byref(b),
                                       _ptr(scores), scores.shape[1], _ptr(ws), nbytes, pg, _stream(stream)))


def sparse_attn_decode_lists(q, k, v, softmax_scale, budget: int, ratio: int, batch: Batch, scores: torch.Tensor,
                             idx: torch.Tensor, out: torch.Tensor, ws: Optional[torch.Tensor], stream=None,
                             paging: Optional[Paging] = None) -> None:
    """qsa_sparse_attn_decode_lists: the selection + attention half of qsa_decode_step."""
    for t, n in ((scores, "scores"), (idx, "idx"), (out, "out")):
        _dev(t, n)
    a = _attn(q, k, v, softmax_scale)
    b = batch._c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    pg = None if paging is None else ctypes.byref(paging._c())
    _check(lib().qsa_sparse_attn_decode_lists(ctypes.byref(a), budget, ratio, ctypes.byref(b), _ptr(scores),
                                              scores.shape[1], _ptr(idx), _ptr(out), _ptr(ws), nbytes, pg,
                                              _stream(stream)))


def topk_workspace_size(batch: Batch, budget: int, ratio: int, recheck=None) -> int:
    b = batch._c()
    ix = None if recheck is None else _indexer(*recheck)
    return int(lib().qsa_topk_workspace_size(ctypes.byref(b), budget, ratio,
                                             None if ix is None else ctypes.byref(ix)))


def topk_blocks(scores, budget: int, ratio: int, batch: Batch, idx: torch.Tensor,
                recheck=None, ws: Optional[torch.Tensor] = None, stream=None,
                local_blocks: int = 0) -> None:
    """qsa_topk_blocks into idx [total_q, budget/ratio] int32.  `recheck` is the
    tuple (q_idx, w, kc, kc_scale) when scores came from QSA_SCORE_MFMA.  With
    local_blocks > 0 this is qsa_topk_blocks_local: idx [total_q, budget/ratio
    + local_blocks] also keeps the last local_blocks complete blocks."""
    _dev(scores, "scores")
    _dev(idx, "idx")
    b = batch._c()
    ix = None if recheck is None else _indexer(*recheck)
    args = (_ptr(scores), scores.shape[1], None if ix is None else ctypes.byref(ix), budget, ratio)
    tail = (ctypes.byref(b), _ptr(idx), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
            _stream(stream))
    if local_blocks:
        _check(lib().qsa_topk_blocks_local(*args, int(local_blocks), *tail))
    else:
        _check(lib().qsa_topk_blocks(*args, *tail))


def _attn(q, k, v, softmax_scale) -> _Attn:
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    return _Attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), q.shape[1], k.shape[1],
                 q.shape[2], float(softmax_scale))


def attn_workspace_size(q, k, v, softmax_scale, budget: int, ratio: int, batch: Batch) -> int:
    a = _attn(q, k, v, softmax_scale)
    b = batch._c()
    return int(lib().qsa_attn_workspace_size(ctypes.byref(b), ctypes.byref(a), budget, ratio))


def _attn_call(fn, fn_paged, q, k, v, softmax_scale, idx, budget, ratio, batch, out, ws, stream,
               paging):
    _dev(idx, "idx")
    _dev(out, "out")
    a = _attn(q, k, v, softmax_scale)
    b = batch._c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    if paging is None:
        _check(fn(ctypes.byref(a), _ptr(idx), budget, ratio, ctypes.byref(b), _ptr(out), _ptr(ws),
                  nbytes, _stream(stream)))
    else:
        pg = paging._c()
        _check(fn_paged(ctypes.byref(a), _ptr(idx), budget, ratio, ctypes.byref(b), _ptr(out),
                        _ptr(ws), nbytes, ctypes.byref(pg), _stream(stream)))


def sparse_attn_decode(q, k, v, softmax_scale, idx, budget, ratio, batch, out, ws=None,
                       stream=None, paging: Optional[Paging] = None) -> None:
    """qsa_sparse_attn_decode (qsa_sparse_attn_decode_paged with `paging`: k, v are pools)."""
    L = lib()
    _attn_call(L.qsa_sparse_attn_decode, L.qsa_sparse_attn_decode_paged, q, k, v, softmax_scale, idx,
               budget, ratio, batch, out, ws, stream, paging)


def attn_layers_workspace_size(q, k, v, softmax_scale, n_layers: int, budget: int, ratio: int,
                               batch: Batch) -> int:
    a = _attn(q, k, v, softmax_scale)
    b = batch._c()
    return int(lib().qsa_attn_layers_workspace_size(ctypes.byref(b), ctypes.byref(a), n_layers, budget, ratio))


def sparse_attn_decode_layers(layers, idx, budget, ratio, batch, outs, ws, stream=None,
                              paging: Optional[Paging] = None) -> None:
    """qsa_sparse_attn_decode_layers: layers = [(q, k, v, softmax_scale), ...]
    sharing idx; outs = one output tensor per layer; ws: device workspace of
    attn_layers_workspace_size bytes."""
    _dev(idx, "idx")
    n = len(layers)
    if len(outs) != n:
        raise ValueError("one output per layer")
    arr = (_Attn * max(n, 1))(*[_attn(*lay) for lay in layers])
    for o in outs:
        _dev(o, "out")
    optrs = (ctypes.c_void_p * max(n, 1))(*[o.data_ptr() for o in outs])
    b = batch._c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    pg = None if paging is None else ctypes.byref(paging._c())
    _check(lib().qsa_sparse_attn_decode_layers(arr, n, _ptr(idx), budget, ratio, ctypes.byref(b), optrs,
                                               _ptr(ws), nbytes, pg, _stream(stream)))


def sparse_attn_decode_static(q, k, v, softmax_scale, idx, budget, ratio, batch, out, stream=None):
    """qsa_sparse_attn_decode_static: decode attention with the split partials
    in the library's static device array (no workspace argument)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (idx, "idx"), (out, "out")):
        _dev(t, n)
    a = _attn(q, k, v, softmax_scale)
    b = batch._c()
    _check(lib().qsa_sparse_attn_decode_static(ctypes.byref(a), _ptr(idx), budget, ratio, ctypes.byref(b),
                                               _ptr(out), _stream(stream)))


def sparse_attn_prefill(q, k, v, softmax_scale, idx, budget, ratio, batch, out, ws=None,
                        stream=None, paging: Optional[Paging] = None) -> None:
    """qsa_sparse_attn_prefill (qsa_sparse_attn_prefill_paged with `paging`: k, v are pools)."""
    L = lib()
    _attn_call(L.qsa_sparse_attn_prefill, L.qsa_sparse_attn_prefill_paged, q, k, v, softmax_scale,
               idx, budget, ratio, batch, out, ws, stream, paging)


def _check_ring_keys(ring: KeyRing, k_new: torch.Tensor) -> None:
    if ring.keys.dtype != k_new.dtype or ring.keys.shape[-1] != k_new.shape[-1]:
        raise TypeError("ring.keys must have the dtype and width of k_new")


def _kv_append(kv) -> Optional[_KvAppend]:
    if kv is None:
        return None
    kn, vn, K, V = kv
    for t, n in ((kn, "kv.k_new"), (vn, "kv.v_new"), (K, "kv.k"), (V, "kv.v")):
        _dev(t, n)
    if not (kn.dtype == vn.dtype == K.dtype == V.dtype):
        raise TypeError("K/V append tensors must share one dtype")
    return _KvAppend(kn.data_ptr(), vn.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(K),
                     K.shape[-2], K.shape[-1])


def ingest(k_new: torch.Tensor, ratio: int, batch: Batch, ring: KeyRing, kc: torch.Tensor,
           kc_scale: Optional[torch.Tensor] = None, kv=None, status: Optional[torch.Tensor] = None,
           stream=None, paging: Optional[Paging] = None) -> None:
    """qsa_ingest: append the new tokens of every sequence (positions N_s - n_s ..
    N_s - 1 with N_s from batch.kv_offsets and n_s from batch.q_offsets, one per
    sequence when None): raw keys into the ring, every block they complete into
    kc [+ kc_scale], and, with kv = (k_new, v_new, K, V), the K/V rows.
    status: device int32 [num_seqs] or None (INGEST_* codes per sequence)."""
    _dev(k_new, "k_new")
    _dev(kc, "kc")
    kcd = QSA_FP8_E4M3 if kc.dtype == torch.uint8 else _dtype_code(kc)
    _check_ring_keys(ring, k_new)
    kva = _kv_append(kv)
    if status is not None:
        _dev(status, "status")
    b, rg = batch._c(), ring._c()
    pg = None if paging is None else paging._c()
    _check(lib().qsa_ingest(_ptr(k_new), _dtype_code(k_new), k_new.shape[-1], ratio, ctypes.byref(b),
                            ctypes.byref(rg), _ptr(kc), kcd, _ptr(kc_scale),
                            None if kva is None else ctypes.byref(kva), _ptr(status),
                            None if pg is None else ctypes.byref(pg), _stream(stream)))


def ingest_index_score(k_new: torch.Tensor, ratio: int, batch: Batch, ring: KeyRing, q_idx, w, kc,
                       kc_scale, scores: torch.Tensor, kv=None, status: Optional[torch.Tensor] = None,
                       stream=None, paging: Optional[Paging] = None) -> None:
    """qsa_ingest_index_score: ingest(k_new, ..., kc, kc_scale, kv, status) then
    index_score(q_idx, w, kc, kc_scale, ...) in one launch, for a decode batch
    (one new token and one query per sequence)."""
    _dev(k_new, "k_new")
    _dev(scores, "scores")
    _check_ring_keys(ring, k_new)
    ix = _indexer(q_idx, w, kc, kc_scale)
    kva = _kv_append(kv)
    if status is not None:
        _dev(status, "status")
    b, rg = batch._c(), ring._c()
    pg = None if paging is None else paging._c()
    _check(lib().qsa_ingest_index_score(_ptr(k_new), _dtype_code(k_new), ratio, ctypes.byref(b), ctypes.byref(rg),
                                        None if kva is None else ctypes.byref(kva), _ptr(status), ctypes.byref(ix),
                                        _ptr(scores), scores.shape[1], None if pg is None else ctypes.byref(pg),
                                        _stream(stream)))


def ingest_index_score_lists(k_new: torch.Tensor, ring: KeyRing, q_idx, w, kc, kc_scale, q, k, v, softmax_scale,
                             budget: int, ratio: int, batch: Batch, scores: torch.Tensor,
                             ws: Optional[torch.Tensor], kv=None, status: Optional[torch.Tensor] = None,
                             stream=None, paging: Optional[Paging] = None) -> None:
    """qsa_ingest_index_score_lists: ingest_index_score that also writes the
    candidate lists into ws; follow it with sparse_attn_decode_lists."""
    _dev(k_new, "k_new")
    _dev(scores, "scores")
    _check_ring_keys(ring, k_new)
    ix = _indexer(q_idx, w, kc, kc_scale)
    a = _attn(q, k, v, softmax_scale)
    kva = _kv_append(kv)
    if status is not None:
        _dev(status, "status")
    b, rg = batch._c(), ring._c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    pg = None if paging is None else ctypes.byref(paging._c())
    _check(lib().qsa_ingest_index_score_lists(_ptr(k_new), _dtype_code(k_new), ctypes.byref(rg),
                                              None if kva is None else ctypes.byref(kva), _ptr(status),
                                              ctypes.byref(ix), ctypes.byref(a), budget, ratio, ctypes.byref(b),
                                              _ptr(scores), scores.shape[1], _ptr(ws), nbytes, pg,
                                              _stream(stream)))


def ring_rewind(batch: Batch, ratio: int, ring: KeyRing, status: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """qsa_ring_rewind: the rollback gate to the lengths in batch.kv_offsets
    (per sequence INGEST_OK, or REWIND_DECLINED with the window unchanged)."""
    if status is not None:
        _dev(status, "status")
    b, rg = batch._c(), ring._c()
    _check(lib().qsa_ring_rewind(ctypes.byref(b), ratio, ctypes.byref(rg), _ptr(status), _stream(stream)))


def pool_scores(tok: torch.Tensor, ratio: int, mode: int, batch: Batch, blk: torch.Tensor,
                stream=None) -> None:
    """qsa_pool_scores: block scores blk [total_q, >= ceil(max_kv_len/ratio)]
    from token scores tok [total_q, >= max_kv_len] (QSA_POOL_MAX or _MEAN)."""
    _dev(tok, "tok")
    _dev(blk, "blk")
    b = batch._c()
    _check(lib().qsa_pool_scores(_ptr(tok), tok.shape[1], ratio, mode, ctypes.byref(b), _ptr(blk),
                                 blk.shape[1], _stream(stream)))
