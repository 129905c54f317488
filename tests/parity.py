"""Shared helpers for GPU-vs-oracle parity tests (imported by the test
modules; not a test file itself)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Output tolerances against the unrounded fp64 oracle:
#   bf16 output: |gpu - o| <= 1e-3 + 2e-3 |o| + half_ulp_bf16(o)
#   fp32 output: |gpu - o| <= 1e-5 + 1e-5 |o|
# The absolute/relative terms bound the computed value; the stored bf16 output
# is then rounded to nearest, which alone can move it by half a bf16 ulp (up
# to 2^-8 |o|, more than the 2e-3 relative term for |o| just above a power of
# two), so that quantisation is added explicitly.
TOL = {"bf16": (1e-3, 2e-3), "f32": (1e-5, 1e-5)}


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(ax)) - 8).astype(np.int64))


def gpu_available() -> bool:
    try:
        return torch.cuda.is_available() and torch.cuda.device_count() > 0
    except Exception:
        return False


def run_gpu(wl, mfma: bool = False, decode=None):
    """Compress + one step on the GPU; returns host copies of every output."""
    from indexer_selected_sparse_amd import pipeline
    dp = pipeline.upload(wl, "cuda", decode=decode, mfma_ws=mfma)
    dp.compress()
    dp.step(mfma=mfma)
    torch.cuda.synchronize()
    def host(t):   # byte formats torch cannot copy as such travel as uint8
        if t.dtype in (torch.float4_e2m1fn_x2, torch.float8_e8m0fnu):
            t = t.view(torch.uint8)
        return t.cpu()

    res = {
        "kc": host(dp.kc), "kc_scale": None if dp.kc_scale is None else host(dp.kc_scale),
        "scores": dp.scores.cpu().numpy(), "idx": dp.idx.cpu().numpy(),
        "out": dp.out.float().cpu().numpy().astype(np.float64),
    }
    return res, dp


def kc_bits(kc: torch.Tensor, kind: str) -> np.ndarray:
    if kind == "f32":
        return kc.numpy().view(np.uint32)
    if kind == "bf16":
        return kc.view(torch.int16).numpy().view(np.uint16)
    return kc.view(torch.uint8).numpy()


def oracle_kc_bits(kc: np.ndarray, kind: str) -> np.ndarray:
    return kc.view(np.uint32) if kind == "f32" else kc


def check_compress(wl, res, ref):
    kind = wl.spec.kc_dtype
    n = ref["kc"].shape[0]
    got = kc_bits(res["kc"], kind)[:n]
    exp = oracle_kc_bits(ref["kc"], kind)
    bad = np.argwhere(got != exp)
    assert len(bad) == 0, f"kc mismatch at {bad[:5].tolist()} ({len(bad)} entries)"
    if kind == "e4m3":
        gs = res["kc_scale"].numpy()[:n].view(np.uint32)
        assert np.array_equal(gs, ref["kc_scale"].view(np.uint32)), "kc_scale mismatch"
    if kind == "fp4":
        gs = res["kc_scale"].numpy()[:n]
        assert np.array_equal(gs, ref["kc_scale"]), "fp4 scale bytes mismatch"


def check_scores(wl, res, ref, query_ids):
    Ls = wl.visible_lengths()
    for j, i in enumerate(query_ids):
        nb = int(Ls[i]) // wl.spec.ratio
        got = res["scores"][i, :nb].view(np.uint32)
        exp = ref["scores"][j].view(np.uint32)
        bad = np.nonzero(got != exp)[0]
        assert len(bad) == 0, (f"query {i}: {len(bad)} score bits differ, first at block {bad[0]}: "
                               f"gpu {res['scores'][i, bad[0]]!r} oracle {ref['scores'][j][bad[0]]!r}")


def check_idx(res, ref, query_ids):
    got = res["idx"][np.asarray(query_ids)]
    bad = np.argwhere(got != ref["idx"])
    assert len(bad) == 0, f"idx differs at (row, slot) {bad[:5].tolist()} of {len(bad)}"


def check_out(wl, res, ref, query_ids):
    atol, rtol = TOL[wl.spec.kv_dtype]
    got = res["out"][np.asarray(query_ids)]
    exp = ref["out"]
    err = np.abs(got - exp)
    lim = atol + rtol * np.abs(exp)
    if wl.spec.kv_dtype == "bf16":
        lim = lim + half_ulp_bf16(exp)
    worst = np.unravel_index(np.argmax(err - lim), err.shape)
    assert np.all(err <= lim), (f"output outside tolerance: worst at {worst}: gpu {got[worst]} "
                                f"oracle {exp[worst]} err {err[worst]:.3g} lim {lim[worst]:.3g}")
    return float(np.max(err / lim))


def full_check(wl, query_ids=None, mfma=False, scores=True):
    """GPU step vs oracle on the given queries (all by default)."""
    if query_ids is None:
        query_ids = np.arange(wl.total_q)
    query_ids = np.asarray(query_ids, dtype=np.int64)
    res, dp = run_gpu(wl, mfma=mfma)
    ref = oracle.run_workload(wl, query_ids=query_ids, want_scores=True)
    check_compress(wl, res, ref)
    if scores and not mfma:
        check_scores(wl, res, ref, query_ids)
    check_idx(res, ref, query_ids)
    ratio = check_out(wl, res, ref, query_ids)
    return res, ref, ratio
