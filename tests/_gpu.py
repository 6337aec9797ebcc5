"""GPU-side test harness: moves synthetic inputs to the device, runs the HIP
library through its C ABI, and checks results against the oracle with the
parity rule of the indexer.

Parity rule per row r (n = min(k, vis)):
  * structure: sparse_indices[r, :n] strictly ascending in [0, vis), the rest
    -1; sparse_values[r, n:] = -inf;
  * scores: |gpu - oracle| <= atol + rtol * |oracle| for every returned index
    (int8: rtol 1e-5, atol 1e-6; fp8: rtol 2e-3, atol 1e-6);
  * sets: vis <= k gives exactly {0..vis-1}; otherwise with tau = the
    oracle's k-th score (stable order) and tol = atol + rtol*|tau|, any index
    the GPU adds has an oracle score >= tau - tol and any it drops <= tau + tol.
"""
from __future__ import annotations

import sys

import numpy as np

INT8_RTOL, FP8_RTOL, ATOL = 1e-5, 2e-3, 1e-6


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(inp: dict):
    import torch
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return dict(query=t(inp["query"].view(np.uint8)), key=t(inp["key"]), weights=t(inp["weights"]),
                q_scale=t(inp["q_scale"]), k_scale=t(inp["k_scale"]), block_table=t(inp["block_table"]))


def make_indexer(inp: dict):
    import sparse_attention_token_paged_amd as qli
    return qli.Indexer(inp["problem"], inp["aslq"], inp["aslk"])


def run_gpu(inp: dict, dev=None, ix=None):
    import torch
    ix = ix or make_indexer(inp)
    dev = dev or device_inputs(inp)
    idx, val = ix.run(dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"])
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (val.cpu().numpy() if val is not None else None), ix


def rtol_of(inp: dict) -> float:
    return FP8_RTOL if inp["problem"]["qk_dtype"] == 1 else INT8_RTOL


def check_structure(idx: np.ndarray, val, vis: np.ndarray, k: int) -> None:
    """Vectorised structural checks over every row."""
    n = np.minimum(vis, k)
    cols = np.arange(k)[None, :]
    live = cols < n[:, None]
    assert np.all(idx[~live] == -1), "padding indices must be -1"
    if val is not None:
        assert np.all(val[~live] == -np.inf), "padding values must be -inf"
        assert np.all(np.isfinite(val[live])), "returned values must be finite"
    assert np.all(idx[live] >= 0)
    assert np.all((idx < vis[:, None])[live]), "index beyond the visible range"
    d = np.diff(idx, axis=1)
    both = live[:, 1:]
    assert np.all(d[both] > 0), "returned indices must be strictly ascending"


def check_row(r: int, vis: int, k: int, gidx: np.ndarray, gval, scores: np.ndarray, rtol: float) -> None:
    n = min(k, vis)
    sel = gidx[:n].astype(np.int64)
    if gval is not None:
        ref = scores[sel]
        err = np.abs(gval[:n].astype(np.float64) - ref)
        bad = err > ATOL + rtol * np.abs(ref)
        assert not bad.any(), "row %d: %d scores out of tolerance, worst %r" % (
            r, bad.sum(), (sel[bad][:3], gval[:n][bad][:3], ref[bad][:3]))
    if vis <= k:
        assert np.array_equal(sel, np.arange(vis)), "row %d: must return every visible index" % r
        return
    order = np.argsort(-scores, kind="stable")
    tau = scores[order[k - 1]]
    tol = ATOL + rtol * abs(tau)
    g, o = set(sel.tolist()), set(order[:k].tolist())
    extra = [i for i in g - o if scores[i] < tau - tol]
    missing = [i for i in o - g if scores[i] > tau + tol]
    assert not extra and not missing, "row %d: set differs beyond tolerance: extra %r missing %r (tau %r)" % (
        r, extra[:5], missing[:5], tau)


def stable_topk_set(scores32: np.ndarray, k: int) -> np.ndarray:
    """Top-k of fp32 scores, ties to the lower index, as sorted indices."""
    order = np.argsort(-scores32.astype(np.float64), kind="stable")
    return np.sort(order[:k])
