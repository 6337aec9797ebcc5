"""CPU oracle for the quantized lightning indexer (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library in
``sparse_attention_token_paged_amd``) never does, and the two share no code.

The arithmetic lives in ``qli_oracle.c`` (plain C, fp64, exact integer dots);
this module only compiles it with gcc and marshals numpy arrays through
ctypes.  Every function is pinned by ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

INT64_MAX = (1 << 63) - 1  # the pre_tokens / next_tokens default: no window

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "qli_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()

OK, E_ARG, E_UNSUPPORTED = 0, 1, 2


def compile_source(src: str, out: str) -> str:
    """gcc -O2 -fopenmp shared library from one C file."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Wno-unused-parameter", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile qli_oracle.c into oracle/liboracle.so."""
    if force or not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_source(SOURCE, LIBRARY)
    return LIBRARY


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle takes C-contiguous numpy arrays"
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


class Oracle:
    """ctypes view of one build of qli_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        c_p = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        lib.qlio_e4m3fn_value.argtypes = [ctypes.c_uint8]
        lib.qlio_e4m3fn_value.restype = ctypes.c_double
        lib.qlio_f16_value.argtypes = [ctypes.c_uint16]
        lib.qlio_f16_value.restype = ctypes.c_double
        lib.qlio_visible.argtypes = [i32, i32, i64, i64, i64]
        lib.qlio_visible.restype = i64
        lib.qlio_topk.argtypes = [c_p, i64, i64, c_p]
        lib.qlio_topk.restype = i64
        lib.qlio_row_visible.argtypes = [i32, i32, i32, i32, i32, c_p, c_p, c_p]
        lib.qlio_row_visible.restype = i32
        lib.qlio_visible_range.argtypes = [i32, i32, i64, i64, i64, i64, i64, c_p]
        lib.qlio_visible_range.restype = i64
        lib.qlio_row_range.argtypes = [i32, i32, i32, i32, i32, c_p, c_p, i64, i64, c_p, c_p]
        lib.qlio_row_range.restype = i32
        lib.qlio_indexer.argtypes = [i32] * 8 + [i64] + [i32] * 3 + [i64, i64] + [c_p] * 10 + [c_p, i64, i32]
        lib.qlio_indexer.restype = i32
        lib.qlio_row_detail.argtypes = [i32] * 7 + [i64] + [i32, i32] + [c_p] * 8 + [i64, i64, i64, c_p, c_p]
        lib.qlio_row_detail.restype = i64
        self.lib = lib
        self.path = path

    def e4m3fn_value(self, code: int) -> float:
        return self.lib.qlio_e4m3fn_value(code)

    def f16_value(self, bits: int) -> float:
        return self.lib.qlio_f16_value(bits)

    def visible(self, sparse_mode: int, cmp_ratio: int, skb: int, s1b: int, i: int) -> int:
        return self.lib.qlio_visible(sparse_mode, cmp_ratio, skb, s1b, i)

    def topk(self, scores, k: int) -> np.ndarray:
        s = np.ascontiguousarray(scores, dtype=np.float64)
        out = np.empty(max(0, min(k, s.size)), dtype=np.int64)
        n = self.lib.qlio_topk(_ptr(s), s.size, k, _ptr(out))
        assert n == out.size
        return out

    def row_visible(self, layout, batch, s1_or_t, sparse_mode, cmp_ratio, aslq, aslk) -> np.ndarray:
        rows = batch * s1_or_t if layout == 0 else s1_or_t
        out = np.zeros(rows, dtype=np.int64)
        aq = None if aslq is None else np.ascontiguousarray(aslq, dtype=np.int32)
        ak = np.ascontiguousarray(aslk, dtype=np.int32)
        self.lib.qlio_row_visible(layout, batch, s1_or_t, sparse_mode, cmp_ratio, _ptr(aq), _ptr(ak), _ptr(out))
        return out

    def visible_range(self, sparse_mode: int, cmp_ratio: int, skb: int, s1b: int, i: int,
                      pre_tokens: int = INT64_MAX, next_tokens: int = INT64_MAX):
        """(lo, hi): query i sees entries [lo, hi)."""
        lo = ctypes.c_int64(0)
        hi = self.lib.qlio_visible_range(sparse_mode, cmp_ratio, skb, s1b, i, pre_tokens, next_tokens,
                                         ctypes.byref(lo))
        return lo.value, hi

    def row_range(self, layout, batch, s1_or_t, sparse_mode, cmp_ratio, aslq, aslk,
                  pre_tokens=INT64_MAX, next_tokens=INT64_MAX):
        """(lo[rows], hi[rows]): row r sees entries [lo[r], hi[r])."""
        rows = batch * s1_or_t if layout == 0 else s1_or_t
        lo = np.zeros(rows, dtype=np.int64)
        hi = np.zeros(rows, dtype=np.int64)
        aq = None if aslq is None else np.ascontiguousarray(aslq, dtype=np.int32)
        ak = np.ascontiguousarray(aslk, dtype=np.int32)
        self.lib.qlio_row_range(layout, batch, s1_or_t, sparse_mode, cmp_ratio, _ptr(aq), _ptr(ak),
                                pre_tokens, next_tokens, _ptr(lo), _ptr(hi))
        return lo, hi

    def indexer(self, inp: dict, *, scores_cols: int = 0, nthreads: int = 0):
        """Whole operator.  Returns (rc, indices[rows,k], values[rows,k], scores or None)."""
        p = inp["problem"]
        rows = p["batch"] * p["s1"] if p["layout_query"] == 0 else p["s1"]
        k = p["sparse_count"]
        idx = np.empty((rows, k), dtype=np.int32)
        val = np.empty((rows, k), dtype=np.float32)
        sc = np.full((rows, scores_cols), np.nan, dtype=np.float64) if scores_cols > 0 else None
        rc = self.lib.qlio_indexer(
            p["qk_dtype"], p["scale_dtype"], p["layout_query"], p["batch"], p["s1"],
            p["num_blocks"], p["block_size"], p["max_blocks_per_seq"], p["key_block_stride"],
            p["sparse_count"], p["sparse_mode"], p["cmp_ratio"],
            p.get("pre_tokens", INT64_MAX), p.get("next_tokens", INT64_MAX),
            _ptr(inp["query"]), _ptr(inp["key"]), _ptr(inp["weights"]), _ptr(inp["q_scale"]),
            _ptr(inp["k_scale"]), _ptr(inp["aslq"]), _ptr(inp["aslk"]), _ptr(inp["block_table"]),
            _ptr(idx), _ptr(val), _ptr(sc), scores_cols, nthreads)
        return rc, idx, val, sc

    def row_detail(self, inp: dict, row: int, j0: int, j1: int):
        """fp64 dots [64, j1-j0] and scores [j1-j0] of one row; returns (vis, dots, scores)."""
        p = inp["problem"]
        n = max(j1 - j0, 0)
        dots = np.zeros((64, n), dtype=np.float64)
        sc = np.zeros(n, dtype=np.float64)
        vis = self.lib.qlio_row_detail(
            p["qk_dtype"], p["scale_dtype"], p["layout_query"], p["batch"], p["s1"],
            p["block_size"], p["max_blocks_per_seq"], p["key_block_stride"],
            p["sparse_mode"], p["cmp_ratio"],
            _ptr(inp["query"]), _ptr(inp["key"]), _ptr(inp["weights"]), _ptr(inp["q_scale"]),
            _ptr(inp["k_scale"]), _ptr(inp["aslq"]), _ptr(inp["aslk"]), _ptr(inp["block_table"]),
            row, j0, j1, _ptr(dots), _ptr(sc))
        return vis, dots, sc


_default = None


def get() -> Oracle:
    """The oracle built from qli_oracle.c (compiled on first use)."""
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())
    return _default
