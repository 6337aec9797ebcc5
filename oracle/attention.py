"""CPU oracle for the sparse attention that consumes the indexer's
sparse_indices (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The arithmetic lives in
``attention_oracle.c`` (plain C, fp64); this module compiles it with gcc and
marshals numpy arrays through ctypes.  Pinned by
``tests/test_oracle_attention.py``.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

from oracle import compile_source

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attention_oracle.c")
LIBRARY = os.path.join(_HERE, "libattention_oracle.so")
_lock = threading.Lock()
OK, E_ARG = 0, 1


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_source(SOURCE, LIBRARY)
    return LIBRARY


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "the oracle takes C-contiguous numpy arrays"
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


class AttentionOracle:
    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i32, i64, dbl, c_p = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.qlao_bf16_value.argtypes = [ctypes.c_uint16]
        lib.qlao_bf16_value.restype = dbl
        lib.qlao_sparse_attention.argtypes = [i32, i32, i32, c_p, i32, i32, i32, i32, i64, c_p, c_p, c_p, c_p,
                                              c_p, i32, dbl, c_p, c_p, i32]
        lib.qlao_sparse_attention.restype = i32
        self.lib = lib
        self.path = path

    def bf16_value(self, bits: int) -> float:
        return self.lib.qlao_bf16_value(bits)

    def attention(self, a: dict, nthreads: int = 0):
        """a: dict from synth.attention_inputs (or the same keys).  Returns
        (rc, out [rows, heads, head_dim] fp64, lse [rows, heads] fp64)."""
        rows, heads, dim = a["q"].shape
        out = np.zeros((rows, heads, dim), dtype=np.float64)
        lse = np.zeros((rows, heads), dtype=np.float64)
        aslq = None if a.get("aslq") is None else np.ascontiguousarray(a["aslq"], dtype=np.int32)
        rc = self.lib.qlao_sparse_attention(
            a["layout"], a["batch"], a["s1"], _ptr(aslq), heads, dim, a["block_size"], a["max_blocks"],
            a["kv_stride"], _ptr(a["q"]), _ptr(a["k_cache"]), _ptr(a["v_cache"]), _ptr(a["block_table"]),
            _ptr(a["indices"]), a["indices"].shape[1], float(a["scale"]), _ptr(out), _ptr(lse), nthreads)
        return rc, out, lse


_default = None


def get() -> AttentionOracle:
    global _default
    with _lock:
        if _default is None:
            _default = AttentionOracle(build())
    return _default
