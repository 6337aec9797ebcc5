"""Quantized lightning indexer for AMD MI355X (gfx950).

Python binding of the C ABI in ``include/qli.h`` (``libqli.so``, built
in-tree by ``python -m sparse_attention_token_paged_amd.build``).  The
functions keep the C names and only marshal arguments: every step of the
indexer runs in the library's HIP kernels.  torch is used for device memory
and streams.  There is no CPU fallback: calling into a missing library
raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libqli.so")

QLI_OK, QLI_ERR_ARG, QLI_ERR_UNSUPPORTED, QLI_ERR_SIZE, QLI_ERR_HIP, QLI_ERR_PLAN = range(6)
QK_INT8, QK_FP8_E4M3FN = 0, 1
SCALE_F16, SCALE_F32 = 0, 1
LAYOUT_BSND, LAYOUT_TND = 0, 1
INT64_MAX = (1 << 63) - 1

EXPORTED = ("qli_status_string", "qli_plan", "qli_plan_info_get", "qli_run", "qli_run_debug", "qli_run_stage",
            "qli_bounded_workspace", "qli_run_bounded", "qli_run_bounded_aslq", "qli_run_bounded_tnd", "qli_run_bounded_static",
            "qli_quantize_query", "qli_append_keys", "qli_sparse_attention_workspace", "qli_sparse_attention")

c_i32, c_i64, c_p, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


class Problem(ctypes.Structure):
    """Mirror of ``qli_problem`` (fixed-width, explicitly padded)."""
    _fields_ = [
        ("batch", c_i32), ("s1", c_i32), ("num_heads_q", c_i32), ("num_heads_k", c_i32),
        ("head_dim", c_i32), ("layout_query", c_i32), ("qk_dtype", c_i32), ("scale_dtype", c_i32),
        ("num_blocks", c_i32), ("block_size", c_i32), ("max_blocks_per_seq", c_i32), ("reserved0", c_i32),
        ("key_block_stride", c_i64),
        ("sparse_count", c_i32), ("sparse_mode", c_i32), ("cmp_ratio", c_i32), ("reserved1", c_i32),
        ("pre_tokens", c_i64), ("next_tokens", c_i64),
        ("query_quant_mode", c_i32), ("key_quant_mode", c_i32), ("return_value", c_i32), ("sort_output", c_i32),
    ]

    @classmethod
    def from_dict(cls, d: dict) -> "Problem":
        p = cls()
        for name, _ in cls._fields_:
            if name in d:
                setattr(p, name, int(d[name]))
        return p


class AttnProblem(ctypes.Structure):
    """Mirror of ``qli_attn_problem`` (the sparse-attention consumer)."""
    _fields_ = [
        ("batch", c_i32), ("s1", c_i32), ("layout_query", c_i32), ("num_heads", c_i32),
        ("head_dim", c_i32), ("num_blocks", c_i32), ("block_size", c_i32), ("max_blocks_per_seq", c_i32),
        ("kv_block_stride", c_i64),
        ("sparse_count", c_i32), ("softmax_scale", ctypes.c_float), ("return_lse", c_i32), ("reserved0", c_i32),
        ("reserved1", c_i32), ("reserved2", c_i32),
    ]

    @classmethod
    def from_dict(cls, d: dict) -> "AttnProblem":
        p = cls()
        for name, _ in cls._fields_:
            if name in d:
                setattr(p, name, float(d[name]) if name == "softmax_scale" else int(d[name]))
        return p


class PlanInfo(ctypes.Structure):
    """Mirror of ``qli_plan_info``."""
    _fields_ = [("rows", c_i64), ("visible_pairs", c_i64), ("plan_bytes", c_i64),
                ("workspace_bytes", c_i64), ("key_entries", c_i64), ("table_entries", c_i64),
                ("active_rows", c_i64), ("score_items", c_i32), ("select_rows", c_i32),
                ("rows_per_item", c_i32), ("keys_per_chunk", c_i32), ("kind", c_i32), ("reserved", c_i32)]


_lib = None
_lock = threading.Lock()


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libqli.so; raises RuntimeError if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIBRARY
        if not os.path.exists(p):
            raise RuntimeError("libqli.so is missing (%s); build it with "
                               "`python -m sparse_attention_token_paged_amd.build`" % p)
        lib = ctypes.CDLL(p)
        lib.qli_status_string.argtypes = [ctypes.c_int]
        lib.qli_status_string.restype = ctypes.c_char_p
        lib.qli_plan.argtypes = [ctypes.POINTER(Problem), c_p, c_p, c_p, c_sz,
                                 ctypes.POINTER(c_sz), ctypes.POINTER(c_sz)]
        lib.qli_plan.restype = ctypes.c_int
        lib.qli_plan_info_get.argtypes = [c_p, ctypes.POINTER(PlanInfo)]
        lib.qli_plan_info_get.restype = ctypes.c_int
        lib.qli_run.argtypes = [ctypes.POINTER(Problem), c_p, c_p] + [c_p] * 9 + [c_p]
        lib.qli_run.restype = ctypes.c_int
        lib.qli_run_debug.argtypes = ([ctypes.POINTER(Problem), c_p, c_p] + [c_p] * 9 +
                                      [c_i64, c_i64, c_i64, c_p, c_p, c_p])
        lib.qli_run_debug.restype = ctypes.c_int
        lib.qli_run_stage.argtypes = [ctypes.POINTER(Problem), c_p, c_p] + [c_p] * 9 + [c_i32, c_p]
        lib.qli_run_stage.restype = ctypes.c_int
        lib.qli_bounded_workspace.argtypes = [ctypes.POINTER(Problem), c_i64, ctypes.POINTER(c_sz)]
        lib.qli_bounded_workspace.restype = ctypes.c_int
        lib.qli_run_bounded.argtypes = [ctypes.POINTER(Problem), c_i64] + [c_p] * 10 + [c_p]
        lib.qli_run_bounded.restype = ctypes.c_int
        lib.qli_run_bounded_tnd.argtypes = [ctypes.POINTER(Problem), c_i64] + [c_p] * 11 + [c_p]
        lib.qli_run_bounded_tnd.restype = ctypes.c_int
        lib.qli_run_bounded_aslq.argtypes = [ctypes.POINTER(Problem), c_i64] + [c_p] * 11 + [c_p]
        lib.qli_run_bounded_aslq.restype = ctypes.c_int
        lib.qli_run_bounded_static.argtypes = [ctypes.POINTER(Problem), c_i64] + [c_p] * 9 + [c_p]
        lib.qli_run_bounded_static.restype = ctypes.c_int
        lib.qli_sparse_attention_workspace.argtypes = [ctypes.POINTER(AttnProblem), ctypes.POINTER(c_sz)]
        lib.qli_sparse_attention_workspace.restype = ctypes.c_int
        lib.qli_sparse_attention.argtypes = [ctypes.POINTER(AttnProblem)] + [c_p] * 10
        lib.qli_sparse_attention.restype = ctypes.c_int
        lib.qli_quantize_query.argtypes = [c_i32, c_i64, c_p, c_p, c_p, c_p]
        lib.qli_quantize_query.restype = ctypes.c_int
        lib.qli_append_keys.argtypes = [c_i32, c_i64, c_p, c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_i64,
                                        c_p, c_p, c_p]
        lib.qli_append_keys.restype = ctypes.c_int
        if path is None:
            _lib = lib
        return lib


class QliError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__("%s failed: %s (%d)" % (what, qli_status_string(code), code))
        self.code = code


def qli_status_string(code: int) -> str:
    return load().qli_status_string(code).decode()


def _addr(x) -> Optional[int]:
    """Device or host address of a torch tensor / numpy array / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data
    # torch.Tensor
    assert x.is_contiguous(), "tensors passed to the indexer must be contiguous"
    return x.data_ptr()


def qli_plan(problem: Problem, aslq, aslk):
    """Returns (status, plan bytes as a uint8 numpy array, workspace bytes)."""
    lib = load()
    aq = None if aslq is None else np.ascontiguousarray(aslq, dtype=np.int32)
    ak = None if aslk is None else np.ascontiguousarray(aslk, dtype=np.int32)
    nb, ws = c_sz(0), c_sz(0)
    rc = lib.qli_plan(ctypes.byref(problem), _addr(aq), _addr(ak), None, 0, ctypes.byref(nb), ctypes.byref(ws))
    if rc != QLI_OK:
        return rc, None, 0
    buf = np.zeros(nb.value, dtype=np.uint8)
    rc = lib.qli_plan(ctypes.byref(problem), _addr(aq), _addr(ak), _addr(buf), buf.size,
                      ctypes.byref(nb), ctypes.byref(ws))
    return rc, (buf if rc == QLI_OK else None), ws.value


def qli_plan_info_get(plan_host: np.ndarray) -> PlanInfo:
    info = PlanInfo()
    rc = load().qli_plan_info_get(_addr(plan_host), ctypes.byref(info))
    if rc != QLI_OK:
        raise QliError(rc, "qli_plan_info_get")
    return info


def qli_run(problem: Problem, plan_host, plan_dev, query, key, weights, q_scale, k_scale,
            block_table, workspace, sparse_indices, sparse_values, stream=None) -> int:
    return load().qli_run(ctypes.byref(problem), _addr(plan_host), _addr(plan_dev), _addr(query),
                          _addr(key), _addr(weights), _addr(q_scale), _addr(k_scale),
                          _addr(block_table), _addr(workspace), _addr(sparse_indices),
                          _addr(sparse_values), stream)


def qli_run_stage(problem: Problem, plan_host, plan_dev, query, key, weights, q_scale, k_scale,
                  block_table, workspace, sparse_indices, sparse_values, stages: int, stream=None) -> int:
    """stages: 1 = scoring kernel only, 2 = final selection only, 3 = both (qli_run)."""
    return load().qli_run_stage(ctypes.byref(problem), _addr(plan_host), _addr(plan_dev), _addr(query),
                                _addr(key), _addr(weights), _addr(q_scale), _addr(k_scale),
                                _addr(block_table), _addr(workspace), _addr(sparse_indices),
                                _addr(sparse_values), stages, stream)


def qli_run_debug(problem: Problem, plan_host, plan_dev, query, key, weights, q_scale, k_scale,
                  block_table, workspace, sparse_indices, sparse_values, row0, row1, cols,
                  dots_out, scores_out, stream=None) -> int:
    return load().qli_run_debug(ctypes.byref(problem), _addr(plan_host), _addr(plan_dev), _addr(query),
                                _addr(key), _addr(weights), _addr(q_scale), _addr(k_scale),
                                _addr(block_table), _addr(workspace), _addr(sparse_indices),
                                _addr(sparse_values), row0, row1, cols, _addr(dots_out),
                                _addr(scores_out), stream)


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def qli_bounded_workspace(problem: Problem, max_seq_len_key: int):
    """Returns (status, workspace bytes) for qli_run_bounded."""
    ws = c_sz(0)
    rc = load().qli_bounded_workspace(ctypes.byref(problem), int(max_seq_len_key), ctypes.byref(ws))
    return rc, int(ws.value)


def qli_run_bounded(problem: Problem, max_seq_len_key: int, aslk_dev, query, key, weights, q_scale, k_scale,
                    block_table, workspace, sparse_indices, sparse_values, stream=None) -> int:
    return load().qli_run_bounded(ctypes.byref(problem), int(max_seq_len_key), _addr(aslk_dev), _addr(query),
                                  _addr(key), _addr(weights), _addr(q_scale), _addr(k_scale),
                                  _addr(block_table), _addr(workspace), _addr(sparse_indices),
                                  _addr(sparse_values), stream)


def qli_run_bounded_static(problem: Problem, max_seq_len_key: int, aslk_dev, query, key, weights, q_scale,
                           k_scale, block_table, sparse_indices, sparse_values, stream=None) -> int:
    """qli_run_bounded without a workspace argument (the library's static one)."""
    return load().qli_run_bounded_static(ctypes.byref(problem), int(max_seq_len_key), _addr(aslk_dev),
                                         _addr(query), _addr(key), _addr(weights), _addr(q_scale),
                                         _addr(k_scale), _addr(block_table), _addr(sparse_indices),
                                         _addr(sparse_values), stream)


def qli_quantize_query(qk_dtype: int, rows: int, x, q_out, scale_out, stream=None) -> int:
    """x: bf16 [rows, 128] (rows = tokens * 64 heads); q_out: [rows, 128] int8 or
    e4m3fn codes; scale_out: [rows] fp16 (int8) or fp32 (e4m3fn)."""
    return load().qli_quantize_query(int(qk_dtype), int(rows), _addr(x), _addr(q_out), _addr(scale_out), stream)


def qli_append_keys(qk_dtype: int, n: int, x, batch_idx, pos, block_table, batch_count: int,
                    max_blocks_per_seq: int, num_blocks: int, block_size: int, key_block_stride: int,
                    key_cache, k_scale, stream=None) -> int:
    """x: bf16 [n, 128] key entries; entry e goes to position pos[e] of sequence
    batch_idx[e] in the paged cache key_cache / k_scale through block_table."""
    return load().qli_append_keys(int(qk_dtype), int(n), _addr(x), _addr(batch_idx), _addr(pos),
                                  _addr(block_table), int(batch_count), int(max_blocks_per_seq),
                                  int(num_blocks), int(block_size), int(key_block_stride),
                                  _addr(key_cache), _addr(k_scale), stream)


def quantize_query(x, qk_dtype: int = QK_INT8, stream: Optional[int] = None):
    """Per-token-head quantization of a bf16 query [..., 64, 128] (torch, on
    the GPU): returns (codes uint8 [..., 64, 128], scales [..., 64]) as the
    query / query_dequant_scale inputs of the indexer."""
    import torch
    assert x.dtype == torch.bfloat16 and x.shape[-1] == 128 and x.is_contiguous()
    rows = x.numel() // 128
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    sc = torch.empty(x.shape[:-1], dtype=torch.float16 if qk_dtype == QK_INT8 else torch.float32, device=x.device)
    rc = qli_quantize_query(qk_dtype, rows, x, q, sc, current_stream() if stream is None else stream)
    if rc != QLI_OK:
        raise QliError(rc, "qli_quantize_query")
    return q, sc


def qli_run_bounded_aslq(problem: Problem, max_seq_len_key: int, aslq_dev, aslk_dev, query, key, weights, q_scale,
                         k_scale, block_table, workspace, sparse_indices, sparse_values, stream=None) -> int:
    return load().qli_run_bounded_aslq(ctypes.byref(problem), int(max_seq_len_key), _addr(aslq_dev), _addr(aslk_dev),
                                       _addr(query), _addr(key), _addr(weights), _addr(q_scale), _addr(k_scale),
                                       _addr(block_table), _addr(workspace), _addr(sparse_indices),
                                       _addr(sparse_values), stream)


def qli_run_bounded_tnd(problem: Problem, max_seq_len_key: int, aslq_dev, aslk_dev, query, key, weights, q_scale,
                        k_scale, block_table, workspace, sparse_indices, sparse_values, stream=None) -> int:
    return load().qli_run_bounded_tnd(ctypes.byref(problem), int(max_seq_len_key), _addr(aslq_dev), _addr(aslk_dev),
                                      _addr(query), _addr(key), _addr(weights), _addr(q_scale), _addr(k_scale),
                                      _addr(block_table), _addr(workspace), _addr(sparse_indices),
                                      _addr(sparse_values), stream)


class BoundedIndexer:
    """Bounded decode: no host plan; the key lengths stay on the device and
    may change between calls (or graph replays) up to max_seq_len_key.
    Holds the problem, the bound and a workspace (torch; marshalling only)."""

    def __init__(self, problem: dict, max_seq_len_key: int, device: str = "cuda"):
        import torch
        self.problem = Problem.from_dict(problem)
        self.max_seq_len_key = int(max_seq_len_key)
        rc, ws = qli_bounded_workspace(self.problem, self.max_seq_len_key)
        if rc != QLI_OK:
            raise QliError(rc, "qli_bounded_workspace")
        self.workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=device) if ws else None
        self.device = device

    def alloc_outputs(self):
        import torch
        tnd = self.problem.layout_query == LAYOUT_TND
        rows = self.problem.s1 if tnd else self.problem.batch * self.problem.s1
        k = self.problem.sparse_count
        idx = torch.empty((rows, k), dtype=torch.int32, device=self.device)
        val = torch.empty((rows, k), dtype=torch.float32, device=self.device) if self.problem.return_value else None
        return idx, val

    def run(self, aslk_dev, query, key, weights, q_scale, k_scale, block_table, out_idx, out_val,
            stream: Optional[int] = None, aslq_dev=None):
        """aslq_dev: device actual_seq_lengths_query (TND: required prefix sums;
        BSND: optional per-batch query counts)."""
        st = current_stream() if stream is None else stream
        if self.problem.layout_query == LAYOUT_TND:
            rc = qli_run_bounded_tnd(self.problem, self.max_seq_len_key, aslq_dev, aslk_dev, query, key, weights,
                                     q_scale, k_scale, block_table, self.workspace, out_idx, out_val, st)
        elif aslq_dev is not None:
            rc = qli_run_bounded_aslq(self.problem, self.max_seq_len_key, aslq_dev, aslk_dev, query, key, weights,
                                      q_scale, k_scale, block_table, self.workspace, out_idx, out_val, st)
        else:
            rc = qli_run_bounded(self.problem, self.max_seq_len_key, aslk_dev, query, key, weights, q_scale,
                                 k_scale, block_table, self.workspace, out_idx, out_val, st)
        if rc != QLI_OK:
            raise QliError(rc, "qli_run_bounded")
        return out_idx, out_val


class Indexer:
    """Plan once, run many times: holds the host plan, its device copy and a
    zero-filled workspace (torch allocations; marshalling only).

    problem: dict with the qli_problem fields; aslq / aslk: host int arrays.
    """

    def __init__(self, problem: dict, aslq, aslk, device: str = "cuda"):
        import torch
        self.problem = Problem.from_dict(problem)
        rc, plan, ws = qli_plan(self.problem, aslq, aslk)
        if rc != QLI_OK:
            raise QliError(rc, "qli_plan")
        self.plan_host = plan
        self.info = qli_plan_info_get(plan)
        self.plan_dev = torch.from_numpy(plan.copy()).to(device)
        self.workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=device) if ws else None
        self.device = device

    @property
    def rows(self) -> int:
        return int(self.info.rows)

    def alloc_outputs(self):
        import torch
        k = self.problem.sparse_count
        idx = torch.empty((self.rows, k), dtype=torch.int32, device=self.device)
        val = torch.empty((self.rows, k), dtype=torch.float32, device=self.device) if self.problem.return_value else None
        return idx, val

    def run(self, query, key, weights, q_scale, k_scale, block_table, out_idx=None, out_val=None,
            stream: Optional[int] = None):
        if out_idx is None:
            out_idx, out_val = self.alloc_outputs()
        st = current_stream() if stream is None else stream
        rc = qli_run(self.problem, self.plan_host, self.plan_dev, query, key, weights, q_scale, k_scale,
                     block_table, self.workspace, out_idx, out_val, st)
        if rc != QLI_OK:
            raise QliError(rc, "qli_run")
        return out_idx, out_val

    def run_stage(self, query, key, weights, q_scale, k_scale, block_table, out_idx, out_val, stages: int,
                  stream: Optional[int] = None):
        st = current_stream() if stream is None else stream
        rc = qli_run_stage(self.problem, self.plan_host, self.plan_dev, query, key, weights, q_scale, k_scale,
                           block_table, self.workspace, out_idx, out_val, stages, st)
        if rc != QLI_OK:
            raise QliError(rc, "qli_run_stage")
        return out_idx, out_val

    def run_debug(self, query, key, weights, q_scale, k_scale, block_table, row0, row1, cols,
                  stream: Optional[int] = None):
        import torch
        out_idx, out_val = self.alloc_outputs()
        dt = torch.int32 if self.problem.qk_dtype == QK_INT8 else torch.float32
        dots = torch.zeros(((row1 - row0) * 64 * cols,), dtype=dt, device=self.device)
        scores = torch.full(((row1 - row0) * cols,), float("nan"), dtype=torch.float32, device=self.device)
        st = current_stream() if stream is None else stream
        rc = qli_run_debug(self.problem, self.plan_host, self.plan_dev, query, key, weights, q_scale,
                           k_scale, block_table, self.workspace, out_idx, out_val, row0, row1, cols,
                           dots if dots.numel() else None, scores if scores.numel() else None, st)
        if rc != QLI_OK:
            raise QliError(rc, "qli_run_debug")
        return out_idx, out_val, dots.view(row1 - row0, 64, cols), scores.view(row1 - row0, cols)


def qli_sparse_attention_workspace(problem: AttnProblem):
    """Returns (status, workspace bytes) for qli_sparse_attention."""
    ws = c_sz(0)
    rc = load().qli_sparse_attention_workspace(ctypes.byref(problem), ctypes.byref(ws))
    return rc, int(ws.value)


def qli_sparse_attention(problem: AttnProblem, aslq_dev, q, k_cache, v_cache, block_table, sparse_indices,
                         workspace, out, lse, stream=None) -> int:
    return load().qli_sparse_attention(ctypes.byref(problem), _addr(aslq_dev), _addr(q), _addr(k_cache),
                                       _addr(v_cache), _addr(block_table), _addr(sparse_indices),
                                       _addr(workspace), _addr(out), _addr(lse), stream)


class SparseAttention:
    """The consumer of sparse_indices: holds the problem and its workspace
    (torch; marshalling only).  problem: dict with the qli_attn_problem fields."""

    def __init__(self, problem: dict, device: str = "cuda"):
        import torch
        self.problem = AttnProblem.from_dict(problem)
        rc, ws = qli_sparse_attention_workspace(self.problem)
        if rc != QLI_OK:
            raise QliError(rc, "qli_sparse_attention_workspace")
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device) if ws else None
        self.device = device

    @property
    def rows(self) -> int:
        p = self.problem
        return p.batch * p.s1 if p.layout_query == LAYOUT_BSND else p.s1

    def alloc_outputs(self):
        import torch
        p = self.problem
        out = torch.empty((self.rows, p.num_heads, p.head_dim), dtype=torch.bfloat16, device=self.device)
        lse = torch.empty((self.rows, p.num_heads), dtype=torch.float32, device=self.device) if p.return_lse else None
        return out, lse

    def run(self, q, k_cache, v_cache, block_table, sparse_indices, out=None, lse=None, aslq_dev=None,
            stream: Optional[int] = None):
        if out is None:
            out, lse = self.alloc_outputs()
        st = current_stream() if stream is None else stream
        rc = qli_sparse_attention(self.problem, aslq_dev, q, k_cache, v_cache, block_table, sparse_indices,
                                  self.workspace, out, lse, st)
        if rc != QLI_OK:
            raise QliError(rc, "qli_sparse_attention")
        return out, lse
