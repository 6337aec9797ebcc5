"""Test-side helpers: brute-force references written independently of the
oracle's C code (Python integers, explicit loops over the block table)."""
from __future__ import annotations

import numpy as np


def e4m3_table() -> np.ndarray:
    """float64 value of every float8_e4m3fn code, from torch's conversion."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def scale_array(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def gather_batch(inp: dict, b: int, n: int):
    """Entries 0..n-1 of batch b, walked through the block table in Python:
    returns (keys [n,128] as int or float64 values, kscale [n] float64)."""
    p = inp["problem"]
    bs = p["block_size"]
    stride = p["key_block_stride"] or bs * 128
    table = inp["block_table"].reshape(p["batch"], -1)
    raw = inp["key"]
    ks = inp["k_scale"].reshape(-1)
    keys = np.zeros((n, 128), dtype=np.float64)
    sk = np.zeros(n, dtype=np.float64)
    lut = e4m3_table() if p["qk_dtype"] == 1 else None
    for j in range(n):
        blk = int(table[b, j // bs])
        slot = j % bs
        start = blk * stride + slot * 128
        row = raw[start:start + 128]
        keys[j] = row.view(np.int8).astype(np.float64) if lut is None else lut[row]
        sk[j] = float(ks[blk * bs + slot])
    return keys, sk


def query_values(inp: dict, r: int) -> np.ndarray:
    q = inp["query"].reshape(-1, 64, 128)[r]
    if inp["problem"]["qk_dtype"] == 1:
        return e4m3_table()[q]
    return q.view(np.int8).astype(np.float64)


def brute_dots_int(inp: dict, r: int, b: int, n: int):
    """int8 dots with Python integers: list of 64 lists of n ints."""
    p = inp["problem"]
    bs = p["block_size"]
    stride = p["key_block_stride"] or bs * 128
    table = inp["block_table"].reshape(p["batch"], -1)
    raw = inp["key"].view(np.int8)
    q = inp["query"].reshape(-1, 64, 128)[r].view(np.int8)
    out = []
    for g in range(64):
        qg = [int(x) for x in q[g]]
        row = []
        for j in range(n):
            blk = int(table[b, j // bs])
            start = blk * stride + (j % bs) * 128
            kj = [int(x) for x in raw[start:start + 128]]
            row.append(sum(a * c for a, c in zip(qg, kj)))
        out.append(row)
    return out


def rows_of(p: dict) -> int:
    return p["batch"] * p["s1"] if p["layout_query"] == 0 else p["s1"]
