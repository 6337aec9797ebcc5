"""CPU oracle of the producer side: per-token-head quantization of the index
query and key (test infrastructure only; the same import rules as the rest of
this package).

The page (EngineX-Ascend "VllmQuantLightningIndexer", 功能说明: query and key
stored and computed in 8 bits; 参数说明 query_quant_mode / key_quant_mode:
per-token-head) names the mode but gives no formula.  reading: symmetric
absmax quantization of each 128-element head vector, every step in fp32 (the
precision the codes are decided in on the GPU), exactly as include/qli.h
states it:

  int8 codes, fp16 scale:    s = fp16(amax / 127) (65504 on overflow),
                             q = clamp(rint(x * (1 / s)), -127, 127), 0 when s == 0
  e4m3fn codes, fp32 scale:  s = amax / 448,
                             q = e4m3fn(clamp(x * (1 / s), -448, 448)), 0 when s == 0
                             or 1 / s is not finite

Plain numpy float32 arithmetic (IEEE, round to nearest even) in the order
written above.  The e4m3fn encoder picks the nearest of the format's values
by enumeration over the decoder's table (ties to the even code), not by bit
manipulation.
"""
from __future__ import annotations

import numpy as np

from . import get as _get_oracle

_E4M3_TABLE = None


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3fn_magnitudes() -> np.ndarray:
    """Values of the codes 0x00..0x7E (all finite non-negative magnitudes),
    from the oracle's OCP E4M3FN decoder."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        ora = _get_oracle()
        _E4M3_TABLE = np.array([ora.e4m3fn_value(c) for c in range(0x7F)], dtype=np.float64)
    return _E4M3_TABLE


def e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """OCP E4M3FN code of each finite float32 y with |y| <= 448: the code whose
    value is nearest to |y|, ties to the code with an even mantissa (even code),
    and the sign bit of y (so -0.0 and negatives that round to 0 give 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64).ravel()
    tab = e4m3fn_magnitudes()
    assert np.all(a <= 448.0), "e4m3fn_encode takes |y| <= 448"
    hi = np.searchsorted(tab, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, len(tab) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - tab[lo], tab[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(tab[hi] == a, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = np.signbit(y.ravel()).astype(np.uint8) << 7
    return (code | sign).reshape(y.shape)


def quantize_rows(x_bits: np.ndarray, qk_dtype: int):
    """Rows of 128 bf16 values -> (codes uint8 [n, 128], scales [n]); scales are
    float16 for int8 (qk_dtype 0) and float32 for e4m3fn (qk_dtype 1)."""
    x = bf16_to_f32(np.asarray(x_bits).reshape(-1, 128))
    n = x.shape[0]
    codes = np.zeros((n, 128), dtype=np.uint8)
    amax = np.max(np.abs(x), axis=1) if n else np.zeros(0, np.float32)
    if qk_dtype == 0:
        with np.errstate(over="ignore"):
            s16 = (amax / np.float32(127.0)).astype(np.float16)
        s16[np.isinf(s16)] = np.float16(65504.0)
        for i in range(n):
            s = np.float32(s16[i])
            if s == 0:
                continue
            r = np.float32(1.0) / s
            q = np.clip(np.rint(x[i] * r), -127, 127).astype(np.int8)
            codes[i] = q.view(np.uint8)
        return codes, s16
    s32 = (amax / np.float32(448.0)).astype(np.float32)
    for i in range(n):
        s = s32[i]
        if s == 0:
            continue
        with np.errstate(divide="ignore", over="ignore"):
            r = np.float32(1.0) / s
        if not np.isfinite(r):
            continue
        y = np.clip(x[i] * r, np.float32(-448.0), np.float32(448.0))
        codes[i] = e4m3fn_encode(y)
    return codes, s32


def append_keys(x_bits, batch_idx, pos, block_table, batch_count, max_blocks, num_blocks, block_size,
                stride, key_cache: np.ndarray, k_scale: np.ndarray, qk_dtype: int) -> None:
    """Quantize key entries and write them in place into numpy copies of the
    paged cache (key_cache: uint8 [num_blocks * stride]; k_scale: [num_blocks *
    block_size]); entries whose sequence, position or block is outside the
    cache are skipped."""
    codes, scales = quantize_rows(x_bits, qk_dtype)
    bt = np.asarray(block_table).reshape(-1)
    for e in range(codes.shape[0]):
        b, p = int(batch_idx[e]), int(pos[e])
        if b < 0 or b >= batch_count or p < 0 or p // block_size >= max_blocks:
            continue
        blk = int(bt[b * max_blocks + p // block_size])
        if blk < 0 or blk >= num_blocks:
            continue
        o = p % block_size
        key_cache[blk * stride + o * 128: blk * stride + o * 128 + 128] = codes[e]
        k_scale[blk * block_size + o] = scales[e]
