"""Seeded synthetic inputs for the quantized lightning indexer.

This module only draws random data with the shapes, dtypes and value
distributions of the workloads; it holds none of the indexer's arithmetic.
It is the one module that both the HIP path's tests/benchmark and the CPU
oracle consume.

Recipe: ``numpy.random.Generator(PCG64(seed))``; draw
order: key lengths (when random), block permutation, K, ScaleK, Q, ScaleQ, W.
  * int8 q/k: integers in [-128, 127] (both ends included)
  * e4m3fn q/k: uniform(-8, 8) in float32, rounded to float8_e4m3fn (RNE)
  * scales: uniform(0, 10); weights: uniform(0, 0.01); cast with RNE to the
    scale dtype (fp16 with int8, fp32 with fp8)
  * paged key cache: sequence b stores ``aslk[b] // cmp_ratio`` entries in
    ceil(entries / block_size) blocks; blocks are either dealt in order
    ("identity") or from one random permutation of all blocks ("permuted");
    unused block-table slots hold -1.

The five named workloads below are the decode / long-context / prefill shapes
of the method page's examples scaled to serving sizes.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

INT8, FP8 = 0, 1
F16, F32 = 0, 1
BSND, TND = 0, 1
INT64_MAX = (1 << 63) - 1


@dataclasses.dataclass
class Spec:
    name: str
    qk: int                      # INT8 or FP8
    layout: int                  # BSND or TND
    batch: int
    s1: int                      # BSND: S1; TND: T
    aslk: object                 # list of key lengths, or ("uniform", lo, hi)
    block_size: int
    sparse_count: int
    sparse_mode: int
    cmp_ratio: int = 1
    aslq: Optional[Sequence[int]] = None   # BSND per-batch counts or TND prefix sums
    table: str = "permuted"      # "identity" or "permuted"
    stride_pad: int = 0          # extra bytes between key blocks (0 = contiguous)
    spare_blocks: int = 0        # extra unused blocks in the cache
    qk_lo: float = -8.0          # fp8 value range
    qk_hi: float = 8.0
    scale_hi: float = 10.0
    weight_hi: float = 0.01
    pre_tokens: int = INT64_MAX  # window bounds (INT64_MAX: none)
    next_tokens: int = INT64_MAX


WORKLOADS = {
    # c0: single-token decode, the method page's example shape cut to B=1.
    "decode_int8_b1_sk1024": Spec(
        "decode_int8_b1_sk1024", INT8, BSND, 1, 1, [1024], 128, 512, 0, 1, table="identity"),
    # c1: BSND decode, 4 query tokens per sequence (multi-token prediction).
    "decode_int8_b24_s4_sk8192": Spec(
        "decode_int8_b24_s4_sk8192", INT8, BSND, 24, 4, [8192] * 24, 128, 2048, 3, 1),
    # c2: fp8 decode over ragged key lengths.
    "decode_fp8_b64_sk4k_64k": Spec(
        "decode_fp8_b64_sk4k_64k", FP8, BSND, 64, 1, ("uniform", 4096, 65536), 64, 512, 0, 1),
    # c3: long-context decode with 4x compressed keys.
    "longctx_int8_b8_s2_sk131072_cmp4": Spec(
        "longctx_int8_b8_s2_sk131072_cmp4", INT8, BSND, 8, 2, [131072] * 8, 256, 2048, 3, 4),
    # c4: TND prefill, 4 sequences of 2048 tokens.
    "prefill_int8_tnd_4x2048": Spec(
        "prefill_int8_tnd_4x2048", INT8, TND, 4, 8192, [2048] * 4, 128, 2048, 3, 1,
        aslq=[2048, 4096, 6144, 8192]),
}
WORKLOAD_ORDER = list(WORKLOADS)


def _to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    import torch  # conversion only (round-to-nearest-even to float8_e4m3fn)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def make_inputs(spec: Spec, seed: int) -> dict:
    """Draw one problem instance.  Arrays are C-contiguous numpy arrays:
    query [rows, 64, 128] (int8 or e4m3 codes as uint8), key bytes
    [num_blocks * stride], weights / q_scale [rows, 64], k_scale
    [num_blocks, block_size], aslq int32[B] or None, aslk int32[B],
    block_table int32[B, max_blocks]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, bs, cmp = spec.batch, spec.block_size, spec.cmp_ratio
    if isinstance(spec.aslk, tuple):
        _, lo, hi = spec.aslk
        aslk = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        aslk = np.asarray(spec.aslk, dtype=np.int32).reshape(B)
    entries = aslk.astype(np.int64) // cmp
    nblk = (entries + bs - 1) // bs
    max_blocks = int(max(1, nblk.max() if B else 1))
    total = int(nblk.sum()) + spec.spare_blocks
    num_blocks = max(total, 1)
    if spec.table == "identity":
        order = np.arange(num_blocks, dtype=np.int64)
    else:
        order = rng.permutation(num_blocks)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        n = int(nblk[b])
        table[b, :n] = order[pos:pos + n]
        pos += n

    stride = bs * 128 + spec.stride_pad
    nbytes = num_blocks * stride
    if spec.qk == INT8:
        key = rng.integers(-128, 128, size=nbytes, dtype=np.int16).astype(np.int8).view(np.uint8)
    else:
        key = _to_e4m3_codes(rng.uniform(spec.qk_lo, spec.qk_hi, size=nbytes).astype(np.float32))
    sdt = np.float16 if spec.qk == INT8 else np.float32
    k_scale = rng.uniform(0.0, spec.scale_hi, size=(num_blocks, bs)).astype(sdt)

    rows = B * spec.s1 if spec.layout == BSND else spec.s1
    if spec.qk == INT8:
        query = rng.integers(-128, 128, size=(rows, 64, 128), dtype=np.int16).astype(np.int8)
    else:
        query = _to_e4m3_codes(rng.uniform(spec.qk_lo, spec.qk_hi, size=(rows, 64, 128)).astype(np.float32))
    q_scale = rng.uniform(0.0, spec.scale_hi, size=(rows, 64)).astype(sdt)
    weights = rng.uniform(0.0, spec.weight_hi, size=(rows, 64)).astype(sdt)
    aslq = None if spec.aslq is None else np.asarray(spec.aslq, dtype=np.int32).reshape(B)

    problem = dict(
        batch=B, s1=spec.s1, num_heads_q=64, num_heads_k=1, head_dim=128,
        layout_query=spec.layout, qk_dtype=spec.qk, scale_dtype=F16 if spec.qk == INT8 else F32,
        num_blocks=num_blocks, block_size=bs, max_blocks_per_seq=max_blocks,
        key_block_stride=stride if spec.stride_pad else 0,
        sparse_count=spec.sparse_count, sparse_mode=spec.sparse_mode, cmp_ratio=cmp,
        pre_tokens=spec.pre_tokens, next_tokens=spec.next_tokens,
        query_quant_mode=0, key_quant_mode=0, return_value=1)
    return dict(problem=problem, query=np.ascontiguousarray(query), key=np.ascontiguousarray(key),
                weights=np.ascontiguousarray(weights), q_scale=np.ascontiguousarray(q_scale),
                k_scale=np.ascontiguousarray(k_scale), aslq=aslq, aslk=aslk,
                block_table=np.ascontiguousarray(table), spec=spec, seed=seed)


def workload(name: str, seed: Optional[int] = None) -> dict:
    """A named workload; the default seed is its position in WORKLOAD_ORDER."""
    return make_inputs(WORKLOADS[name], WORKLOAD_ORDER.index(name) if seed is None else seed)


def small(name: str = "tiny", **kw) -> Spec:
    """A small spec for tests; keyword arguments override the fields."""
    base = dict(name=name, qk=INT8, layout=BSND, batch=2, s1=2, aslk=[300, 200],
                block_size=64, sparse_count=64, sparse_mode=0, cmp_ratio=1)
    base.update(kw)
    return Spec(**base)


# ---------------------------------------------------------------------------
# Producer workloads: bf16 head vectors before quantization.
# ---------------------------------------------------------------------------
# Recipe: PCG64(seed); each 128-element row is standard normal times a
# per-row factor 2^U(-4, 4) (activation-like spread of row magnitudes), cast
# to bf16 with round-to-nearest-even.  Key appends write every entry of every
# sequence of an indexer workload's paged cache (positions 0 .. entries-1,
# as a prefill writing its context), through that workload's block table.

PRODUCER_WORKLOADS = {
    # the prefill workload's query: 8192 tokens x 64 heads
    "quantize_query_prefill_t8192": dict(kind="query", tokens=8192, qk=INT8),
    # the headline decode workload's whole key cache: 24 sequences x 8192 entries, block 128, permuted
    "append_keys_decode_b24_sk8192": dict(kind="keys", base="decode_int8_b24_s4_sk8192", qk=INT8),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_rows(rng: np.random.Generator, n: int) -> np.ndarray:
    x = rng.standard_normal((n, 128), dtype=np.float32)
    x *= np.exp2(rng.uniform(-4.0, 4.0, (n, 1))).astype(np.float32)
    return to_bf16_bits(x)


def producer_inputs(name: str, seed: Optional[int] = None) -> dict:
    """bf16 rows (uint16 [n, 128]) and, for key appends, the destination of each
    entry (batch_idx, pos) and the cache geometry of the base workload."""
    w = PRODUCER_WORKLOADS[name]
    rng = np.random.default_rng(list(PRODUCER_WORKLOADS).index(name) + 100 if seed is None else seed)
    if w["kind"] == "query":
        return dict(kind="query", qk=w["qk"], x=bf16_rows(rng, w["tokens"] * 64))
    base = workload(w["base"])
    p = base["problem"]
    cmp = p["cmp_ratio"]
    ents = [int(v) // cmp for v in base["aslk"]]
    bidx = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(ents)])
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in ents])
    return dict(kind="keys", qk=w["qk"], x=bf16_rows(rng, bidx.size), batch_idx=bidx, pos=pos,
                block_table=base["block_table"], batch=p["batch"], max_blocks=p["max_blocks_per_seq"],
                num_blocks=p["num_blocks"], block_size=p["block_size"],
                stride=p["key_block_stride"] or p["block_size"] * 128)


# ---------------------------------------------------------------------------
# Consumer inputs: sparse attention over the indexer's selected entries.
# ---------------------------------------------------------------------------
# Recipe: PCG64(seed); query [rows, heads, 128] and the key / value caches
# [num_blocks, block_size, 128] (one head, the indexer workload's block
# geometry and block table) are standard normal cast to bf16 (round to
# nearest even).  Unless given, each row's list holds min(k, n_b) distinct
# entries drawn uniformly from the n_b = aslk[b] // cmp_ratio entries its
# batch's cache stores, in ascending order, padded with -1 (the shape of the
# indexer's sparse_indices).


def attention_inputs(inp: dict, heads: int, seed: int, indices=None, kv_stride_pad: int = 0,
                     scale: Optional[float] = None) -> dict:
    """Consumer inputs over an indexer input dict ``inp`` (its layout, rows,
    lengths, block table and sparse_count): bf16 bit patterns (uint16) for q,
    k_cache and v_cache; indices int32 [rows, k]."""
    p = inp["problem"]
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = p["batch"] * p["s1"] if p["layout_query"] == BSND else p["s1"]
    bs, nb = p["block_size"], p["num_blocks"]
    dim = 128
    stride = bs * dim + kv_stride_pad
    q = to_bf16_bits(rng.standard_normal((rows, heads, dim), dtype=np.float32))
    kc = to_bf16_bits(rng.standard_normal(nb * stride, dtype=np.float32))
    vc = to_bf16_bits(rng.standard_normal(nb * stride, dtype=np.float32))
    k = p["sparse_count"]
    if indices is None:
        ents = inp["aslk"].astype(np.int64) // p["cmp_ratio"]
        indices = np.full((rows, k), -1, dtype=np.int32)
        if p["layout_query"] == BSND:
            batch_of = np.repeat(np.arange(p["batch"]), p["s1"])
        else:
            ends = np.asarray(inp["aslq"], dtype=np.int64)
            batch_of = np.searchsorted(ends, np.arange(rows), side="right")
        for r in range(rows):
            b = int(batch_of[r])
            if b >= p["batch"]:
                continue
            n = int(min(k, ents[b]))
            indices[r, :n] = np.sort(rng.choice(int(ents[b]), size=n, replace=False))
    return dict(layout=p["layout_query"], batch=p["batch"], s1=p["s1"], aslq=inp["aslq"], heads=heads,
                block_size=bs, max_blocks=p["max_blocks_per_seq"], num_blocks=nb,
                kv_stride=stride if kv_stride_pad else 0, q=q, k_cache=kc, v_cache=vc,
                block_table=inp["block_table"], indices=np.ascontiguousarray(indices, dtype=np.int32),
                scale=(1.0 / np.sqrt(dim)) if scale is None else scale)
