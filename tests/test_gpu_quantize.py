"""GPU parity of the producer kernels (qli_quantize_query, qli_append_keys)
through the C ABI against the CPU oracle (oracle/quantize.py): codes and
scales bit-exact (integer decisions taken in fp32 on both sides), every byte
of the paged cache equal, and the quantized inputs feeding the indexer."""
import numpy as np
import pytest

import synth
from oracle import quantize as oq
from tests._gpu import check_row, check_structure, log, rtol_of
from tests._helpers import rows_of

pytestmark = pytest.mark.gpu

DT = {0: "int8", 1: "e4m3fn"}


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import sparse_attention_token_paged_amd as qli
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qli.load()


def bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def query_rows(seed: int, n: int) -> np.ndarray:
    """bf16 rows over a wide exponent range plus the special cases of the
    quantizer's definition."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32) * np.exp2(rng.uniform(-40, 40, (n, 1))).astype(np.float32)
    x[0] = 0.0                                  # zero row: scale 0, codes 0
    x[1] = 0.0
    x[1, 77] = -5.5                             # single spike: the extreme code
    x[2] = 3.25                                 # constant row
    x[3] = 3.0e38                               # int8 scale overflows fp16: capped at 65504
    x[3, 64:] = -3.0e38
    x[4] = rng.standard_normal(128) * 1e-39     # bf16 subnormals: int8 scale 0, fp8 1/s not finite
    x[5] = rng.standard_normal(128) * 1e-36     # fp8 scale subnormal in fp32
    x[6] = np.round(rng.standard_normal(128) * 40) / 4  # many exact .5 multiples of the step
    return bf16_bits(x)


@pytest.mark.parametrize("qk", [0, 1], ids=["int8", "e4m3fn"])
def test_quantize_query_bit_exact(qk):
    import torch
    import sparse_attention_token_paged_amd as qli
    n = 4099  # not a multiple of 4 rows per wave nor of the grid: the masked tail runs
    xb = query_rows(21 + qk, n)
    log("quantize_query %s rows=%d" % (DT[qk], n))
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    q = torch.full((n, 128), 0x5A, dtype=torch.uint8, device="cuda")
    sdt = torch.float16 if qk == 0 else torch.float32
    s = torch.full((n,), 123.0, dtype=sdt, device="cuda")
    rc = qli.qli_quantize_query(qk, n, x, q, s, qli.current_stream())
    assert rc == qli.QLI_OK
    torch.cuda.synchronize()
    codes, scales = oq.quantize_rows(xb, qk)
    gq, gs = q.cpu().numpy(), s.cpu().numpy()
    bad = np.nonzero(np.any(gq != codes, axis=1))[0]
    assert bad.size == 0, "rows %r: codes differ (first %r vs %r)" % (bad[:5], gq[bad[0]][:8], codes[bad[0]][:8])
    sv = gs.view(np.uint16 if qk == 0 else np.uint32)
    ov = scales.view(np.uint16 if qk == 0 else np.uint32)
    assert np.array_equal(sv, ov), "scales differ at rows %r" % np.nonzero(sv != ov)[0][:5]


@pytest.mark.parametrize("qk,bs,pad", [(0, 16, 0), (0, 128, 48), (1, 64, 16), (1, 256, 0)],
                         ids=["int8_bs16", "int8_bs128_pad", "fp8_bs64_pad", "fp8_bs256"])
def test_append_keys_bit_exact(qk, bs, pad):
    import torch
    import sparse_attention_token_paged_amd as qli
    rng = np.random.default_rng(31 + bs)
    B, mb = 3, 5
    nb = B * mb + 2                      # two physical blocks no sequence owns
    stride = bs * 128 + pad
    table = rng.permutation(nb)[:B * mb].astype(np.int32).reshape(B, mb)
    table[2, 4] = -1                     # an unused table entry
    slots = rng.permutation(B * mb * bs)[:min(600, B * mb * bs - bs)]
    bidx = (slots // (mb * bs)).astype(np.int32)
    pos = (slots % (mb * bs)).astype(np.int32)
    # entries outside the cache are skipped
    bidx = np.concatenate([bidx, [-1, B, 0, 0, 2]]).astype(np.int32)
    pos = np.concatenate([pos, [0, 1, -3, mb * bs, 4 * bs + 1]]).astype(np.int32)
    n = bidx.size
    xb = query_rows(41 + bs, n)
    log("append_keys %s n=%d block_size=%d stride=%d" % (DT[qk], n, bs, stride))
    sdt_np = np.float16 if qk == 0 else np.float32
    kc0 = np.full(nb * stride, 0xA5, np.uint8)
    ks0 = np.full(nb * bs, 7.0, sdt_np)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc, ks = dev(kc0), dev(ks0)
    rc = qli.qli_append_keys(qk, n, dev(xb.view(np.int16)), dev(bidx), dev(pos), dev(table), B, mb, nb, bs,
                             stride, kc, ks, qli.current_stream())
    assert rc == qli.QLI_OK
    torch.cuda.synchronize()
    oq.append_keys(xb, bidx, pos, table, B, mb, nb, bs, stride, kc0, ks0, qk)
    gk = kc.cpu().numpy()
    bad = np.nonzero(gk != kc0)[0]
    assert bad.size == 0, "cache bytes differ from offset %d (%d bytes)" % (bad[0], bad.size)
    gs = ks.cpu().numpy()
    assert np.array_equal(gs.view(np.uint16 if qk == 0 else np.uint32), ks0.view(np.uint16 if qk == 0 else np.uint32))


@pytest.mark.parametrize("qk", [0, 1], ids=["int8", "e4m3fn"])
def test_quantized_inputs_feed_the_indexer(ora, qk):
    """bf16 query and key -> producer kernels -> indexer, against the oracle's
    quantizer and indexer on the same bf16 inputs."""
    import torch
    import sparse_attention_token_paged_amd as qli
    spec = synth.small(qk=synth.FP8 if qk else synth.INT8, batch=2, s1=2, aslk=[700, 300], block_size=64,
                       sparse_count=128, sparse_mode=3)
    inp = synth.make_inputs(spec, 5)
    p = inp["problem"]
    rows = rows_of(p)
    rng = np.random.default_rng(51)
    qb = bf16_bits(rng.standard_normal((rows * 64, 128)).astype(np.float32) * 0.5)
    # key entries 0..aslk[b]-1 of every sequence, in the cache the workload's block table describes
    bidx = np.concatenate([np.full(n, b, np.int32) for b, n in enumerate(inp["aslk"])])
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in inp["aslk"]])
    kb = bf16_bits(rng.standard_normal((bidx.size, 128)).astype(np.float32))
    bs, mb, nb = p["block_size"], p["max_blocks_per_seq"], p["num_blocks"]
    stride = p["key_block_stride"] or bs * 128
    # oracle side
    qc, qs = oq.quantize_rows(qb, qk)
    inp["query"] = qc.reshape(rows, 64, 128).view(inp["query"].dtype)
    inp["q_scale"] = qs.reshape(rows, 64)
    kc = np.zeros_like(inp["key"])
    ks = np.zeros_like(inp["k_scale"]).reshape(-1)
    oq.append_keys(kb, bidx, pos, inp["block_table"], p["batch"], mb, nb, bs, stride, kc.view(np.uint8), ks, qk)
    inp["key"], inp["k_scale"] = kc, ks.reshape(inp["k_scale"].shape)
    # GPU side: the producer kernels write the indexer's inputs
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    gq = torch.empty((rows * 64, 128), dtype=torch.uint8, device="cuda")
    gqs = torch.empty((rows * 64,), dtype=torch.float16 if qk == 0 else torch.float32, device="cuda")
    assert qli.qli_quantize_query(qk, rows * 64, dev(qb.view(np.int16)), gq, gqs, qli.current_stream()) == 0
    gk = torch.zeros(inp["key"].size, dtype=torch.uint8, device="cuda")
    gks = torch.zeros(ks.size, dtype=gqs.dtype, device="cuda")
    bt = dev(inp["block_table"])
    assert qli.qli_append_keys(qk, bidx.size, dev(kb.view(np.int16)), dev(bidx), dev(pos), bt, p["batch"], mb, nb,
                               bs, stride, gk, gks, qli.current_stream()) == 0
    ix = qli.Indexer(p, inp["aslq"], inp["aslk"])
    idx, val = ix.run(gq, gk, dev(inp["weights"]), gqs, gks, bt)
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), qc) and np.array_equal(gk.cpu().numpy(), kc.view(np.uint8).reshape(-1))
    vis = ora.row_visible(p["layout_query"], p["batch"], p["s1"], p["sparse_mode"], p["cmp_ratio"],
                          inp["aslq"], inp["aslk"])
    rc, _, _, sc = ora.indexer(inp, scores_cols=int(vis.max()))
    assert rc == 0
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    check_structure(idx, val, vis, p["sparse_count"])
    for r in range(rows):
        check_row(r, int(vis[r]), p["sparse_count"], idx[r], val[r], sc[r, :vis[r]], rtol_of(inp))


def test_chain_graph_replay(ora):
    """One decode step as a HIP graph captured once: quantize the bf16 query,
    append each sequence's newest bf16 key entries into the paged cache, run
    the indexer with the key lengths read on the device (no host plan).
    Replayed with new inputs, positions and lengths (written eagerly between
    replays, from a restored cache each time), every replay equals the same
    chain run eagerly, bit for bit, and the oracle's chain (its quantizer,
    its cache append and its indexer on the same bf16 inputs) on every row."""
    import torch
    import sparse_attention_token_paged_amd as qli
    # every sequence's block table covers the bound, so any drawn length reads only real blocks
    spec = synth.small(batch=3, s1=2, aslk=[1500] * 3, block_size=64, sparse_count=128, sparse_mode=3)
    inp = synth.make_inputs(spec, 9)
    p = inp["problem"]
    B, S1, bs, mb, nb = p["batch"], p["s1"], p["block_size"], p["max_blocks_per_seq"], p["num_blocks"]
    stride = p["key_block_stride"] or bs * 128
    rows, new = B * S1, 16
    bound = 1500
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    st = qli.current_stream
    # static buffers of the captured step
    qb, kb = torch.empty((rows * 64, 128), dtype=torch.int16, device="cuda"), \
        torch.empty((B * new, 128), dtype=torch.int16, device="cuda")
    bidx = dev(np.repeat(np.arange(B, dtype=np.int32), new))
    pos = torch.empty((B * new,), dtype=torch.int32, device="cuda")
    aslk = torch.empty((B,), dtype=torch.int32, device="cuda")
    q, qs = torch.empty((rows * 64, 128), dtype=torch.uint8, device="cuda"), \
        torch.empty((rows * 64,), dtype=torch.float16, device="cuda")
    pristine_k, pristine_ks = dev(inp["key"]), dev(inp["k_scale"].reshape(-1))
    key, ks = pristine_k.clone(), pristine_ks.clone()
    w, bt = dev(inp["weights"]), dev(inp["block_table"])
    bix = qli.BoundedIndexer(p, bound)
    idx, val = bix.alloc_outputs()

    def step():
        assert qli.qli_quantize_query(0, rows * 64, qb, q, qs, st()) == qli.QLI_OK
        assert qli.qli_append_keys(0, B * new, kb, bidx, pos, bt, B, mb, nb, bs, stride, key, ks, st()) == qli.QLI_OK
        bix.run(aslk, q, key, w, qs, ks, bt, idx, val)

    def load_inputs(seed):
        rng = np.random.default_rng(seed)
        lens = rng.integers(200, bound + 1, B).astype(np.int32)
        qh = bf16_bits(rng.standard_normal((rows * 64, 128)).astype(np.float32))
        kh = bf16_bits(rng.standard_normal((B * new, 128)).astype(np.float32))
        ph = np.concatenate([np.arange(n - new, n, dtype=np.int32) for n in lens])
        qb.copy_(dev(qh.view(np.int16)))
        kb.copy_(dev(kh.view(np.int16)))
        pos.copy_(dev(ph))
        aslk.copy_(dev(lens))
        key.copy_(pristine_k)
        ks.copy_(pristine_ks)
        return qh, kh, ph, lens

    def oracle_chain(qh, kh, ph, lens):
        """The same step on the CPU: oracle quantizer, oracle append, oracle indexer."""
        qc, qsc = oq.quantize_rows(qh, 0)
        kc = inp["key"].copy()
        ksc = inp["k_scale"].reshape(-1).copy()
        oq.append_keys(kh, np.repeat(np.arange(B, dtype=np.int32), new), ph, inp["block_table"], B, mb, nb, bs,
                       stride, kc.view(np.uint8), ksc, 0)
        sub = dict(inp, query=qc.reshape(rows, 64, 128).view(inp["query"].dtype), q_scale=qsc.reshape(rows, 64),
                   key=kc, k_scale=ksc.reshape(inp["k_scale"].shape), aslk=lens)
        vis = ora.row_visible(p["layout_query"], B, S1, p["sparse_mode"], p["cmp_ratio"], None, lens)
        rc, _, _, sc = ora.indexer(sub, scores_cols=int(vis.max()))
        assert rc == 0
        return sub, vis, sc

    load_inputs(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # first launches (occupancy queries) outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        log("chain graph replay %d" % rep)
        host = load_inputs(100 + rep)
        idx.fill_(-7)
        val.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        g_idx, g_val, g_key = idx.cpu().numpy(), val.cpu().numpy(), key.cpu().numpy()
        load_inputs(100 + rep)
        step()
        torch.cuda.synchronize()
        assert np.array_equal(g_key, key.cpu().numpy()), "replay %d: cache differs" % rep
        assert np.array_equal(g_idx, idx.cpu().numpy()), "replay %d: indices differ" % rep
        assert np.array_equal(g_val, val.cpu().numpy()), "replay %d: values differ" % rep
        assert (g_idx[:, 0] >= 0).all()
        sub, vis, sc = oracle_chain(*host)
        check_structure(g_idx, g_val, vis, p["sparse_count"])
        for r in range(rows):
            check_row(r, int(vis[r]), p["sparse_count"], g_idx[r], g_val[r], sc[r, :vis[r]], rtol_of(sub))


@pytest.mark.parametrize("name", ["quantize_query_prefill_t8192", "append_keys_decode_b24_sk8192"])
def test_producer_full_size(name):
    """The producer workloads at the benchmark's sizes (524288 query head
    vectors; the headline decode cache's 196608 key entries through its
    permuted block table), every row against the oracle, bit-exact."""
    import torch
    import sparse_attention_token_paged_amd as qli
    w = synth.producer_inputs(name)
    qk, x = w["qk"], w["x"]
    n = x.shape[0]
    log("producer full size %s: %d rows" % (name, n))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sdt = torch.float16 if qk == 0 else torch.float32
    if w["kind"] == "query":
        q = torch.full((n, 128), 0x5A, dtype=torch.uint8, device="cuda")
        s = torch.zeros((n,), dtype=sdt, device="cuda")
        assert qli.qli_quantize_query(qk, n, dev(x.view(np.int16)), q, s, qli.current_stream()) == qli.QLI_OK
        torch.cuda.synchronize()
        codes, scales = oq.quantize_rows(x, qk)
        assert np.array_equal(q.cpu().numpy(), codes)
        assert np.array_equal(s.cpu().numpy().view(np.uint16), scales.view(np.uint16))
    else:
        bs, nb, stride = w["block_size"], w["num_blocks"], w["stride"]
        kc0 = np.full(nb * stride, 0xA5, np.uint8)
        ks0 = np.full(nb * bs, 7.0, np.float16 if qk == 0 else np.float32)
        kc, ks = dev(kc0), dev(ks0)
        assert qli.qli_append_keys(qk, n, dev(x.view(np.int16)), dev(w["batch_idx"]), dev(w["pos"]),
                                   dev(w["block_table"]), w["batch"], w["max_blocks"], nb, bs, stride, kc, ks,
                                   qli.current_stream()) == qli.QLI_OK
        torch.cuda.synchronize()
        oq.append_keys(x, w["batch_idx"], w["pos"], w["block_table"], w["batch"], w["max_blocks"], nb, bs, stride,
                       kc0, ks0, qk)
        assert np.array_equal(kc.cpu().numpy(), kc0)
        assert np.array_equal(ks.cpu().numpy(), ks0)


@pytest.mark.parametrize("qk,n", [(0, 1), (1, 3), (0, 5)])
def test_quantize_query_tiny(qk, n):
    """1, 3 and 5 rows: a partial 4-row group (and one group plus a partial)."""
    import torch
    import sparse_attention_token_paged_amd as qli
    xb = query_rows(61 + n, max(n, 7))[:n]
    q = torch.full((n, 128), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.zeros((n,), dtype=torch.float16 if qk == 0 else torch.float32, device="cuda")
    assert qli.qli_quantize_query(qk, n, torch.from_numpy(xb.view(np.int16)).cuda(), q, s,
                                  qli.current_stream()) == qli.QLI_OK
    torch.cuda.synchronize()
    codes, scales = oq.quantize_rows(xb, qk)
    assert np.array_equal(q.cpu().numpy(), codes)
    dt = np.uint16 if qk == 0 else np.uint32
    assert np.array_equal(s.cpu().numpy().view(dt), scales.view(dt))


@pytest.mark.parametrize("qk", [0, 1], ids=["int8", "e4m3fn"])
def test_append_keys_block_1024(qk):
    """The largest block size (1024 entries per block, 128 KiB blocks) with a padded stride."""
    import torch
    import sparse_attention_token_paged_amd as qli
    rng = np.random.default_rng(71)
    B, mb, bs = 2, 3, 1024
    nb, stride = B * mb + 1, bs * 128 + 32
    table = rng.permutation(nb)[:B * mb].astype(np.int32).reshape(B, mb)
    slots = rng.permutation(B * mb * bs)[:3000]
    bidx, pos = (slots // (mb * bs)).astype(np.int32), (slots % (mb * bs)).astype(np.int32)
    xb = query_rows(72, bidx.size)
    kc0 = np.full(nb * stride, 0xA5, np.uint8)
    ks0 = np.full(nb * bs, 7.0, np.float16 if qk == 0 else np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc, ks = dev(kc0), dev(ks0)
    assert qli.qli_append_keys(qk, bidx.size, dev(xb.view(np.int16)), dev(bidx), dev(pos), dev(table), B, mb, nb,
                               bs, stride, kc, ks, qli.current_stream()) == qli.QLI_OK
    torch.cuda.synchronize()
    oq.append_keys(xb, bidx, pos, table, B, mb, nb, bs, stride, kc0, ks0, qk)
    assert np.array_equal(kc.cpu().numpy(), kc0)
    dt = np.uint16 if qk == 0 else np.uint32
    assert np.array_equal(ks.cpu().numpy().view(dt), ks0.view(dt))


@pytest.mark.parametrize("i", range(10))
def test_producer_random(i):
    """Seeded random producer problems: dtype, query row count, cache geometry
    (block size, padded stride, sequences, table width, spare blocks), a random
    subset of distinct slots plus entries outside the cache; query codes and
    the whole cache bit-exact against the oracle."""
    import torch
    import sparse_attention_token_paged_amd as qli
    rng = np.random.default_rng(9000 + i)
    qk = int(rng.integers(0, 2))
    dt = np.uint16 if qk == 0 else np.uint32
    sdt = torch.float16 if qk == 0 else torch.float32
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    # query
    n = int(rng.integers(1, 3000))
    xb = query_rows(9100 + i, max(n, 7))[:n]
    q = torch.full((n, 128), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.zeros((n,), dtype=sdt, device="cuda")
    assert qli.qli_quantize_query(qk, n, dev(xb.view(np.int16)), q, s, qli.current_stream()) == qli.QLI_OK
    # key cache
    bs = int(rng.choice([16, 32, 48, 64, 128, 256, 512]))
    B, mb = int(rng.integers(1, 5)), int(rng.integers(1, 6))
    nb = B * mb + int(rng.integers(0, 3))
    stride = bs * 128 + 16 * int(rng.integers(0, 4))
    table = rng.permutation(nb)[:B * mb].astype(np.int32).reshape(B, mb)
    m = int(rng.integers(1, B * mb * bs + 1))
    slots = rng.permutation(B * mb * bs)[:m]
    bidx = np.concatenate([slots // (mb * bs), rng.integers(-2, B + 2, 4)]).astype(np.int32)
    pos = np.concatenate([slots % (mb * bs), rng.integers(-3, mb * bs + 3, 4)]).astype(np.int32)
    # the random extra entries must not collide with a chosen slot: move colliding ones out of range
    taken = set(zip((slots // (mb * bs)).tolist(), (slots % (mb * bs)).tolist()))
    for e in range(m, bidx.size):
        if (int(bidx[e]), int(pos[e])) in taken:
            pos[e] = -1
    kb = query_rows(9200 + i, max(bidx.size, 7))[:bidx.size]
    log("producer random %d: qk %d n %d bs %d B %d mb %d entries %d" % (i, qk, n, bs, B, mb, bidx.size))
    kc0 = np.full(nb * stride, 0xA5, np.uint8)
    ks0 = np.full(nb * bs, 7.0, np.float16 if qk == 0 else np.float32)
    kc, ks = dev(kc0), dev(ks0)
    assert qli.qli_append_keys(qk, bidx.size, dev(kb.view(np.int16)), dev(bidx), dev(pos), dev(table), B, mb, nb,
                               bs, stride, kc, ks, qli.current_stream()) == qli.QLI_OK
    torch.cuda.synchronize()
    codes, scales = oq.quantize_rows(xb, qk)
    assert np.array_equal(q.cpu().numpy(), codes)
    assert np.array_equal(s.cpu().numpy().view(dt), scales.view(dt))
    oq.append_keys(kb, bidx, pos, table, B, mb, nb, bs, stride, kc0, ks0, qk)
    assert np.array_equal(kc.cpu().numpy(), kc0)
    assert np.array_equal(ks.cpu().numpy().view(dt), ks0.view(dt))
