"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small cases are compared on every row and span several 64-key tiles, ragged
tails, block sizes that are not powers of two, padded block strides, causal
and compressed visibility, rows below and above sparse_count, TND and BSND.
The five full-size workloads run in the benchmark's launch configuration,
every row against the oracle; int8 dots of sampled full-size rows bit-exact.
Runs without a host plan (bounded) and graph replays are checked against
the oracle on every row as well as against the planned run.
"""
import numpy as np
import pytest

import synth
from tests._gpu import (ATOL, INT8_RTOL, check_row, check_structure, device_inputs, log, make_indexer, rtol_of,
                        run_gpu, stable_topk_set)
from tests._helpers import rows_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import sparse_attention_token_paged_amd as qli
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qli.load()  # fails loudly if the HIP library is missing


def vis_of(ora, inp):
    p = inp["problem"]
    return ora.row_visible(p["layout_query"], p["batch"], p["s1"], p["sparse_mode"], p["cmp_ratio"],
                           inp["aslq"], inp["aslk"])


SMALL = {
    "bsnd_int8_causal_bs48_pad": synth.small(batch=3, s1=4, aslk=[700, 389, 1500], block_size=48,
                                             sparse_count=256, sparse_mode=3, stride_pad=32),
    "bsnd_int8_mode0_identity": synth.small(batch=2, s1=1, aslk=[1000, 64 + 13], block_size=128,
                                            sparse_count=512, table="identity"),
    "bsnd_int8_cmp4_bs16": synth.small(batch=2, s1=2, aslk=[4099, 777], block_size=16, sparse_count=128,
                                       sparse_mode=3, cmp_ratio=4),
    "bsnd_int8_unused_rows": synth.small(batch=3, s1=3, aslk=[150, 40, 0], aslq=[3, 2, 3], block_size=32,
                                         sparse_count=64, sparse_mode=3, cmp_ratio=2),
    "bsnd_int8_k1": synth.small(batch=2, s1=3, aslk=[333, 97], block_size=32, sparse_count=1, sparse_mode=3),
    "bsnd_int8_k2048": synth.small(batch=1, s1=2, aslk=[5000], block_size=256, sparse_count=2048,
                                   sparse_mode=3),
    "bsnd_int8_vis_equals_k": synth.small(batch=1, s1=1, aslk=[640], block_size=64, sparse_count=640),
    "bsnd_int8_s1_3": synth.small(batch=2, s1=3, aslk=[900, 2100], block_size=64, sparse_count=300,
                                  sparse_mode=3),
    "tnd_int8_prefill_mixed": synth.small(layout=synth.TND, batch=3, s1=210, aslq=[70, 140, 200],
                                          aslk=[70, 100, 300], block_size=32, sparse_count=64, sparse_mode=3),
    "tnd_int8_prefill_long": synth.small(layout=synth.TND, batch=1, s1=40, aslq=[40], aslk=[6000],
                                         block_size=128, sparse_count=100, sparse_mode=3),
    "bsnd_fp8_mode0": synth.small(qk=synth.FP8, batch=4, s1=1, aslk=[3000, 200, 1777, 64], block_size=64,
                                  sparse_count=300),
    "bsnd_fp8_causal_s2": synth.small(qk=synth.FP8, batch=2, s1=2, aslk=[2500, 900], block_size=32,
                                      sparse_count=128, sparse_mode=3, stride_pad=16),
    "tnd_fp8_prefill": synth.small(qk=synth.FP8, layout=synth.TND, batch=2, s1=50, aslq=[20, 50],
                                   aslk=[400, 30], block_size=16, sparse_count=32, sparse_mode=3),
    # every batch alike: items addressed from their position
    "regular_causal_s3": synth.small(batch=5, s1=3, aslk=[3000] * 5, block_size=64, sparse_count=256, sparse_mode=3),
    "regular_s1_fp8": synth.small(qk=synth.FP8, batch=4, s1=1, aslk=[900] * 4, block_size=16, sparse_count=300),
    # the remaining compression ratios and the largest block sizes (参数说明 cmp_ratio, 约束说明 block_size)
    "bsnd_int8_cmp8_causal": synth.small(batch=2, s1=3, aslk=[9000, 3001], block_size=64, sparse_count=256,
                                         sparse_mode=3, cmp_ratio=8),
    "bsnd_int8_cmp16_mode0": synth.small(batch=3, s1=2, aslk=[20000, 7777, 15], block_size=32, sparse_count=200,
                                         cmp_ratio=16),
    "tnd_int8_cmp32_causal": synth.small(layout=synth.TND, batch=2, s1=10, aslq=[3, 10], aslk=[40000, 9000],
                                         block_size=128, sparse_count=300, sparse_mode=3, cmp_ratio=32),
    "bsnd_fp8_cmp64_causal": synth.small(qk=synth.FP8, batch=2, s1=2, aslk=[70000, 20000], block_size=64,
                                         sparse_count=128, sparse_mode=3, cmp_ratio=64),
    "bsnd_int8_cmp128_bs16": synth.small(batch=2, s1=1, aslk=[130000, 1000], block_size=16, sparse_count=100,
                                         cmp_ratio=128),
    "bsnd_int8_bs1024": synth.small(batch=2, s1=2, aslk=[5000, 2100], block_size=1024, sparse_count=512,
                                    sparse_mode=3),
    "bsnd_fp8_bs512_pad": synth.small(qk=synth.FP8, batch=2, s1=1, aslk=[3000, 1500], block_size=512,
                                      sparse_count=700, stride_pad=64),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_parity_small(ora, name):
    inp = synth.make_inputs(SMALL[name], 7)
    p = inp["problem"]
    log("case %s: rows=%d k=%d" % (name, rows_of(p), p["sparse_count"]))
    vis = vis_of(ora, inp)
    cols = max(1, int(vis.max()) if vis.size else 1)
    rc, oidx, oval, osc = ora.indexer(inp, scores_cols=cols)
    assert rc == 0
    gidx, gval, _ = run_gpu(inp)
    k = p["sparse_count"]
    check_structure(gidx, gval, vis, k)
    for r in range(rows_of(p)):
        check_row(r, int(vis[r]), k, gidx[r], gval[r], osc[r, :vis[r]], rtol_of(inp))


@pytest.mark.parametrize("name", ["bsnd_int8_causal_bs48_pad", "bsnd_int8_cmp4_bs16", "tnd_int8_prefill_mixed",
                                  "bsnd_fp8_causal_s2", "bsnd_int8_cmp8_causal", "bsnd_int8_bs1024"])
def test_debug_dump(ora, name):
    """Dots straight from the matrix cores (int8: bit-exact), scores within
    tolerance, and the selection equal to the stable top-k of the GPU's own
    fp32 scores (exact: integer/index work)."""
    import torch
    inp = synth.make_inputs(SMALL[name], 11)
    p = inp["problem"]
    vis = vis_of(ora, inp)
    rows, k = rows_of(p), p["sparse_count"]
    cols = int(vis.max())
    log("case %s: debug dump rows=%d cols=%d" % (name, rows, cols))
    ix = make_indexer(inp)
    dev = device_inputs(inp)
    gidx, gval, dots, scores = ix.run_debug(dev["query"], dev["key"], dev["weights"], dev["q_scale"],
                                            dev["k_scale"], dev["block_table"], 0, rows, cols)
    torch.cuda.synchronize()
    gidx, gval = gidx.cpu().numpy(), gval.cpu().numpy()
    dots, scores = dots.cpu().numpy(), scores.cpu().numpy()
    fp8 = p["qk_dtype"] == 1
    for r in range(rows):
        v = int(vis[r])
        if v == 0:
            continue
        _, odots, osc = ora.row_detail(inp, r, 0, v)
        if fp8:
            # the f8f6f4 MFMA accumulates in fp32 with its own order
            assert np.all(np.abs(dots[r, :, :v] - odots) <= 1e-3 * (np.abs(odots) + 64.0))
        else:
            assert np.array_equal(dots[r, :, :v].astype(np.float64), odots), "row %d: int8 dots differ" % r
        ref = osc
        assert np.all(np.abs(scores[r, :v] - ref) <= ATOL + rtol_of(inp) * np.abs(ref)), "row %d scores" % r
        n = min(k, v)
        assert np.array_equal(gidx[r, :n], stable_topk_set(scores[r, :v], k)), "row %d selection" % r
        assert np.array_equal(gval[r, :n], scores[r, gidx[r, :n]]), "row %d values" % r


LONG = {
    # rows longer than one selection segment: segment top-k, then a merge
    "long_rt1_ragged": synth.small(batch=16, s1=1, aslk=[70000 - 977 * i for i in range(16)], block_size=64,
                                    sparse_count=256),
    "long_rt2_causal": synth.small(batch=8, s1=2, aslk=[70000] * 8, block_size=32, sparse_count=256,
                                    sparse_mode=3),
    "long_rt1_fp8": synth.small(qk=synth.FP8, batch=12, s1=1, aslk=[60000 + 1111 * i for i in range(12)],
                                 block_size=64, sparse_count=200),
    # merges of 5, 13 and 18 segments' winners (k = 2048): 10240, 26624 and 36864 candidates,
    # i.e. the 4- and 8-group register selections and the re-reading one
    "long_merge_r4": synth.small(batch=2, s1=1, aslk=[40000, 38500], block_size=64, sparse_count=2048),
    "long_merge_r8": synth.small(batch=1, s1=1, aslk=[100000], block_size=128, sparse_count=2048),
    "long_merge_global": synth.small(batch=1, s1=1, aslk=[140000], block_size=128, sparse_count=2048)
}


@pytest.mark.parametrize("name", list(LONG))
def test_parity_long_rows(ora, name):
    """Rows longer than one selection segment: structure on every row, oracle on
    sampled rows, and the GPU's own dumped scores select exactly the returned set."""
    import torch
    inp = synth.make_inputs(LONG[name], 13)
    p = inp["problem"]
    rows, k = rows_of(p), p["sparse_count"]
    vis = vis_of(ora, inp)
    ix = make_indexer(inp)
    assert int(vis.max()) > 8192  # rows selected in two passes (segments, then a merge)
    log("case %s: rows=%d k=%d chunk=%d" % (name, rows, k, ix.info.keys_per_chunk))
    dev = device_inputs(inp)
    dump_rows = min(2, rows)
    cols = int(vis[:dump_rows].max())
    gidx, gval, dots, scores = ix.run_debug(dev["query"], dev["key"], dev["weights"], dev["q_scale"],
                                            dev["k_scale"], dev["block_table"], 0, dump_rows, cols)
    torch.cuda.synchronize()
    gidx, gval, scores = gidx.cpu().numpy(), gval.cpu().numpy(), scores.cpu().numpy()
    check_structure(gidx, gval, vis, k)
    for r in range(dump_rows):
        v = int(vis[r])
        assert np.array_equal(gidx[r, :k], stable_topk_set(scores[r, :v], k)), "row %d selection" % r
        assert np.array_equal(gval[r, :k], scores[r, gidx[r, :k]]), "row %d values" % r
    for r in sorted({0, rows // 2, rows - 1}):
        v = int(vis[r])
        log("  oracle row %d vis %d" % (r, v))
        _, _, osc = ora.row_detail(inp, r, 0, v)
        check_row(r, v, k, gidx[r], gval[r], osc, rtol_of(inp))


LONG_DENSE = {
    # every score staged: rows of 8193..40000 candidates (segment selections, then merges)
    "dense_rows_20k": synth.small(batch=2, s1=3, aslk=[20000, 9000], block_size=64, sparse_count=1500,
                                  sparse_mode=3),
    "dense_rows_40k": synth.small(batch=1, s1=3, aslk=[40000], block_size=128, sparse_count=300, sparse_mode=3),
}


@pytest.mark.parametrize("name", list(LONG_DENSE))
def test_parity_long_dense_rows(ora, name):
    inp = synth.make_inputs(LONG_DENSE[name], 17)
    p = inp["problem"]
    rows, k = rows_of(p), p["sparse_count"]
    vis = vis_of(ora, inp)
    ix = make_indexer(inp)
    log("case %s: rows=%d k=%d max vis=%d" % (name, rows, k, int(vis.max())))
    gidx, gval, _ = run_gpu(inp, ix=ix)
    check_structure(gidx, gval, vis, k)
    rc, _, _, osc = ora.indexer(inp, scores_cols=int(vis.max()))
    assert rc == 0
    for r in range(rows):
        check_row(r, int(vis[r]), k, gidx[r], gval[r], osc[r, :vis[r]], rtol_of(inp))



def test_parity_maximum_key_length(ora):
    """One row at the longest key length the plan accepts, 2^22 - 1 entries
    (512 MiB of int8 keys in blocks of 1024): 1024 decode items of 4096
    entries, 512 first-pass segment selections and one merge of 1,048,576
    candidates in the re-reading selection kernel, against the oracle; the
    bounded run (device length) gives the same bits."""
    import torch
    n = (1 << 22) - 1
    inp = synth.make_inputs(synth.small(batch=1, s1=1, aslk=[n], block_size=1024, sparse_count=2048), 23)
    vis = vis_of(ora, inp)
    assert int(vis[0]) == n
    log("case max key length: %d entries" % n)
    dev = device_inputs(inp)
    gidx, gval, _ = run_gpu(inp, dev)
    check_structure(gidx, gval, vis, 2048)
    bix = qli_mod().BoundedIndexer(inp["problem"], n)
    idx, val = bix.alloc_outputs()
    bix.run(torch.tensor([n], dtype=torch.int32, device="cuda"), dev["query"], dev["key"], dev["weights"],
            dev["q_scale"], dev["k_scale"], dev["block_table"], idx, val)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), gidx) and np.array_equal(val.cpu().numpy(), gval)
    log("  oracle over %d entries" % n)
    rc, _, _, osc = ora.indexer(inp, scores_cols=n)
    assert rc == 0
    check_row(0, n, 2048, gidx[0], gval[0], osc[0], rtol_of(inp))

def _extreme_fp16(rng, shape):
    """fp16 values over the whole non-negative range: zeros, the smallest
    subnormal and normal, the largest finite value, and log-uniform values
    between 2^-24 and 65504."""
    special = np.array([0.0, 2.0 ** -24, 2.0 ** -14, 0.5, 1.0, 65504.0])
    v = np.exp2(rng.uniform(-24.0, 15.99, size=shape))
    pick = rng.random(shape) < 0.3
    v[pick] = rng.choice(special, size=int(pick.sum()))
    return v.astype(np.float16)


EXTREME = {
    "decode_bsnd_causal": synth.small(batch=3, s1=4, aslk=[1500, 700, 2300], block_size=64, sparse_count=256,
                                      sparse_mode=3),
    "prefill_tnd_causal": synth.small(layout=synth.TND, batch=2, s1=150, aslq=[70, 150], aslk=[300, 900],
                                      block_size=32, sparse_count=128, sparse_mode=3),
}


@pytest.mark.parametrize("name", list(EXTREME))
def test_extreme_fp16_scales(ora, name):
    """int8 path with weights and both dequant scales spanning every fp16
    exponent (0, subnormals, 65504): the epilogue carries W * ScaleQ and
    ScaleK with fixed power-of-two factors and reads relu'd int32 dots as fp32
    denormals, which is exact only if no product or partial sum leaves the
    normal range; dots bit-exact, scores within the int8 tolerance, selection
    consistent with the GPU's own scores."""
    import torch
    inp = synth.make_inputs(EXTREME[name], 17)
    rng = np.random.default_rng(1234)
    for key in ("weights", "q_scale", "k_scale"):
        inp[key] = _extreme_fp16(rng, inp[key].shape)
    p = inp["problem"]
    vis = vis_of(ora, inp)
    rows, k = rows_of(p), p["sparse_count"]
    cols = int(vis.max())
    log("case %s: extreme fp16 scales rows=%d cols=%d" % (name, rows, cols))
    ix = make_indexer(inp)
    dev = device_inputs(inp)
    gidx, gval, dots, scores = ix.run_debug(dev["query"], dev["key"], dev["weights"], dev["q_scale"],
                                            dev["k_scale"], dev["block_table"], 0, rows, cols)
    torch.cuda.synchronize()
    gidx, gval = gidx.cpu().numpy(), gval.cpu().numpy()
    dots, scores = dots.cpu().numpy(), scores.cpu().numpy()
    check_structure(gidx, gval, vis, k)
    for r in range(rows):
        v = int(vis[r])
        if v == 0:
            continue
        _, odots, osc = ora.row_detail(inp, r, 0, v)
        assert np.array_equal(dots[r, :, :v].astype(np.float64), odots), "row %d: int8 dots differ" % r
        assert np.all(np.isfinite(scores[r, :v])), "row %d: non-finite score" % r
        assert np.all(np.abs(scores[r, :v] - osc) <= ATOL + INT8_RTOL * np.abs(osc)), "row %d scores" % r
        n = min(k, v)
        assert np.array_equal(gidx[r, :n], stable_topk_set(scores[r, :v], k)), "row %d selection" % r
        assert np.array_equal(gval[r, :n], scores[r, gidx[r, :n]]), "row %d values" % r


def test_ties_go_to_lower_index(ora):
    """Identical keys give bit-identical scores; the lowest indices win."""
    spec = synth.small(batch=2, s1=2, aslk=[1500, 800], block_size=64, sparse_count=200, sparse_mode=3,
                       table="identity")
    inp = synth.make_inputs(spec, 5)
    keys = inp["key"].reshape(-1, 128)
    keys[:] = keys[0]
    kb = inp["k_scale"].reshape(-1)
    kb[:] = kb[0]
    vis = vis_of(ora, inp)
    gidx, gval, _ = run_gpu(inp)
    rc, oidx, oval, osc = ora.indexer(inp, scores_cols=int(vis.max()))
    for r in range(rows_of(inp["problem"])):
        n = min(200, int(vis[r]))
        assert np.array_equal(gidx[r, :n], np.arange(n)), r
        assert np.all(gval[r, :n] == gval[r, 0])


def test_empty_and_degenerate():
    import sparse_attention_token_paged_amd as qli
    for spec in (synth.small(batch=0, s1=4, aslk=[]),
                 synth.small(layout=synth.TND, batch=1, s1=5, aslq=[0], aslk=[50]),
                 synth.small(batch=2, s1=2, aslk=[0, 0])):
        inp = synth.make_inputs(spec, 1)
        gidx, gval, _ = run_gpu(inp)
        assert np.all(gidx == -1) and (gval is None or np.all(gval == -np.inf))


def test_repeat_runs_identical():
    inp = synth.make_inputs(SMALL["bsnd_int8_causal_bs48_pad"], 3)
    dev = device_inputs(inp)
    a_idx, a_val, ix = run_gpu(inp, dev)
    b_idx, b_val, _ = run_gpu(inp, dev, ix)
    assert np.array_equal(a_idx, b_idx) and np.array_equal(a_val, b_val)


@pytest.mark.parametrize("case", ["regular_causal_s3", "long_rt2_causal"])
def test_graph_replay(ora, case):
    """qli_run captured in a HIP graph (no host synchronisation, no memset
    nodes) and replayed: every replay, with eager work in between, gives the
    eager outputs, which match the oracle on every row.  Plan, workspace and
    outputs keep their addresses."""
    import torch
    inp = synth.make_inputs(SMALL[case] if case in SMALL else LONG[case], 5)
    dev = device_inputs(inp)
    a_idx, a_val, ix = run_gpu(inp, dev)
    oracle_check(ora, inp, a_idx, a_val)
    b_idx, b_val = ix.alloc_outputs()
    args = (dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
            b_idx, b_val)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ix.run(*args)  # first launches (occupancy queries) outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ix.run(*args)
    for rep in range(4):
        b_idx.fill_(-7)
        if b_val is not None:
            b_val.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(a_idx, b_idx.cpu().numpy()), "replay %d" % rep
        assert a_val is None or np.array_equal(a_val, b_val.cpu().numpy()), "replay %d" % rep
        ix.run(*args)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["bsnd_int8_causal_bs48_pad"])
def test_stages_compose(name):
    """Scoring stage then selection stage, as two calls, gives qli_run's outputs,
    also for long rows (segment selections, then merges), from a workspace that
    starts as garbage, and the selection stage alone gives them again."""
    import torch
    for inp in (synth.make_inputs(SMALL[name], 3), synth.make_inputs(LONG["long_rt2_causal"], 2)):
        dev = device_inputs(inp)
        a_idx, a_val, ix = run_gpu(inp, dev)
        b_idx, b_val = ix.alloc_outputs()
        args = (dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
                b_idx, b_val)
        if ix.workspace is not None:
            ix.workspace.fill_(0x5A)
        ix.run_stage(*args, stages=1)
        for rep in range(3):
            b_idx.fill_(7)
            if b_val is not None:
                b_val.fill_(7.0)
            ix.run_stage(*args, stages=2)
            torch.cuda.synchronize()
            assert np.array_equal(a_idx, b_idx.cpu().numpy()), "selection %d" % rep
            assert a_val is None or np.array_equal(a_val, b_val.cpu().numpy()), "selection %d" % rep


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_workload_full_size(ora, name):
    """Each named workload at full size, in the benchmark's launch
    configuration: structure and the full oracle check (scores within
    tolerance, index sets exact up to ties) on every row."""
    import time
    inp = synth.workload(name)
    p = inp["problem"]
    rows, k = rows_of(p), p["sparse_count"]
    log("workload %s: rows=%d k=%d" % (name, rows, k))
    vis = vis_of(ora, inp)
    gidx, gval, ix = run_gpu(inp)
    check_structure(gidx, gval, vis, k)
    t0 = time.perf_counter()
    rc, _, _, osc = ora.indexer(inp, scores_cols=max(1, int(vis.max())), nthreads=0)
    assert rc == 0
    log("  oracle over %d rows (%d visible pairs) in %.1f s" % (rows, int(vis.sum()), time.perf_counter() - t0))
    for r in range(rows):
        check_row(r, int(vis[r]), k, gidx[r], gval[r], osc[r, :vis[r]], rtol_of(inp))


# Full-size int8 dumps: rows [row0, row1) of a workload, dots bit-exact and
# scores within tolerance against the oracle, the selection equal to the
# stable top-k of the GPU's own scores.
FULL_DUMPS = [
    ("decode_int8_b24_s4_sk8192", 0, 2),
    ("decode_int8_b24_s4_sk8192", 94, 96),
    ("longctx_int8_b8_s2_sk131072_cmp4", 0, 2),
    ("longctx_int8_b8_s2_sk131072_cmp4", 14, 16),
    ("prefill_int8_tnd_4x2048", 2045, 2049),
    ("prefill_int8_tnd_4x2048", 8190, 8192),
]


@pytest.mark.parametrize("name,row0,row1", FULL_DUMPS, ids=["%s-%d" % (n, a) for n, a, _ in FULL_DUMPS])
def test_workload_full_size_dump(ora, name, row0, row1):
    import torch
    inp = synth.workload(name)
    p = inp["problem"]
    k = p["sparse_count"]
    vis = vis_of(ora, inp)
    cols = int(vis[row0:row1].max())
    log("workload dump %s rows [%d, %d) cols %d" % (name, row0, row1, cols))
    ix = make_indexer(inp)
    dev = device_inputs(inp)
    gidx, gval, dots, scores = ix.run_debug(dev["query"], dev["key"], dev["weights"], dev["q_scale"],
                                            dev["k_scale"], dev["block_table"], row0, row1, cols)
    torch.cuda.synchronize()
    gidx, gval = gidx.cpu().numpy(), gval.cpu().numpy()
    dots, scores = dots.cpu().numpy(), scores.cpu().numpy()
    for u, r in enumerate(range(row0, row1)):
        v = int(vis[r])
        _, odots, osc = ora.row_detail(inp, r, 0, v)
        assert np.array_equal(dots[u, :, :v].astype(np.float64), odots), "row %d: int8 dots differ" % r
        assert np.all(np.abs(scores[u, :v] - osc) <= ATOL + INT8_RTOL * np.abs(osc)), "row %d scores" % r
        n = min(k, v)
        assert np.array_equal(gidx[r, :n], stable_topk_set(scores[u, :v], k)), "row %d selection" % r
        assert np.array_equal(gval[r, :n], scores[u, gidx[r, :n]]), "row %d values" % r


# --- bounded decode: no host plan, key lengths on the device -------------------
BOUNDED = {
    # (spec with every batch at the bound: the cache and block table hold that much; actual lengths)
    "int8_s4_merges": (synth.small(batch=3, s1=4, aslk=[24000] * 3, block_size=64, sparse_count=2048,
                                   sparse_mode=3), [20000, 5000, 0]),
    "fp8_s1_mode0": (synth.small(qk=synth.FP8, batch=3, s1=1, aslk=[9000] * 3, block_size=64, sparse_count=300),
                     [3000, 100, 9000]),
    "int8_s2_cmp4": (synth.small(batch=2, s1=2, aslk=[40000] * 2, block_size=128, sparse_count=512,
                                 sparse_mode=3, cmp_ratio=4), [40000, 39999]),
    "int8_s3_short": (synth.small(batch=2, s1=3, aslk=[1500] * 2, block_size=32, sparse_count=256,
                                  sparse_mode=3), [1500, 700]),
    # more than 4 query rows per batch: 4-row groups that follow from the item's position
    "int8_s8_prefill": (synth.small(batch=2, s1=8, aslk=[3000] * 2, block_size=64, sparse_count=256,
                                    sparse_mode=3), [3000, 1200]),
    "int8_s13_chunks_merges": (synth.small(batch=2, s1=13, aslk=[20000] * 2, block_size=128, sparse_count=2048,
                                           sparse_mode=3), [20000, 9000]),
    "fp8_s6_mode0": (synth.small(qk=synth.FP8, batch=3, s1=6, aslk=[5000] * 3, block_size=32, sparse_count=300),
                     [5000, 17, 0]),
    "int8_s64_cmp2": (synth.small(batch=1, s1=64, aslk=[10000], block_size=128, sparse_count=512, sparse_mode=3,
                                  cmp_ratio=2), [9999]),
}


def bounded_case(name, seed=4):
    import torch
    spec, lens = BOUNDED[name]
    inp = synth.make_inputs(spec, seed)
    bound = int(spec.aslk[0])
    dev = device_inputs(inp)
    bix = qli_mod().BoundedIndexer(inp["problem"], bound)
    return inp, dev, bix, bound, lens


def qli_mod():
    import sparse_attention_token_paged_amd as q
    return q


def planned(inp, dev, lens):
    """qli_plan + qli_run for the same inputs with actual key lengths lens."""
    sub = dict(inp, aslk=np.asarray(lens, dtype=np.int32))
    idx, val, _ = run_gpu(sub, dev)
    return idx, val


@pytest.mark.parametrize("name", list(BOUNDED))
def test_bounded_matches_planned(ora, name):
    """qli_run_bounded gives exactly qli_run's outputs (same kernels, same
    arithmetic; the lengths are read on the device), checked against the
    oracle's structure too."""
    import torch
    inp, dev, bix, bound, lens = bounded_case(name)
    log("bounded %s: bound %d lens %s" % (name, bound, lens))
    aslk = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx, val = bix.alloc_outputs()
    bix.run(aslk, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
            idx, val)
    torch.cuda.synchronize()
    p_idx, p_val = planned(inp, dev, lens)
    assert np.array_equal(idx.cpu().numpy(), p_idx)
    assert p_val is None or np.array_equal(val.cpu().numpy(), p_val)
    oracle_check(ora, dict(inp, aslk=np.asarray(lens, dtype=np.int32)), idx.cpu().numpy(),
                 None if val is None else val.cpu().numpy())


def oracle_check(ora, inp, idx, val):
    """Structure and the full oracle check on every row."""
    p = inp["problem"]
    vis = vis_of(ora, inp)
    k = p["sparse_count"]
    check_structure(idx, val, vis, k)
    rc, _, _, sc = ora.indexer(inp, scores_cols=max(1, int(vis.max()) if vis.size else 1))
    assert rc == 0
    for r in range(vis.size):
        check_row(r, int(vis[r]), k, idx[r], None if val is None else val[r], sc[r, :vis[r]], rtol_of(inp))


GRAPH_LENS = {
    "int8_s4_merges": ([24000, 24000, 24000], [9000, 0, 23999], [1, 2048, 12000], [3000, 17000, 8193]),
    "int8_s13_chunks_merges": ([20000, 20000], [0, 4097], [8193, 12], [19999, 5000]),
}


@pytest.mark.parametrize("case", list(GRAPH_LENS))
def test_bounded_graph_replay(ora, case):
    """qli_run_bounded captured once in a HIP graph, replayed after the device
    key lengths change: every replay equals qli_plan + qli_run for the new
    lengths (including a batch that sees nothing and one longer than a segment)."""
    import torch
    inp, dev, bix, bound, _ = bounded_case(case, seed=6)
    aslk = torch.tensor([bound] * inp["problem"]["batch"], dtype=torch.int32, device="cuda")
    idx, val = bix.alloc_outputs()
    args = (aslk, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
            idx, val)
    bix.run(*args)  # first launches (occupancy queries) outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bix.run(*args)
    for lens in GRAPH_LENS[case]:
        aslk.copy_(torch.tensor(lens, dtype=torch.int32))
        idx.fill_(-7)
        val.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        p_idx, p_val = planned(inp, dev, lens)
        assert np.array_equal(idx.cpu().numpy(), p_idx), "lengths %s" % lens
        assert np.array_equal(val.cpu().numpy(), p_val), "lengths %s" % lens
        oracle_check(ora, dict(inp, aslk=np.asarray(lens, dtype=np.int32)), idx.cpu().numpy(), val.cpu().numpy())


BOUNDED_TND = {
    # (spec whose cache holds the bound for every batch, device aslq, actual key lengths)
    "tnd_mixed_padding_rows": (synth.small(layout=synth.TND, batch=3, s1=40, aslq=[5, 25, 33], aslk=[2000] * 3,
                                           block_size=64, sparse_count=256, sparse_mode=3), [5, 25, 33],
                               [300, 2000, 900]),
    "tnd_chunks_merges": (synth.small(layout=synth.TND, batch=2, s1=20, aslq=[7, 20], aslk=[20000] * 2,
                                      block_size=128, sparse_count=2048, sparse_mode=3), [7, 20], [20000, 9000]),
    "tnd_fp8_mode0_empty_batches": (synth.small(qk=synth.FP8, layout=synth.TND, batch=4, s1=30,
                                                aslq=[0, 10, 10, 28], aslk=[5000] * 4, block_size=32,
                                                sparse_count=300), [0, 10, 10, 28], [100, 5000, 300, 0]),
    "tnd_decode_like_cmp2": (synth.small(layout=synth.TND, batch=4, s1=8, aslq=[2, 4, 6, 8], aslk=[3000] * 4,
                                         block_size=64, sparse_count=256, sparse_mode=3, cmp_ratio=2),
                             [2, 4, 6, 8], [3000, 100, 2500, 1]),
}


def bounded_tnd_run(name, aslq, lens, seed=4):
    import torch
    spec = BOUNDED_TND[name][0]
    inp = synth.make_inputs(spec, seed)
    dev = device_inputs(inp)
    bix = qli_mod().BoundedIndexer(inp["problem"], int(spec.aslk[0]))
    q = torch.tensor(aslq, dtype=torch.int32, device="cuda")
    k = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx, val = bix.alloc_outputs()
    bix.run(k, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
            idx, val, aslq_dev=q)
    torch.cuda.synchronize()
    return inp, dev, idx.cpu().numpy(), val.cpu().numpy()


@pytest.mark.parametrize("name", list(BOUNDED_TND))
def test_bounded_tnd_matches_planned(ora, name):
    """qli_run_bounded_tnd (query and key lengths read on the device) against
    qli_plan + qli_run: bit-identical where the plan also takes 4-row items
    (some batch has at least 3 rows), else within the parity rule of the
    oracle; every row's structure checked."""
    _, aslq, lens = BOUNDED_TND[name]
    log("bounded tnd %s: aslq %s lens %s" % (name, aslq, lens))
    inp, dev, idx, val = bounded_tnd_run(name, aslq, lens)
    p = inp["problem"]
    aq, ak = np.asarray(aslq, dtype=np.int32), np.asarray(lens, dtype=np.int32)
    vis = ora.row_visible(p["layout_query"], p["batch"], p["s1"], p["sparse_mode"], p["cmp_ratio"], aq, ak)
    check_structure(idx, val, vis, p["sparse_count"])
    per_batch = np.diff(np.concatenate([[0], aq]))
    sub = dict(inp, aslq=aq, aslk=ak)
    if per_batch.max() >= 3:
        p_idx, p_val = planned(sub, dev, lens)
        assert np.array_equal(idx, p_idx) and np.array_equal(val, p_val)
    oracle_check(ora, sub, idx, val)


def test_bounded_tnd_prefix_sums_out_of_contract(ora):
    """Device query prefix sums that break the contract (decreasing, beyond T,
    negative) are taken as their running maximum clamped to [0, T]: the run
    completes and equals qli_plan + qli_run on that partition."""
    name = "tnd_mixed_padding_rows"
    spec = BOUNDED_TND[name][0]
    bad, lens = [30, -4, 70], [2000, 700, 1500]
    clamped = list(np.minimum(np.maximum.accumulate(np.maximum(bad, 0)), spec.s1))
    inp, dev, idx, val = bounded_tnd_run(name, bad, lens)
    sub = dict(inp, aslq=np.asarray(clamped, dtype=np.int32))
    p_idx, p_val = planned(sub, dev, lens)
    assert np.array_equal(idx, p_idx) and np.array_equal(val, p_val)
    oracle_check(ora, dict(sub, aslk=np.asarray(lens, dtype=np.int32)), idx, val)


def tnd_many_batches(nb, bound, seed):
    """nb batches of 0 to 3 query rows (batch 100 % nb has 9, so qli_plan
    takes 4-row items too) and key lengths 0 to bound, batch 5 empty."""
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 4, size=nb)
    counts[100 % nb] = 9
    lens = rng.integers(0, bound + 1, size=nb)
    lens[5] = 0
    return [int(x) for x in np.cumsum(counts)], [int(x) for x in lens]


@pytest.mark.parametrize("nb", [128, 129, 4096])
def test_bounded_tnd_most_batches(ora, nb):
    """TND around the kernels' own partition (up to 128 batches) and the
    table kernel (129 up to its limit of 4096): bit-identical to qli_plan +
    qli_run and oracle-checked on every row."""
    import torch
    bound = 300
    aslq, lens = tnd_many_batches(nb, bound, 41)
    spec = synth.small(layout=synth.TND, batch=nb, s1=aslq[-1], aslq=aslq, aslk=[bound] * nb, block_size=16,
                       sparse_count=64, sparse_mode=3)
    inp = synth.make_inputs(spec, 9)
    dev = device_inputs(inp)
    log("bounded tnd: %d batches, %d rows" % (nb, aslq[-1]))
    bix = qli_mod().BoundedIndexer(inp["problem"], bound)
    idx, val = bix.alloc_outputs()
    bix.run(torch.tensor(lens, dtype=torch.int32, device="cuda"), dev["query"], dev["key"], dev["weights"],
            dev["q_scale"], dev["k_scale"], dev["block_table"], idx, val,
            aslq_dev=torch.tensor(aslq, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    p_idx, p_val = planned(inp, dev, lens)
    assert np.array_equal(idx, p_idx) and np.array_equal(val, p_val)
    oracle_check(ora, dict(inp, aslk=np.asarray(lens, dtype=np.int32)), idx, val)


@pytest.mark.parametrize("nb", [128, 129])
def test_bounded_tnd_many_batches_graph_replay(ora, nb):
    """Both ways to the TND partition (in the kernels, through the table
    kernel) captured once and replayed with new query prefix sums and key
    lengths (the row count T fixed, later batches' rows past the last prefix
    sum in one set): every replay equals qli_plan + qli_run."""
    import torch
    bound = 2500
    sets = [tnd_many_batches(nb, bound, s) for s in (51, 52, 53)]
    t = max(q[-1] for q, _ in sets)
    sets[2] = ([min(x, t // 2) for x in sets[2][0]], sets[2][1])  # rows from t // 2 on belong to no batch
    spec = synth.small(layout=synth.TND, batch=nb, s1=t, aslq=sets[0][0][:-1] + [t], aslk=[bound] * nb,
                       block_size=64, sparse_count=1024, sparse_mode=3)
    inp = synth.make_inputs(spec, 10)
    dev = device_inputs(inp)
    log("bounded tnd graph: %d batches, %d rows" % (nb, t))
    bix = qli_mod().BoundedIndexer(inp["problem"], bound)
    q = torch.tensor(spec.aslq, dtype=torch.int32, device="cuda")
    k = torch.tensor([bound] * nb, dtype=torch.int32, device="cuda")
    idx, val = bix.alloc_outputs()
    args = (k, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"], idx, val)
    bix.run(*args, aslq_dev=q)  # first launches outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bix.run(*args, aslq_dev=q)
    for aslq, lens in sets:
        q.copy_(torch.tensor(aslq, dtype=torch.int32))
        k.copy_(torch.tensor(lens, dtype=torch.int32))
        idx.fill_(-7)
        val.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        sub = dict(inp, aslq=np.asarray(aslq, dtype=np.int32))
        p_idx, p_val = planned(sub, dev, lens)
        assert np.array_equal(idx.cpu().numpy(), p_idx), "aslq %s" % aslq[:8]
        assert np.array_equal(val.cpu().numpy(), p_val), "aslq %s" % aslq[:8]
        oracle_check(ora, dict(sub, aslk=np.asarray(lens, dtype=np.int32)), idx.cpu().numpy(), val.cpu().numpy())


def test_bounded_tnd_graph_replay(ora):
    """qli_run_bounded_tnd captured once; between replays both the device query
    prefix sums and the key lengths change (rows move between batches, batches
    empty out, rows fall past the last prefix sum): every replay equals
    qli_plan + qli_run for the new lengths."""
    import torch
    name = "tnd_chunks_merges"
    spec = BOUNDED_TND[name][0]
    inp = synth.make_inputs(spec, 6)
    dev = device_inputs(inp)
    bound = int(spec.aslk[0])
    bix = qli_mod().BoundedIndexer(inp["problem"], bound)
    q = torch.tensor([7, 20], dtype=torch.int32, device="cuda")
    k = torch.tensor([bound, bound], dtype=torch.int32, device="cuda")
    idx, val = bix.alloc_outputs()
    args = (k, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"], idx, val)
    bix.run(*args, aslq_dev=q)  # first launches outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bix.run(*args, aslq_dev=q)
    for aslq, lens in (([7, 20], [20000, 20000]), ([0, 12], [5000, 8193]), ([20, 20], [12, 20000]),
                       ([3, 9], [19999, 0])):
        q.copy_(torch.tensor(aslq, dtype=torch.int32))
        k.copy_(torch.tensor(lens, dtype=torch.int32))
        idx.fill_(-7)
        val.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        sub = dict(inp, aslq=np.asarray(aslq, dtype=np.int32))
        p_idx, p_val = planned(sub, dev, lens)
        assert np.array_equal(idx.cpu().numpy(), p_idx), "aslq %s lens %s" % (aslq, lens)
        assert np.array_equal(val.cpu().numpy(), p_val), "aslq %s lens %s" % (aslq, lens)
        oracle_check(ora, dict(sub, aslk=np.asarray(lens, dtype=np.int32)), idx.cpu().numpy(), val.cpu().numpy())


# --- bounded BSND with actual_seq_lengths_query on the device ---------------
BOUNDED_ASLQ = {
    # decode items built on the device: staged rows, merges, unused rows, an empty batch
    "decode_s4": (synth.small(batch=4, s1=4, aslk=[20000] * 4, block_size=64, sparse_count=512, sparse_mode=3),
                  [4, 2, 0, 3], [20000, 9000, 20000, 1]),
    "decode_s1_fp8": (synth.small(qk=synth.FP8, batch=5, s1=1, aslk=[9000] * 5, block_size=32, sparse_count=300),
                      [1, 0, 1, 1, 1], [9000, 9000, 150, 0, 4097]),
    # prefill items (S1 > 4): rows past the count are padding
    "prefill_s13": (synth.small(batch=3, s1=13, aslk=[12000] * 3, block_size=128, sparse_count=1024,
                                sparse_mode=3), [13, 5, 9], [12000, 3000, 11999]),
}


@pytest.mark.parametrize("name", list(BOUNDED_ASLQ))
def test_bounded_aslq_matches_planned(ora, name):
    """qli_run_bounded_aslq gives exactly qli_plan + qli_run with the same host
    query counts, and matches the oracle on every row."""
    import torch
    spec, aslq, lens = BOUNDED_ASLQ[name]
    inp = synth.make_inputs(spec, 8)
    dev = device_inputs(inp)
    bound = int(spec.aslk[0])
    log("bounded aslq %s: aslq %s lens %s" % (name, aslq, lens))
    bix = qli_mod().BoundedIndexer(inp["problem"], bound)
    idx, val = bix.alloc_outputs()
    bix.run(torch.tensor(lens, dtype=torch.int32, device="cuda"), dev["query"], dev["key"], dev["weights"],
            dev["q_scale"], dev["k_scale"], dev["block_table"], idx, val,
            aslq_dev=torch.tensor(aslq, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    sub = dict(inp, aslq=np.asarray(aslq, dtype=np.int32))
    p_idx, p_val = planned(sub, dev, lens)
    assert np.array_equal(idx.cpu().numpy(), p_idx) and np.array_equal(val.cpu().numpy(), p_val)
    oracle_check(ora, dict(sub, aslk=np.asarray(lens, dtype=np.int32)), idx.cpu().numpy(), val.cpu().numpy())


def test_bounded_aslq_graph_replay(ora):
    """qli_run_bounded_aslq captured once (device item table included);
    between replays the query counts and key lengths change: every replay
    equals qli_plan + qli_run for the new lengths."""
    import torch
    spec = BOUNDED_ASLQ["decode_s4"][0]
    inp = synth.make_inputs(spec, 9)
    dev = device_inputs(inp)
    bound = int(spec.aslk[0])
    bix = qli_mod().BoundedIndexer(inp["problem"], bound)
    q = torch.tensor([4, 4, 4, 4], dtype=torch.int32, device="cuda")
    k = torch.tensor([bound] * 4, dtype=torch.int32, device="cuda")
    idx, val = bix.alloc_outputs()
    args = (k, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"], idx, val)
    bix.run(*args, aslq_dev=q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bix.run(*args, aslq_dev=q)
    for aslq, lens in (([4, 4, 4, 4], [20000] * 4), ([1, 0, 3, 4], [700, 20000, 8193, 16000]),
                       ([2, 2, 2, 2], [0, 12, 19999, 5000]), ([4, 3, 0, 1], [20000, 20000, 20000, 20000])):
        q.copy_(torch.tensor(aslq, dtype=torch.int32))
        k.copy_(torch.tensor(lens, dtype=torch.int32))
        idx.fill_(-7)
        val.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        sub = dict(inp, aslq=np.asarray(aslq, dtype=np.int32))
        p_idx, p_val = planned(sub, dev, lens)
        assert np.array_equal(idx.cpu().numpy(), p_idx), "aslq %s lens %s" % (aslq, lens)
        assert np.array_equal(val.cpu().numpy(), p_val), "aslq %s lens %s" % (aslq, lens)
        oracle_check(ora, dict(sub, aslk=np.asarray(lens, dtype=np.int32)), idx.cpu().numpy(), val.cpu().numpy())


@pytest.mark.parametrize("nb", [256, 257, 300])
def test_bounded_many_batches_table(ora, nb):
    """Around the scoring kernel's own split limit: at 256 batches it plans
    the items itself, above that the separate planning kernel writes the item
    table.  Ragged lengths with empty batches and query counts; bit-identical
    to qli_plan + qli_run and oracle-checked, twice with different lengths
    from the same workspace."""
    import torch
    rng = np.random.default_rng(5)
    lens0 = [int(x) for x in rng.integers(0, 3000, size=nb)]
    lens0[7] = 0
    bound = 3000
    # every batch's blocks cover the bound: the lengths below only ever read allocated blocks
    spec = synth.small(batch=nb, s1=2, aslk=[bound] * nb, block_size=32, sparse_count=256, sparse_mode=3)
    inp = synth.make_inputs(spec, 12)
    dev = device_inputs(inp)
    bix = qli_mod().BoundedIndexer(inp["problem"], bound)
    for lens, aslq in ((lens0, None), ([int(x) for x in rng.integers(0, 3001, size=nb)],
                                       [int(x) for x in rng.integers(0, 3, size=nb)])):
        idx, val = bix.alloc_outputs()
        q = None if aslq is None else torch.tensor(aslq, dtype=torch.int32, device="cuda")
        bix.run(torch.tensor(lens, dtype=torch.int32, device="cuda"), dev["query"], dev["key"], dev["weights"],
                dev["q_scale"], dev["k_scale"], dev["block_table"], idx, val, aslq_dev=q)
        torch.cuda.synchronize()
        sub = dict(inp, aslq=None if aslq is None else np.asarray(aslq, dtype=np.int32))
        p_idx, p_val = planned(sub, dev, lens)
        assert np.array_equal(idx.cpu().numpy(), p_idx) and np.array_equal(val.cpu().numpy(), p_val)
        oracle_check(ora, dict(sub, aslk=np.asarray(lens, dtype=np.int32)), idx.cpu().numpy(), val.cpu().numpy())


# --- seeded random problems -----------------------------------------------------
def random_spec(i: int):
    """A random small problem (seeded by i): dtype, layout, batch, ragged key
    lengths (zeros included), query counts, compression, mode, block size,
    sparse_count and stride padding, resampled until it has at most 300k
    visible pairs (so the oracle scores every row quickly)."""
    rng = np.random.default_rng(20260 + i)
    while True:
        qk = int(rng.choice([synth.INT8, synth.FP8]))
        layout = int(rng.choice([synth.BSND, synth.TND], p=[0.7, 0.3]))
        batch = int(rng.integers(1, 5))
        cmp = int(rng.choice([1, 1, 2, 4, 8, 16]))
        aslk = [int(rng.integers(0, 12000)) if rng.random() > 0.1 else 0 for _ in range(batch)]
        kw = dict(qk=qk, layout=layout, batch=batch, aslk=aslk, cmp_ratio=cmp,
                  sparse_mode=int(rng.choice([0, 3])), block_size=int(rng.choice([16, 32, 48, 64, 128, 256, 512])),
                  sparse_count=int(rng.choice([1, 7, 64, 300, 1000, 2048])),
                  stride_pad=int(rng.choice([0, 0, 16, 64])))
        if layout == synth.BSND:
            s1 = int(rng.integers(1, 9))
            kw["s1"] = s1
            if rng.random() < 0.3:
                kw["aslq"] = [int(rng.integers(0, s1 + 1)) for _ in range(batch)]
        else:
            counts = [int(rng.integers(0, 40)) for _ in range(batch)]
            kw["aslq"] = list(np.cumsum(counts))
            kw["s1"] = int(sum(counts)) + int(rng.integers(0, 5))
        spec = synth.small(name="random%d" % i, **kw)
        rows_vis = 0
        for b in range(batch):
            nq = (kw["aslq"][b] if "aslq" in kw and layout == synth.BSND else kw["s1"]) if layout == synth.BSND \
                else counts[b]
            rows_vis += nq * (aslk[b] // cmp)
        if 0 < rows_vis <= 300000:
            return spec


@pytest.mark.parametrize("i", range(24))
def test_parity_random(ora, i):
    spec = random_spec(i)
    inp = synth.make_inputs(spec, i)
    p = inp["problem"]
    log("random %d: %s" % (i, spec))
    vis = vis_of(ora, inp)
    cols = max(1, int(vis.max()) if vis.size else 1)
    rc, oidx, oval, osc = ora.indexer(inp, scores_cols=cols)
    assert rc == 0
    gidx, gval, _ = run_gpu(inp)
    k = p["sparse_count"]
    check_structure(gidx, gval, vis, k)
    for r in range(rows_of(p)):
        check_row(r, int(vis[r]), k, gidx[r], gval[r], osc[r, :vis[r]], rtol_of(inp))


@pytest.mark.parametrize("i", range(12))
def test_bounded_random(ora, i):
    """Seeded random problems (the generator above) run without a host plan,
    lengths (and query counts, BSND ones included) on the device and the bound
    at the longest key: bit-identical to qli_plan + qli_run where the plan uses
    the same tiles (every BSND problem, TND with a batch of more than 4 rows),
    else within the parity rule of the oracle."""
    import torch
    spec = random_spec(100 + i)
    inp = synth.make_inputs(spec, i)
    p = inp["problem"]
    log("bounded random %d: %s" % (i, spec))
    dev = device_inputs(inp)
    bound = max(1, int(max(inp["aslk"])))
    bix = qli_mod().BoundedIndexer(p, bound)
    k_dev = torch.from_numpy(inp["aslk"].astype(np.int32)).cuda()
    q_dev = torch.from_numpy(np.asarray(inp["aslq"], dtype=np.int32)).cuda() if inp["aslq"] is not None else None
    idx, val = bix.alloc_outputs()
    bix.run(k_dev, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
            idx, val, aslq_dev=q_dev)
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    vis = vis_of(ora, inp)
    check_structure(idx, val, vis, p["sparse_count"])
    tiles_match = spec.layout == synth.BSND or np.diff(np.concatenate([[0], inp["aslq"]])).max() >= 3
    if tiles_match:
        p_idx, p_val, _ = run_gpu(inp, dev)
        assert np.array_equal(idx, p_idx) and np.array_equal(val, p_val)
    oracle_check(ora, inp, idx, val)


@pytest.mark.parametrize("i", range(10))
def test_bounded_random_windowed(ora, i):
    """The random problems above with random pre/next_tokens windows, run
    without a host plan: bit-identical to qli_plan + qli_run where the plan
    uses the same tiles, and every row against the oracle's window."""
    import dataclasses
    import torch
    rng = np.random.default_rng(991 + i)
    spec = dataclasses.replace(random_spec(300 + i),
                               pre_tokens=int(rng.choice([0, 1, 7, 100, 1000, 5000, synth.INT64_MAX])),
                               next_tokens=int(rng.choice([0, 3, 50, synth.INT64_MAX])))
    inp = synth.make_inputs(spec, i)
    p = inp["problem"]
    log("bounded random windowed %d: %s" % (i, spec))
    dev = device_inputs(inp)
    bound = max(1, int(max(inp["aslk"])))
    bix = qli_mod().BoundedIndexer(p, bound)
    k_dev = torch.from_numpy(inp["aslk"].astype(np.int32)).cuda()
    q_dev = torch.from_numpy(np.asarray(inp["aslq"], dtype=np.int32)).cuda() if inp["aslq"] is not None else None
    idx, val = bix.alloc_outputs()
    bix.run(k_dev, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
            idx, val, aslq_dev=q_dev)
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    tiles_match = spec.layout == synth.BSND or np.diff(np.concatenate([[0], inp["aslq"]])).max() >= 3
    if tiles_match:
        p_idx, p_val, _ = run_gpu(inp, dev)
        assert np.array_equal(idx, p_idx) and np.array_equal(val, p_val)
    check_windowed(ora, inp, idx, val)


@pytest.mark.parametrize("case", ["bsnd_int8_causal_bs48_pad", "long_rt2_causal", "tnd_int8_prefill_mixed"])
def test_without_values(case):
    """return_value = 0 (参数说明: sparse_values optional): no value buffer, the
    same indices as with values."""
    inp = synth.make_inputs(SMALL[case] if case in SMALL else LONG[case], 8)
    dev = device_inputs(inp)
    a_idx, a_val, _ = run_gpu(inp, dev)
    assert a_val is not None
    noval = dict(inp, problem=dict(inp["problem"], return_value=0))
    b_idx, b_val, _ = run_gpu(noval, dev)
    assert b_val is None and np.array_equal(a_idx, b_idx)


def test_bounded_without_values():
    import torch
    inp, dev, _, bound, lens = bounded_case("int8_s4_merges")
    p0 = dict(inp["problem"], return_value=0)
    bix = qli_mod().BoundedIndexer(p0, bound)
    aslk = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx, val = bix.alloc_outputs()
    assert val is None
    bix.run(aslk, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
            idx, None)
    torch.cuda.synchronize()
    p_idx, _ = planned(inp, dev, lens)
    assert np.array_equal(idx.cpu().numpy(), p_idx)


# --- pre_tokens / next_tokens windows (qli_plan / qli_run) -------------------
WINDOWED = {
    # decode items (4 rows): staged rows with a window start, and short direct rows
    "win_decode_rt4_staged": synth.small(batch=3, s1=4, aslk=[5000, 700, 90], block_size=64, sparse_count=256,
                                         sparse_mode=3, pre_tokens=1000, next_tokens=0),
    # one-row items, mode 0 with a window on both sides: direct rows whose range starts past 0
    "win_decode_rt1_direct": synth.small(batch=4, s1=1, aslk=[3000, 2000, 100, 64], block_size=32,
                                         sparse_count=300, pre_tokens=200, next_tokens=5),
    # prefill items, compressed keys, staged rows
    "win_prefill_mode0_cmp2": synth.small(batch=2, s1=40, aslk=[3000, 2500], block_size=32, sparse_count=64,
                                          cmp_ratio=2, pre_tokens=300, next_tokens=50),
    # TND prefill, direct rows with a window start
    "win_tnd_prefill_direct": synth.small(layout=synth.TND, batch=2, s1=30, aslq=[12, 30], aslk=[500, 4000],
                                          block_size=32, sparse_count=128, sparse_mode=3, cmp_ratio=4,
                                          pre_tokens=300, next_tokens=0),
    # windows longer than one selection segment: segments based at the window start, then a merge
    "win_long_segments": synth.small(batch=2, s1=2, aslk=[70000, 65000], block_size=128, sparse_count=512,
                                     sparse_mode=3, pre_tokens=30000),
    "win_fp8_decode": synth.small(qk=synth.FP8, batch=3, s1=1, aslk=[9000, 4000, 300], block_size=64,
                                  sparse_count=200, pre_tokens=2500, next_tokens=0),
    # pre = next = 0: each row sees its own position only
    "win_zero_width": synth.small(batch=2, s1=5, aslk=[100, 50], block_size=16, sparse_count=8,
                                  pre_tokens=0, next_tokens=0),
}


def check_windowed(ora, inp, gidx, gval):
    """Every row against the oracle's scores of its window [lo, hi): positions
    relative to lo go through the same checks as unwindowed rows."""
    p = inp["problem"]
    lo, hi = ora.row_range(p["layout_query"], p["batch"], p["s1"], p["sparse_mode"], p["cmp_ratio"], inp["aslq"],
                           inp["aslk"], p["pre_tokens"], p["next_tokens"])
    rc, _, _, osc = ora.indexer(inp, scores_cols=max(1, int(hi.max()) if hi.size else 1))
    assert rc == 0
    k = p["sparse_count"]
    rel = np.where(gidx >= 0, gidx - lo[:, None], -1)
    check_structure(rel, gval, hi - lo, k)
    for r in range(rows_of(p)):
        check_row(r, int(hi[r] - lo[r]), k, rel[r], None if gval is None else gval[r], osc[r, lo[r]:hi[r]],
                  rtol_of(inp))
    return lo, hi


@pytest.mark.parametrize("name", list(WINDOWED))
def test_parity_windowed(ora, name):
    inp = synth.make_inputs(WINDOWED[name], 17)
    p = inp["problem"]
    log("case %s: rows=%d k=%d pre=%d next=%d" % (name, rows_of(p), p["sparse_count"], p["pre_tokens"],
                                                   p["next_tokens"]))
    gidx, gval, _ = run_gpu(inp)
    lo, hi = check_windowed(ora, inp, gidx, gval)
    assert lo.max() > 0   # every case has rows whose window starts past entry 0


# --- windows in bounded runs (qli_run_bounded* with pre/next_tokens) ---------
BOUNDED_WINDOWED = dict(WINDOWED)
# decode of more than 256 batches: the device item table carries each row's window start
BOUNDED_WINDOWED["win_decode_table_300"] = synth.small(
    batch=300, s1=2, aslk=[int(x) for x in np.random.default_rng(61).integers(0, 3000, size=300)], block_size=64,
    sparse_count=128, sparse_mode=3, pre_tokens=700, next_tokens=0)
# prefill groups whose windows start past several chunks of the bound
BOUNDED_WINDOWED["win_prefill_far_start"] = synth.small(batch=2, s1=24, aslk=[9000, 6000], block_size=128,
                                                        sparse_count=256, sparse_mode=3, pre_tokens=600)
# TND of more than 128 batches (the table kernel's partition) under a window, mode 0 with a lookahead
_tnd_counts = np.random.default_rng(62).integers(0, 4, size=160)
_tnd_counts[7] = 9
BOUNDED_WINDOWED["win_tnd_table_160"] = synth.small(
    layout=synth.TND, batch=160, s1=int(_tnd_counts.sum()), aslq=[int(x) for x in np.cumsum(_tnd_counts)],
    aslk=[int(x) for x in np.random.default_rng(63).integers(0, 2500, size=160)], block_size=32,
    sparse_count=96, sparse_mode=0, pre_tokens=400, next_tokens=30)


def bounded_windowed_run(inp, dev, lens, bound, aslq=None):
    import torch
    bix = qli_mod().BoundedIndexer(inp["problem"], bound)
    idx, val = bix.alloc_outputs()
    q = None if aslq is None else torch.tensor(aslq, dtype=torch.int32, device="cuda")
    bix.run(torch.tensor(lens, dtype=torch.int32, device="cuda"), dev["query"], dev["key"], dev["weights"],
            dev["q_scale"], dev["k_scale"], dev["block_table"], idx, val, aslq_dev=q)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


@pytest.mark.parametrize("name", list(BOUNDED_WINDOWED))
def test_bounded_windowed_matches_planned(ora, name):
    """Windows in bounded runs: each row's range [lo, hi) is derived on the
    device (decode items planned in the kernel or by the item-table kernel,
    4-row groups, TND), scores land at entry - lo of the row's region and the
    selection is based at lo.  Bit-identical to qli_plan + qli_run and checked
    against the oracle's window on every row."""
    inp = synth.make_inputs(BOUNDED_WINDOWED[name], 17)
    p = inp["problem"]
    bound = int(max(inp["aslk"])) if p["batch"] else 0
    log("bounded windowed %s: rows=%d pre=%d next=%d bound=%d" % (name, rows_of(p), p["pre_tokens"],
                                                                   p["next_tokens"], bound))
    dev = device_inputs(inp)
    tnd = p["layout_query"] == synth.TND
    idx, val = bounded_windowed_run(inp, dev, [int(x) for x in inp["aslk"]], bound,
                                    aslq=[int(x) for x in inp["aslq"]] if tnd else None)
    p_idx, p_val, _ = run_gpu(inp, dev)
    assert np.array_equal(idx, p_idx) and np.array_equal(val, p_val)
    check_windowed(ora, inp, idx, val)


@pytest.mark.parametrize("name", ["win_decode_rt4_staged", "win_decode_table_300", "win_tnd_prefill_direct"])
def test_bounded_windowed_graph_replay(ora, name):
    """A windowed bounded run captured once, replayed with other key lengths
    (and TND prefix sums): the windows follow each row's new position; every
    replay equals qli_plan + qli_run and the oracle."""
    import dataclasses
    import torch
    spec = BOUNDED_WINDOWED[name]
    bound = int(max(spec.aslk))
    spec = dataclasses.replace(spec, aslk=[bound] * spec.batch)  # every batch's cache holds the bound
    inp = synth.make_inputs(spec, 18)
    p = inp["problem"]
    dev = device_inputs(inp)
    tnd = p["layout_query"] == synth.TND
    bix = qli_mod().BoundedIndexer(p, bound)
    k = torch.tensor([bound] * p["batch"], dtype=torch.int32, device="cuda")
    q = torch.tensor(inp["aslq"], dtype=torch.int32, device="cuda") if tnd else None
    idx, val = bix.alloc_outputs()
    args = (k, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"], idx, val)
    bix.run(*args, aslq_dev=q)  # first launches outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bix.run(*args, aslq_dev=q)
    rng = np.random.default_rng(19)
    for rep in range(3):
        lens = [int(x) for x in rng.integers(0, bound + 1, size=p["batch"])]
        lens[0] = bound if rep == 0 else lens[0]
        sub = dict(inp, aslk=np.asarray(lens, dtype=np.int32))
        if tnd:
            cuts = np.sort(rng.integers(0, p["s1"] + 1, size=p["batch"]))
            sub["aslq"] = cuts.astype(np.int32)
            q.copy_(torch.from_numpy(sub["aslq"]))
        k.copy_(torch.tensor(lens, dtype=torch.int32))
        idx.fill_(-7)
        val.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        p_idx, p_val, _ = run_gpu(sub, dev)
        assert np.array_equal(idx.cpu().numpy(), p_idx), "replay %d" % rep
        assert np.array_equal(val.cpu().numpy(), p_val), "replay %d" % rep
        check_windowed(ora, sub, idx.cpu().numpy(), val.cpu().numpy())


# --- score-ordered output (sort_output = 1) -----------------------------------
SORTED = {
    "decode_rt4_staged": SMALL["bsnd_int8_causal_bs48_pad"],
    "tnd_prefill_mixed": SMALL["tnd_int8_prefill_mixed"],
    "fp8_mode0": SMALL["bsnd_fp8_mode0"],
    "k2048": SMALL["bsnd_int8_k2048"],
    "k1": SMALL["bsnd_int8_k1"],
    "long_segments": LONG["long_rt1_ragged"],
    "windowed": WINDOWED["win_decode_rt4_staged"],
}


def by_score(idx, val):
    """Each row's listed slots reordered by descending value, equal values by
    ascending index; padding stays at the tail."""
    out_i, out_v = np.full_like(idx, -1), np.full_like(val, -np.inf)
    for r in range(idx.shape[0]):
        n = int((idx[r] >= 0).sum())
        o = np.lexsort((idx[r, :n], -val[r, :n].astype(np.float64)))
        out_i[r, :n], out_v[r, :n] = idx[r, o], val[r, o]
    return out_i, out_v


@pytest.mark.parametrize("name", list(SORTED))
def test_sorted_output(ora, name):
    """sort_output reorders exactly the selection of the default run (index
    work: bit-exact), also without returned values, and the order agrees with
    the oracle's fp64 ranking up to the score tolerance."""
    inp = synth.make_inputs(SORTED[name], 23)
    p = inp["problem"]
    log("case %s: sorted output rows=%d k=%d" % (name, rows_of(p), p["sparse_count"]))
    dev = device_inputs(inp)
    gidx, gval, _ = run_gpu(inp, dev)
    sidx, sval, _ = run_gpu(dict(inp, problem=dict(p, sort_output=1)), dev)
    want_i, want_v = by_score(gidx, gval)
    assert np.array_equal(sidx, want_i) and np.array_equal(sval, want_v)
    nidx, nval, _ = run_gpu(dict(inp, problem=dict(p, sort_output=1, return_value=0)), dev)
    assert nval is None and np.array_equal(nidx, sidx)
    lo, hi = ora.row_range(p["layout_query"], p["batch"], p["s1"], p["sparse_mode"], p["cmp_ratio"], inp["aslq"],
                           inp["aslk"], p["pre_tokens"], p["next_tokens"])
    _, oidx, _, osc = ora.indexer(inp, scores_cols=max(1, int(hi.max())))
    tol = lambda s: ATOL + rtol_of(inp) * np.abs(s)
    for r in range(rows_of(p)):
        n = int((sidx[r] >= 0).sum())
        s = osc[r, sidx[r, :n]]
        assert np.all(s[:-1] >= s[1:] - tol(s[1:]) - tol(s[:-1])), "row %d: order against the oracle" % r
        # where the oracle's scores are well separated, the positions agree with the oracle's own ranking
        sep = np.abs(np.diff(osc[r, oidx[r, :n]])) > 4 * tol(osc[r, oidx[r, 1:n]]) if n > 1 else np.zeros(0, bool)
        if n and np.all(sep):
            assert np.array_equal(sidx[r, :n], oidx[r, :n])


def test_sorted_output_bounded(ora):
    """The bounded path orders its outputs the same way (bit-identical to the
    planned sorted run)."""
    import torch
    inp, dev, _, bound, lens = bounded_case("int8_s4_merges")
    p = dict(inp["problem"], sort_output=1)
    inp = dict(inp, problem=p)
    bix = qli_mod().BoundedIndexer(p, bound)
    aslk = torch.tensor(lens, dtype=torch.int32, device="cuda")
    idx, val = bix.alloc_outputs()
    bix.run(aslk, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
            idx, val)
    torch.cuda.synchronize()
    p_idx, p_val = planned(inp, dev, lens)
    assert np.array_equal(idx.cpu().numpy(), p_idx) and np.array_equal(val.cpu().numpy(), p_val)
    rows = p_idx.shape[0]
    assert any(np.any(np.diff(p_idx[r][p_idx[r] >= 0]) < 0) for r in range(rows))   # really reordered


def test_negative_query_scale_follows_the_documented_reading(ora):
    """Out of contract: negative dequant scales.  The kernels fold ScaleQ into W
    and take ScaleK out of the ReLU, so they compute
    sum_g W_g ScaleQ_g ScaleK relu(dot_g), which equals the page's
    sum_g W_g relu(ScaleQ_g ScaleK dot_g) only for non-negative scales.  This
    test pins that documented behaviour: with some ScaleQ negated, the GPU's
    scores match the factored form (from the exact int8 dots), and differ from
    the literal formula that the oracle evaluates."""
    import torch
    spec = synth.small(batch=1, s1=1, aslk=[256], block_size=64, sparse_count=256)
    inp = synth.make_inputs(spec, 41)
    inp["q_scale"][0, ::3] = -inp["q_scale"][0, ::3]
    p = inp["problem"]
    ix = make_indexer(inp)
    dev = device_inputs(inp)
    _, _, dots, scores = ix.run_debug(dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"],
                                      dev["block_table"], 0, 1, 256)
    torch.cuda.synchronize()
    dots, scores = dots.cpu().numpy()[0].astype(np.float64), scores.cpu().numpy()[0].astype(np.float64)
    w = inp["weights"][0].astype(np.float64)
    sq = inp["q_scale"][0].astype(np.float64)
    blk = inp["block_table"][0]
    sk = np.array([float(inp["k_scale"][blk[j // 64], j % 64]) for j in range(256)])
    terms = (w * sq)[:, None] * np.maximum(dots, 0.0) * sk[None, :]
    factored = terms.sum(axis=0)
    # fp32 accumulation: error relative to the sum of the terms' magnitudes (they now cancel)
    assert np.all(np.abs(scores - factored) <= ATOL + INT8_RTOL * np.abs(terms).sum(axis=0))
    _, odots, literal = ora.row_detail(inp, 0, 0, 256)
    assert np.array_equal(odots, dots)
    assert np.max(np.abs(literal - factored)) > 1e-2 * np.max(np.abs(literal))


@pytest.mark.parametrize("i", range(12))
def test_parity_random_windowed(ora, i):
    """Seeded random problems with random pre/next_tokens windows (and, for
    half of them, score-ordered output) against the oracle on every row."""
    import dataclasses
    rng = np.random.default_rng(777 + i)
    spec = dataclasses.replace(random_spec(200 + i),
                               pre_tokens=int(rng.choice([0, 1, 7, 100, 1000, 5000, synth.INT64_MAX])),
                               next_tokens=int(rng.choice([0, 3, 50, synth.INT64_MAX])))
    inp = synth.make_inputs(spec, i)
    p = inp["problem"]
    log("random windowed %d: %s" % (i, spec))
    dev = device_inputs(inp)
    gidx, gval, _ = run_gpu(inp, dev)
    check_windowed(ora, inp, gidx, gval)
    if i % 2:
        sidx, sval, _ = run_gpu(dict(inp, problem=dict(p, sort_output=1)), dev)
        want_i, want_v = by_score(gidx, gval)
        assert np.array_equal(sidx, want_i) and np.array_equal(sval, want_v)
