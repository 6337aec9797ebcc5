"""GPU parity of the sparse-attention consumer (qli_sparse_attention, through
the C ABI) against the fp64 oracle (oracle/attention_oracle.c).

Tolerance, derived from the arithmetic (bf16 inputs; fp32 logits, softmax and
accumulation; the probabilities rounded to bf16 for the PV product; the
output rounded to bf16):
  * out:  |gpu - oracle| <= 2^-7 * (vmax + |oracle|) + 1e-6, with vmax the
    largest |V| over the row's listed entries -- rounding each probability to
    bf16 (relative 2^-8) moves the output by at most 2^-8 vmax, rounding the
    output by 2^-8 |out|; the factor 2 covers the fp32 parts;
  * lse:  |gpu - oracle| <= 1e-3 + 1e-5 |oracle| (fp32 logits and sums),
    -inf exactly where the row lists nothing;
  * uniform weights (a softmax scale so small that every probability is 1.0
    in fp32 and bf16): out is the mean of the listed value rows, within the
    output rounding alone, 2^-8 |oracle| + 1e-6 vmax -- this pins every
    gathered entry.
"""
import numpy as np
import pytest

import synth
from tests._gpu import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    import sparse_attention_token_paged_amd as qli
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qli.load()


@pytest.fixture(scope="module")
def aor():
    import oracle.attention as oa
    return oa.get()


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attn_problem(a, return_lse=1):
    return dict(batch=a["batch"], s1=a["s1"], layout_query=a["layout"], num_heads=a["heads"], head_dim=128,
                num_blocks=a["num_blocks"], block_size=a["block_size"], max_blocks_per_seq=a["max_blocks"],
                kv_block_stride=a["kv_stride"], sparse_count=a["indices"].shape[1], softmax_scale=a["scale"],
                return_lse=return_lse)


def run_gpu(a, indices=None):
    import torch
    import sparse_attention_token_paged_amd as qli
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    att = qli.SparseAttention(attn_problem(a))
    aslq = t(np.asarray(a["aslq"], dtype=np.int32)) if a["layout"] == synth.TND else None
    out, lse = att.run(t(a["q"].view(np.int16)), t(a["k_cache"].view(np.int16)), t(a["v_cache"].view(np.int16)),
                       t(a["block_table"]), t(a["indices"] if indices is None else indices), aslq_dev=aslq)
    torch.cuda.synchronize()
    return bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16)), lse.cpu().numpy().astype(np.float64)


def listed_vmax(a):
    """Largest |V| over each row's listed entries (0 for an empty list)."""
    rows = a["q"].shape[0]
    bs = a["block_size"]
    stride = a["kv_stride"] or bs * 128
    v = bf16_to_f64(a["v_cache"])
    if a["layout"] == synth.BSND:
        batch_of = np.arange(rows) // a["s1"]
    else:
        batch_of = np.searchsorted(np.asarray(a["aslq"]), np.arange(rows), side="right")
    out = np.zeros(rows)
    for r in range(rows):
        js = a["indices"][r]
        js = js[js >= 0]
        if js.size == 0 or batch_of[r] >= a["batch"]:
            continue
        blk = a["block_table"][batch_of[r], js // bs].astype(np.int64)
        offs = blk * stride + (js % bs) * 128
        out[r] = np.max(np.abs(v[offs[:, None] + np.arange(128)[None, :]]))
    return out


def check(a, out, lse, ref, ref_lse, uniform=False):
    vmax = listed_vmax(a)[:, None, None]
    err = np.abs(out - ref)
    if uniform:
        tol = 2.0 ** -8 * np.abs(ref) + 1e-6 * vmax
    else:
        tol = 2.0 ** -7 * (vmax + np.abs(ref)) + 1e-6
    bad = err > tol
    assert not bad.any(), "%d outputs out of tolerance, worst at %s: gpu %r oracle %r" % (
        bad.sum(), np.unravel_index(np.argmax(err - tol), err.shape), out.flat[np.argmax(err - tol)],
        ref.flat[np.argmax(err - tol)])
    empty = ref_lse == -np.inf
    assert np.all(lse[empty] == -np.inf), "rows that list nothing must give lse = -inf"
    assert np.all(out[np.broadcast_to(empty[:, :, None], out.shape)] == 0.0)
    d = np.abs(lse[~empty] - ref_lse[~empty])
    assert np.all(d <= 1e-3 + 1e-5 * np.abs(ref_lse[~empty])), "lse worst %r" % d.max()


def compare(aor, a, uniform=False):
    out, lse = run_gpu(a)
    rc, ref, ref_lse = aor.attention(a)
    assert rc == 0
    check(a, out, lse, ref, ref_lse, uniform)
    return out, lse


CASES = {
    # (indexer-shaped spec, heads, kv stride pad); lists drawn by synth (ascending, -1 padded)
    "bsnd_h64_split": (synth.small(batch=2, s1=2, aslk=[3000, 1700], block_size=64, sparse_count=1024), 64, 0),
    "bsnd_h128_bs16_pad": (synth.small(batch=3, s1=1, aslk=[900, 60, 2500], block_size=16, sparse_count=700),
                           128, 24),
    "bsnd_h16_bs48": (synth.small(batch=2, s1=3, aslk=[500, 777], block_size=48, sparse_count=300), 16, 0),
    "bsnd_h32_k2048": (synth.small(batch=1, s1=2, aslk=[5000], block_size=256, sparse_count=2048), 32, 8),
    "tnd_h64_many_rows": (synth.small(layout=synth.TND, batch=3, s1=600, aslq=[200, 450, 590],
                                      aslk=[300, 2000, 90], block_size=32, sparse_count=128), 64, 0),
    "bsnd_h64_k1": (synth.small(batch=4, s1=1, aslk=[40, 1, 0, 900], block_size=16, sparse_count=1), 64, 0),
    "bsnd_h64_bs1024": (synth.small(batch=2, s1=2, aslk=[3000, 1500], block_size=1024, sparse_count=512), 64, 0),
    "bsnd_h64_ragged_tail": (synth.small(batch=2, s1=1, aslk=[1000, 97], block_size=64, sparse_count=97), 64, 0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_parity_small(aor, name):
    spec, heads, pad = CASES[name]
    inp = synth.make_inputs(spec, 3)
    a = synth.attention_inputs(inp, heads, 41, kv_stride_pad=pad)
    log("attention %s: rows %d heads %d k %d" % (name, a["q"].shape[0], heads, a["indices"].shape[1]))
    compare(aor, a)


@pytest.mark.parametrize("name", ["bsnd_h64_split", "bsnd_h128_bs16_pad", "tnd_h64_many_rows", "bsnd_h32_k2048"])
def test_uniform_weights_pin_every_entry(aor, name):
    """softmax_scale 1e-30: every probability is exactly 1, so out is the mean of
    the listed value rows to within the output rounding."""
    spec, heads, pad = CASES[name]
    inp = synth.make_inputs(spec, 5)
    a = synth.attention_inputs(inp, heads, 43, kv_stride_pad=pad, scale=1e-30)
    compare(aor, a, uniform=True)


def test_peaked_softmax(aor):
    """A large scale: one entry dominates each head's row, so a wrong gather
    shows at full size."""
    spec, heads, pad = CASES["bsnd_h64_split"]
    inp = synth.make_inputs(spec, 6)
    a = synth.attention_inputs(inp, heads, 44, scale=2.0)
    compare(aor, a)


def test_holes_invalid_and_empty_rows(aor):
    """-1 between listed entries, entries past the block table and on an
    unused block-table slot (skipped by the kernel: compared with the oracle on
    the list with them replaced by -1), rows listing nothing, TND rows past the
    last prefix sum."""
    spec = synth.small(layout=synth.TND, batch=2, s1=40, aslq=[15, 33], aslk=[700, 200], block_size=32,
                       sparse_count=256)
    inp = synth.make_inputs(spec, 7)
    a = synth.attention_inputs(inp, 64, 45)
    idx = a["indices"]
    idx[:, 1::3] = -1
    idx[3, :] = -1                                      # an empty row of batch 0
    bad = idx.copy()
    jmax = a["max_blocks"] * a["block_size"]
    bad[0, 0] = jmax + 5                               # past the block table
    idx[0, 0] = -1
    bad[20, 2] = 250                                    # batch 1 stores 200 entries: slot 7 of its table is -1
    idx[20, 2] = -1
    assert a["block_table"][1, 250 // 32] == -1
    out, lse = run_gpu(a, indices=bad)
    rc, ref, ref_lse = aor.attention(a)               # the same lists with the skipped entries as -1
    assert rc == 0
    check(a, out, lse, ref, ref_lse)
    assert np.all(lse[33:] == -np.inf) and np.all(out[33:] == 0)
    assert np.all(lse[3] == -np.inf)


def test_full_size_decode_shape(aor):
    """The headline decode shape (24 sequences x 4 query tokens, 8192 entries,
    block 128, permuted table), 64 heads, 2048 listed entries per row: every
    row against the oracle."""
    import time
    inp = synth.workload("decode_int8_b24_s4_sk8192")
    a = synth.attention_inputs(inp, 64, 46)
    log("attention full size: rows %d" % a["q"].shape[0])
    out, lse = run_gpu(a)
    t0 = time.perf_counter()
    rc, ref, ref_lse = aor.attention(a)
    assert rc == 0
    log("  oracle %.1f s" % (time.perf_counter() - t0))
    check(a, out, lse, ref, ref_lse)


def test_indexer_output_feeds_the_consumer(aor):
    """The indexer's own sparse_indices (GPU) as the consumer's lists."""
    import torch
    import sparse_attention_token_paged_amd as qli
    from tests._gpu import device_inputs
    spec = synth.small(batch=3, s1=4, aslk=[3000, 1200, 2500], block_size=64, sparse_count=512, sparse_mode=3)
    inp = synth.make_inputs(spec, 8)
    ix = qli.Indexer(inp["problem"], inp["aslq"], inp["aslk"])
    dev = device_inputs(inp)
    gidx, _ = ix.run(dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"])
    torch.cuda.synchronize()
    a = synth.attention_inputs(inp, 64, 47, indices=gidx.cpu().numpy())
    compare(aor, a)


def test_graph_replay_with_new_lists(aor):
    """qli_sparse_attention captured once in a HIP graph; the device lists
    change between replays; every replay matches the oracle and the eager run."""
    import torch
    import sparse_attention_token_paged_amd as qli
    spec, heads, _ = CASES["bsnd_h64_split"]
    inp = synth.make_inputs(spec, 9)
    a = synth.attention_inputs(inp, heads, 48)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    att = qli.SparseAttention(attn_problem(a))
    q, kc, vc, bt = (t(a["q"].view(np.int16)), t(a["k_cache"].view(np.int16)), t(a["v_cache"].view(np.int16)),
                     t(a["block_table"]))
    idx = t(a["indices"])
    out, lse = att.alloc_outputs()
    att.run(q, kc, vc, bt, idx, out, lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        att.run(q, kc, vc, bt, idx, out, lse)
    for rep in range(3):
        b = synth.attention_inputs(inp, heads, 48, indices=None)
        b["q"], b["k_cache"], b["v_cache"] = a["q"], a["k_cache"], a["v_cache"]
        rng = np.random.default_rng(rep)
        b["indices"] = np.ascontiguousarray(np.where(rng.random(b["indices"].shape) < 0.2, -1, b["indices"]),
                                            dtype=np.int32)
        idx.copy_(t(b["indices"]))
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        go = bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))
        gl = lse.cpu().numpy().astype(np.float64)
        rc, ref, ref_lse = aor.attention(b)
        assert rc == 0
        check(b, go, gl, ref, ref_lse)
        e_out, e_lse = att.run(q, kc, vc, bt, idx)
        torch.cuda.synchronize()
        assert np.array_equal(e_out.view(torch.int16).cpu().numpy(), out.view(torch.int16).cpu().numpy())
