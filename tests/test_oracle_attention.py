"""Pins for the sparse-attention oracle (the consumer of sparse_indices).

Reading (VllmQuantLightningIndexer page, 功能说明 step 3: the Top-k indices
are the input of Attention; 参数说明 sparse_indices / block_table): softmax
attention of each query head over the listed entries of its batch's paged
key / value caches.  Each pin fixes a part a plausible mistake would break:
brute force with Python floats, dense attention from torch's
scaled_dot_product_attention when every visible entry is listed, closed
forms (one entry, zero scale), invariances (list order, -1 padding, paging,
TND = BSND), and overflow-free large logits.
"""
import math

import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def aor():
    import oracle.attention as oa
    return oa.get()


def bf16(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def gather(a, b, j):
    """Entry j of batch b (key, value) as float64 vectors, walked in Python."""
    bs = a["block_size"]
    stride = a["kv_stride"] or bs * 128
    blk = int(a["block_table"][b, j // bs])
    off = blk * stride + (j % bs) * 128
    return bf16(a["k_cache"][off:off + 128]), bf16(a["v_cache"][off:off + 128])


def batch_of_row(a, r):
    if a["layout"] == synth.BSND:
        return r // a["s1"]
    for b, e in enumerate(a["aslq"]):
        if r < e:
            return b
    return -1


def brute(a, r, h):
    """Python floats and math.exp, one listed entry at a time."""
    b = batch_of_row(a, r)
    q = bf16(a["q"][r, h])
    logits, vals = [], []
    for j in a["indices"][r]:
        if j < 0 or b < 0:
            continue
        k, v = gather(a, b, int(j))
        logits.append(a["scale"] * math.fsum(q * k))
        vals.append(v)
    if not logits:
        return np.zeros(128), -math.inf
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    l = math.fsum(w)
    out = np.array([math.fsum(wi * v[d] for wi, v in zip(w, vals)) / l for d in range(128)])
    return out, m + math.log(l)


def small_inputs(seed=0, layout=synth.BSND, heads=4, **kw):
    base = dict(batch=2, s1=3, aslk=[200, 77], block_size=32, sparse_count=24)
    base.update(kw)
    if layout == synth.TND:
        base.setdefault("aslq", [2, 5])
    inp = synth.make_inputs(synth.small(layout=layout, **base), seed)
    return inp, synth.attention_inputs(inp, heads, seed + 100)


def test_bf16_decoding(aor):
    import torch
    codes = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([aor.bf16_value(int(c)) for c in codes])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


@pytest.mark.parametrize("layout", [synth.BSND, synth.TND])
def test_brute_force(aor, layout):
    inp, a = small_inputs(1, layout)
    a["indices"][1, 5:9] = -1          # holes in a list
    rc, out, lse = aor.attention(a)
    assert rc == 0
    for r in range(a["q"].shape[0]):
        for h in range(a["heads"]):
            ref, rl = brute(a, r, h)
            np.testing.assert_allclose(out[r, h], ref, rtol=1e-12, atol=1e-14)
            assert (rl == -math.inf and lse[r, h] == -math.inf) or abs(lse[r, h] - rl) <= 1e-12 * abs(rl)


def test_dense_causal_equals_sdpa(aor):
    """Every visible entry listed (sparse_count >= the visible count): the
    consumer is dense bottom-right-causal attention, which torch computes in
    float64 (scaled_dot_product_attention with an explicit mask)."""
    import torch
    import torch.nn.functional as F
    spec = synth.small(batch=2, s1=4, aslk=[40, 19], block_size=16, sparse_count=64, sparse_mode=3)
    inp = synth.make_inputs(spec, 2)
    rows, heads = 8, 3
    idx = np.full((rows, 64), -1, np.int32)
    for b in range(2):
        n = int(inp["aslk"][b])
        for i in range(4):
            vis = n - 4 + i + 1                      # bottom-right causal
            idx[b * 4 + i, :vis] = np.arange(vis)
    a = synth.attention_inputs(inp, heads, 3, indices=idx)
    rc, out, lse = aor.attention(a)
    assert rc == 0
    for b in range(2):
        n = int(inp["aslk"][b])
        K = np.stack([gather(a, b, j)[0] for j in range(n)])
        V = np.stack([gather(a, b, j)[1] for j in range(n)])
        Q = bf16(a["q"][b * 4:(b + 1) * 4]).transpose(1, 0, 2)          # [heads, 4, 128]
        mask = np.zeros((4, n), dtype=bool)
        for i in range(4):
            mask[i, :n - 4 + i + 1] = True
        ref = F.scaled_dot_product_attention(torch.from_numpy(Q), torch.from_numpy(K)[None].expand(heads, n, 128),
                                             torch.from_numpy(V)[None].expand(heads, n, 128),
                                             attn_mask=torch.from_numpy(mask), scale=a["scale"]).numpy()
        np.testing.assert_allclose(out[b * 4:(b + 1) * 4], ref.transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
        logits = np.einsum("hid,jd->hij", Q, K) * a["scale"]
        logits[:, ~mask] = -np.inf
        ref_lse = torch.logsumexp(torch.from_numpy(logits), dim=-1).numpy().T
        np.testing.assert_allclose(lse[b * 4:(b + 1) * 4], ref_lse, rtol=1e-12)


def test_single_entry_and_zero_scale(aor):
    """One listed entry: out = its value row exactly, lse = its logit.  Zero
    scale: uniform weights, out = the mean of the listed value rows, lse =
    log(count)."""
    inp, a = small_inputs(4)
    a["indices"][:] = -1
    a["indices"][0, 7] = 11
    rc, out, lse = aor.attention(a)
    k, v = gather(a, 0, 11)
    for h in range(a["heads"]):
        assert np.array_equal(out[0, h], v)
        assert lse[0, h] == a["scale"] * math.fsum(bf16(a["q"][0, h]) * k)
    assert np.all(out[1:] == 0) and np.all(lse[1:] == -np.inf)
    _, a = small_inputs(5)
    a["scale"] = 0.0
    rc, out, lse = aor.attention(a)
    for r in (0, 4):
        b = batch_of_row(a, r)
        lst = [int(j) for j in a["indices"][r] if j >= 0]
        mean = np.mean([gather(a, b, j)[1] for j in lst], axis=0)
        np.testing.assert_allclose(out[r, 2], mean, rtol=1e-12, atol=1e-14)
        assert abs(lse[r, 2] - math.log(len(lst))) < 1e-12


def test_list_order_and_padding(aor):
    inp, a = small_inputs(6)
    rc, out0, lse0 = aor.attention(a)
    rng = np.random.default_rng(0)
    b = dict(a, indices=a["indices"].copy())
    for r in range(b["indices"].shape[0]):
        n = int((b["indices"][r] >= 0).sum())
        b["indices"][r, :n] = rng.permutation(b["indices"][r, :n])
    _, out1, lse1 = aor.attention(b)
    np.testing.assert_allclose(out1, out0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse1, lse0, rtol=1e-13)
    c = dict(a, indices=np.full((a["indices"].shape[0], 40), -1, np.int32))
    c["indices"][:, ::2][:, :20] = a["indices"][:, :20]     # -1 between every listed entry
    c["indices"] = np.ascontiguousarray(c["indices"])
    d = dict(a, indices=np.ascontiguousarray(a["indices"][:, :20]))
    _, out2, lse2 = aor.attention(c)
    _, out3, lse3 = aor.attention(d)
    assert np.array_equal(out2, out3) and np.array_equal(lse2, lse3)


def test_paging_and_layout_invariance(aor):
    """A padded block stride, and TND with equal lengths, give the BSND
    contiguous result exactly."""
    inp, a = small_inputs(7, batch=2, s1=3, aslk=[150, 150])
    _, out0, lse0 = aor.attention(a)
    pad = synth.attention_inputs(inp, a["heads"], 107, indices=a["indices"], kv_stride_pad=96)
    assert pad["kv_stride"] == 32 * 128 + 96
    st = pad["kv_stride"]
    for name in ("k_cache", "v_cache"):                   # same values, padded layout
        src = a[name].reshape(-1, 32 * 128)
        dst = pad[name].reshape(-1, st)
        dst[:, :32 * 128] = src
    pad["q"] = a["q"]
    _, out1, lse1 = aor.attention(pad)
    assert np.array_equal(out1, out0) and np.array_equal(lse1, lse0)
    tnd = dict(a, layout=synth.TND, s1=6, aslq=np.array([3, 6], np.int32))
    _, out2, lse2 = aor.attention(tnd)
    assert np.array_equal(out2, out0) and np.array_equal(lse2, lse0)


def test_large_logits_stay_finite(aor):
    """Logits in the thousands: the max is subtracted before exp."""
    inp, a = small_inputs(8)
    a["scale"] = 400.0
    rc, out, lse = aor.attention(a)
    assert rc == 0 and np.all(np.isfinite(out)) and np.all(np.isfinite(lse[lse > -np.inf]))
    for r, h in ((0, 0), (4, 3)):
        ref, rl = brute(a, r, h)
        np.testing.assert_allclose(out[r, h], ref, rtol=1e-9, atol=1e-12)
        assert abs(lse[r, h] - rl) <= 1e-12 * abs(rl)
        assert np.max(np.abs(lse[r])) > 500.0


def test_rejects_entries_past_the_table(aor):
    inp, a = small_inputs(9)
    a["indices"][0, 0] = a["max_blocks"] * a["block_size"]
    rc, _, _ = aor.attention(a)
    assert rc == 1
