"""Pins of the producer oracle (oracle/quantize.py): per-token-head
quantization of the index query and key.

What fixes it independently of its own code: torch's float32 -> float8_e4m3fn
conversion (a library routine, round to nearest even) for the e4m3fn
encoder; closed forms (one non-zero value quantizes to the extreme code, a
zero row to zeros with scale 0, a constant row to +-127 / +-448);
the rounding bound |x*r - q| <= 1/2 of a symmetric quantizer; invariances
(sign flips the codes, a power-of-two factor scales s and keeps the codes);
and paging invariance of the key append (a permuted block table with
permuted physical blocks, or a padded stride, holds the same entries).
"""
import numpy as np
import pytest

from oracle import quantize as oq

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs here are
    chosen representable, so this is exact where it matters)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def test_bf16_decode_is_top_half_of_fp32():
    vals = np.array([0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-40, 65504.0], dtype=np.float32)
    bits = bf16_bits(vals)
    back = oq.bf16_to_f32(bits)
    torch = pytest.importorskip("torch")
    ref = torch.tensor(vals).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(back.view(np.uint32), ref.view(np.uint32))


def test_e4m3fn_encoder_matches_torch():
    torch = pytest.importorskip("torch")
    tab = oq.e4m3fn_magnitudes()
    assert tab[0] == 0.0 and tab[-1] == 448.0 and len(tab) == 127
    mids = (tab[:-1] + tab[1:]) / 2  # exact ties (representable in fp32)
    rng = np.random.default_rng(0)
    rand = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.02, 0.02, 20000),
                           np.exp2(rng.uniform(-12, 8.8, 20000)) * rng.choice([-1, 1], 20000)])
    rand = np.clip(rand, -448, 448)
    y = np.concatenate([tab, -tab, mids, -mids, rand]).astype(np.float32)
    ours = oq.e4m3fn_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = ours != ref
    assert not bad.any(), (y[bad][:5], ours[bad][:5], ref[bad][:5])


def test_e4m3fn_encoder_keeps_sign_of_zero():
    y = np.array([0.0, -0.0, -1e-9, 1e-9], dtype=np.float32)
    assert list(oq.e4m3fn_encode(y)) == [0x00, 0x80, 0x80, 0x00]


@pytest.mark.parametrize("qk", [0, 1])
def test_single_spike_takes_the_extreme_code(qk):
    rng = np.random.default_rng(1)
    for v in [1.0, -3.5, 1e-3, -7.0e4, 2.0 ** -100, 1e30]:
        x = np.zeros((1, 128), np.float32)
        j = int(rng.integers(128))
        x[0, j] = v
        codes, s = oq.quantize_rows(bf16_bits(x), qk)
        vb = float(oq.bf16_to_f32(bf16_bits(np.float32(v))))
        others = np.delete(codes[0], j)
        if qk == 0:
            s_ref = np.float16(np.float32(abs(vb)) / np.float32(127))
            if np.isinf(s_ref):
                s_ref = np.float16(65504)
            assert s[0] == s_ref
            if s_ref == 0:
                assert not codes.any()
                continue
            assert int(np.int8(codes[0, j].astype(np.int8))) == (127 if vb > 0 else -127)
            assert not others.any()
        else:
            assert s[0] == np.float32(np.float32(abs(vb)) / np.float32(448))
            r = np.float32(1) / s[0]
            if not np.isfinite(r):
                assert not codes.any()
                continue
            assert codes[0, j] == (0x7E if vb > 0 else 0xFE)
            assert not others.any()


@pytest.mark.parametrize("qk", [0, 1])
def test_zero_and_constant_rows(qk):
    x = np.zeros((3, 128), np.float32)
    x[1] = 2.75
    x[2] = -0.1
    codes, s = oq.quantize_rows(bf16_bits(x), qk)
    assert s[0] == 0 and not codes[0].any()
    top = 127 if qk == 0 else 0x7E
    neg = np.uint8(np.int8(-127).view(np.uint8)) if qk == 0 else 0xFE
    assert np.all(codes[1] == top) and np.all(codes[2] == neg)


def test_int8_rounding_bound_and_clamp():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((400, 128)) * np.exp2(rng.uniform(-20, 20, (400, 1)))).astype(np.float32)
    xb = bf16_bits(x)
    xf = oq.bf16_to_f32(xb).reshape(-1, 128)
    codes, s = oq.quantize_rows(xb, 0)
    q = codes.view(np.int8).astype(np.float64)
    for i in range(x.shape[0]):
        if s[i] == 0:  # amax / 127 underflows fp16: every code is 0 by definition
            assert not codes[i].any()
            continue
        r = np.float32(1) / np.float32(s[i])
        y = (xf[i] * r).astype(np.float64)
        inside = np.abs(y) <= 127
        assert np.all(np.abs(y[inside] - q[i, inside]) <= 0.5)
        assert np.all(np.abs(q[i, ~inside]) == 127) and np.all(np.sign(q[i, ~inside]) == np.sign(y[~inside]))
        # with a normal fp16 scale (relative rounding <= 2^-11) the extreme element lands on
        # +-127 or +-126; a subnormal scale carries fewer bits and may land lower
        if s[i] >= np.float16(2.0 ** -14):
            assert np.max(np.abs(q[i])) >= 126


def test_e4m3_dequant_error_within_half_spacing():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((200, 128)) * np.exp2(rng.uniform(-30, 30, (200, 1)))).astype(np.float32)
    xb = bf16_bits(x)
    xf = oq.bf16_to_f32(xb).reshape(-1, 128).astype(np.float64)
    codes, s = oq.quantize_rows(xb, 1)
    tab = oq.e4m3fn_magnitudes()
    for i in range(x.shape[0]):
        r = np.float32(1) / s[i]
        y = np.clip((oq.bf16_to_f32(xb[i]) * r).astype(np.float64), -448, 448)
        val = tab[codes[i] & 0x7F] * np.where(codes[i] & 0x80, -1.0, 1.0)
        # nearest representable: no table value is closer to |y|
        best = np.min(np.abs(np.abs(y)[:, None] - tab[None, :]), axis=1)
        assert np.allclose(np.abs(np.abs(y) - np.abs(val)), best, rtol=0, atol=0)


@pytest.mark.parametrize("qk", [0, 1])
def test_sign_and_power_of_two_invariance(qk):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((50, 128)) * 3.0).astype(np.float32)
    xb = bf16_bits(x)
    c0, s0 = oq.quantize_rows(xb, qk)
    c1, s1 = oq.quantize_rows(xb ^ np.uint16(0x8000), qk)  # negate every value
    assert np.array_equal(s0, s1)
    if qk == 0:
        assert np.array_equal(c1.view(np.int8), -c0.view(np.int8))
    else:
        nz = (c0 & 0x7F) != 0
        assert np.array_equal(c1[nz], c0[nz] ^ 0x80)
    c2, s2 = oq.quantize_rows(bf16_bits(oq.bf16_to_f32(xb) * np.float32(8.0)), qk)
    assert np.array_equal(c2, c0)
    assert np.array_equal(s2.astype(np.float64), s0.astype(np.float64) * 8.0)


def test_int8_scale_saturates_at_fp16_max():
    x = np.full((1, 128), 3.0e38, np.float32)
    x[0, 5] = 1.0
    x[0, 64:] = -3.0e38
    codes, s = oq.quantize_rows(bf16_bits(x), 0)
    assert s[0] == np.float16(65504)
    q = codes.view(np.int8)[0]
    assert q[5] == 0 and np.all(q[:5] == 127) and np.all(q[6:64] == 127) and np.all(q[64:] == -127)


def _cache(num_blocks, bs, stride, qk):
    kc = np.full(num_blocks * stride, 0xA5, np.uint8)
    ks = np.full(num_blocks * bs, 7, np.float16 if qk == 0 else np.float32)
    return kc, ks


@pytest.mark.parametrize("qk", [0, 1])
def test_append_paging_invariance_and_skips(qk):
    rng = np.random.default_rng(5)
    B, bs, mb = 3, 32, 4
    nb = B * mb
    n = 200
    x = bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    bidx = rng.integers(0, B, n).astype(np.int32)
    pos = rng.permutation(np.arange(B * mb * bs))[:n].astype(np.int32) % (mb * bs)
    # distinct (batch, pos) slots
    keys = {}
    for e in range(n):
        keys[(int(bidx[e]), int(pos[e]))] = e
    sel = np.array(sorted(keys.values()), dtype=np.int64)
    x, bidx, pos = x[sel], bidx[sel], pos[sel]
    n = len(sel)
    ident = np.arange(nb, dtype=np.int32).reshape(B, mb)
    perm = rng.permutation(nb).astype(np.int32)
    permuted = perm[ident]
    kc_i, ks_i = _cache(nb, bs, bs * 128, qk)
    oq.append_keys(x, bidx, pos, ident, B, mb, nb, bs, bs * 128, kc_i, ks_i, qk)
    kc_p, ks_p = _cache(nb, bs, bs * 128 + 64, qk)
    oq.append_keys(x, bidx, pos, permuted, B, mb, nb, bs, bs * 128 + 64, kc_p, ks_p, qk)
    for b in range(B):
        for j in range(mb):
            li, lp = ident[b, j], permuted[b, j]
            a = kc_i[li * bs * 128:(li + 1) * bs * 128]
            c = kc_p[lp * (bs * 128 + 64): lp * (bs * 128 + 64) + bs * 128]
            assert np.array_equal(a, c)
            assert np.array_equal(ks_i[li * bs:(li + 1) * bs], ks_p[lp * bs:(lp + 1) * bs])
    codes, scales = oq.quantize_rows(x, qk)
    for e in range(n):
        blk = ident[bidx[e], pos[e] // bs]
        o = pos[e] % bs
        assert np.array_equal(kc_i[blk * bs * 128 + o * 128: blk * bs * 128 + o * 128 + 128], codes[e])
        assert ks_i[blk * bs + o] == scales[e]
    # entries outside the cache are skipped: nothing changes
    kc_s, ks_s = _cache(nb, bs, bs * 128, qk)
    bad_b = np.array([-1, B, 0, 0, 2], np.int32)  # (0, mb * bs): one past the table row, whose next entry is valid
    bad_p = np.array([0, 0, -5, mb * bs, 3], np.int32)
    table = ident.copy()
    table[2, 0] = -1
    oq.append_keys(x[:5], bad_b, bad_p, table, B, mb, nb, bs, bs * 128, kc_s, ks_s, qk)
    ref_c, ref_s = _cache(nb, bs, bs * 128, qk)
    assert np.array_equal(kc_s, ref_c) and np.array_equal(ks_s, ref_s)
