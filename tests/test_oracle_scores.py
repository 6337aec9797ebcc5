"""Pins for the oracle's dot products and score formula.

Formula (VllmQuantLightningIndexer page, section 功能说明):
    out = Top-k{ [1]_{1xg} @ [ (W @ [1]_{1xSk}) (.) ReLU( (ScaleQ @ ScaleK^T) (.) (Q @ K^T) ) ] }
Each pin below fixes a part that a plausible mistake would break: the
hand-derived worked example, brute-force integer dots through the block
table, exact fp8 dots, closed forms, single-head and non-negative special
cases, the ReLU placement (inside W, outside the scales) and linearity.
"""
import math
import os

import numpy as np
import pytest

import synth
from tests._helpers import brute_dots_int, gather_batch, query_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_int8.txt")
GOLDEN_FP8 = os.path.join(os.path.dirname(__file__), "golden", "worked_example_fp8_f32.txt")


def load_worked_example():
    spec = synth.small(batch=1, s1=1, aslk=[3], block_size=16, sparse_count=2, table="identity")
    inp = synth.make_inputs(spec, 0)
    inp["query"][:] = 0
    inp["key"][:] = 0
    inp["q_scale"][:] = 1.0
    inp["k_scale"][:] = 1.0
    inp["weights"][:] = 1.0
    exp = {}
    with open(GOLDEN) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "q":
                inp["query"][0, int(t[1]), int(t[2])] = int(t[3])
            elif t[0] == "k":
                inp["key"][int(t[1]) * 128 + int(t[2])] = np.int8(int(t[3])).view(np.uint8)
            elif t[0] == "sq":
                inp["q_scale"][0, int(t[1])] = float(t[2])
            elif t[0] == "sk":
                inp["k_scale"].reshape(-1)[int(t[1])] = float(t[2])
            elif t[0] == "w":
                inp["weights"][0, int(t[1])] = float(t[2])
            elif t[0] == "dot":
                exp.setdefault("dot", {})[int(t[1])] = [float(x) for x in t[2:]]
            else:
                exp[t[0]] = [float(x) for x in t[1:]]
    return inp, exp


def load_worked_example_fp8():
    """The FLOAT8_e4m3fn + FLOAT32 worked example: codes written as given in
    the file (no encoder involved), fp32 scales and weights parsed from their
    exact decimal expansions."""
    spec = synth.small(qk=synth.FP8, batch=1, s1=1, aslk=[3], block_size=16, sparse_count=2, table="identity")
    inp = synth.make_inputs(spec, 0)
    assert inp["problem"]["scale_dtype"] == synth.F32
    inp["query"][:] = 0
    inp["key"][:] = 0
    inp["q_scale"][:] = 1.0
    inp["k_scale"][:] = 1.0
    inp["weights"][:] = 1.0
    exp, codes = {}, {}
    with open(GOLDEN_FP8) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "q":
                inp["query"][0, int(t[1]), int(t[2])] = int(t[3], 16)
                codes[int(t[3], 16)] = float(t[4])
            elif t[0] == "k":
                inp["key"][int(t[1]) * 128 + int(t[2])] = int(t[3], 16)
                codes[int(t[3], 16)] = float(t[4])
            elif t[0] in ("sq", "sk", "w"):
                v = np.float32(t[2])
                assert float(v) == float(t[2]), "listed fp32 values are exact"
                if t[0] == "sq":
                    inp["q_scale"][0, int(t[1])] = v
                elif t[0] == "sk":
                    inp["k_scale"].reshape(-1)[int(t[1])] = v
                else:
                    inp["weights"][0, int(t[1])] = v
            elif t[0] == "dot":
                exp.setdefault("dot", {})[int(t[1])] = [float(x) for x in t[2:]]
            else:
                exp[t[0]] = [float(x) for x in t[1:]]
    return inp, exp, codes


def test_worked_example(ora):
    inp, exp = load_worked_example()
    vis, dots, sc = ora.row_detail(inp, 0, 0, 3)
    assert vis == 3
    for g, row in exp["dot"].items():
        assert list(dots[g]) == row
    assert np.all(dots[2:] == 0)
    assert list(sc) == exp["score"]
    rc, idx, val, _ = ora.indexer(inp)
    assert rc == 0
    assert list(idx[0]) == [int(x) for x in exp["topk"]]
    assert list(val[0]) == [1.625, 0.46875]


def test_worked_example_fp8_f32(ora):
    """FLOAT8_e4m3fn codes with FLOAT32 weights and scales (values that fp16
    cannot hold): dots, fp64 scores, the top-2 and its fp32 values, all exact."""
    inp, exp, codes = load_worked_example_fp8()
    for c, v in codes.items():
        assert ora.e4m3fn_value(c) == v, "code 0x%02X" % c
    vis, dots, sc = ora.row_detail(inp, 0, 0, 3)
    assert vis == 3
    for g, row in exp["dot"].items():
        assert list(dots[g]) == row
    assert np.all(dots[2:] == 0)
    assert list(sc) == exp["score"]
    rc, idx, val, _ = ora.indexer(inp)
    assert rc == 0
    assert list(idx[0]) == [int(x) for x in exp["topk"]]
    assert list(val[0].astype(np.float64)) == exp["values"]


@pytest.mark.parametrize("stride_pad", [0, 48])
def test_int8_dots_brute_force(ora, stride_pad):
    spec = synth.small(batch=2, s1=2, aslk=[40, 23], block_size=16, sparse_count=8,
                       stride_pad=stride_pad, spare_blocks=3)
    inp = synth.make_inputs(spec, 11)
    for r, b in ((0, 0), (1, 0), (3, 1)):
        n = int(inp["aslk"][b])
        vis, dots, _ = ora.row_detail(inp, r, 0, n)
        assert vis == n
        ref = brute_dots_int(inp, r, b, n)
        assert np.array_equal(dots, np.array(ref, dtype=np.float64))


def test_int8_dot_closed_forms(ora):
    spec = synth.small(batch=1, s1=1, aslk=[48], block_size=16, sparse_count=4, table="identity")
    inp = synth.make_inputs(spec, 3)
    keys = inp["key"].view(np.int8).reshape(-1, 128)
    # one-hot query: dot = the key's element at that dim
    inp["query"][:] = 0
    for g in range(64):
        inp["query"][0, g, (7 * g + 5) % 128] = 1
    _, dots, _ = ora.row_detail(inp, 0, 0, 48)
    for g in range(64):
        assert np.array_equal(dots[g], keys[:48, (7 * g + 5) % 128].astype(np.float64))
    # constants: 128*a*b, and the extreme -128 * -128 * 128 = 2^21
    inp["query"][0] = -128
    keys[:48] = -128
    _, dots, _ = ora.row_detail(inp, 0, 0, 48)
    assert np.all(dots == 2097152.0)
    inp["query"][0] = 3
    keys[:48] = -7
    _, dots, _ = ora.row_detail(inp, 0, 0, 48)
    assert np.all(dots == 128 * 3 * -7)


def test_fp8_dots_exact(ora):
    spec = synth.small(qk=synth.FP8, batch=1, s1=1, aslk=[33], block_size=16, sparse_count=4)
    inp = synth.make_inputs(spec, 5)
    _, dots, _ = ora.row_detail(inp, 0, 0, 33)
    keys, _ = gather_batch(inp, 0, 33)
    q = query_values(inp, 0)
    for g in (0, 17, 63):
        for j in range(33):
            assert dots[g, j] == math.fsum(q[g] * keys[j])  # products are exact; fsum is the exact sum


def test_single_head_special_case(ora):
    """Only head h weighted: score_j = W_h * ReLU(SQ_h * SK_j * dot_hj)."""
    spec = synth.small(batch=1, s1=1, aslk=[64], block_size=32, sparse_count=8)
    inp = synth.make_inputs(spec, 8)
    h = 37
    inp["weights"][:] = 0
    inp["weights"][0, h] = 0.0078125
    _, sk = gather_batch(inp, 0, 64)
    dots = np.array(brute_dots_int(inp, 0, 0, 64)[h], dtype=np.float64)
    sq = float(inp["q_scale"][0, h])
    ref = 0.0078125 * np.maximum(0.0, sq * sk * dots)
    _, _, sc = ora.row_detail(inp, 0, 0, 64)
    np.testing.assert_allclose(sc, ref, rtol=1e-15, atol=0)
    assert np.any(dots < 0) and np.all(sc[dots < 0] == 0)


def test_nonnegative_inputs_reduce_to_gemv(ora):
    """q, k >= 0 and scales >= 0: ReLU is the identity and
    score_j = SK_j * K_j . (sum_g W_g SQ_g Q_g)  (one matrix-vector product)."""
    spec = synth.small(batch=1, s1=2, aslk=[96], block_size=32, sparse_count=8)
    inp = synth.make_inputs(spec, 9)
    inp["query"][:] = np.abs(inp["query"].astype(np.int16)).clip(0, 127).astype(np.int8)
    raw = inp["key"].view(np.int8)
    raw[:] = np.abs(raw.astype(np.int16)).clip(0, 127).astype(np.int8)
    keys, sk = gather_batch(inp, 0, 96)
    for r in (0, 1):
        q = query_values(inp, r)
        wq = inp["weights"][r].astype(np.float64) * inp["q_scale"][r].astype(np.float64)
        ref = sk * np.matmul(keys, np.matmul(wq, q))
        _, _, sc = ora.row_detail(inp, r, 0, 96)
        np.testing.assert_allclose(sc, ref, rtol=1e-12)


def test_relu_kills_anticorrelated_keys(ora):
    spec = synth.small(batch=1, s1=1, aslk=[32], block_size=16, sparse_count=4, table="identity")
    inp = synth.make_inputs(spec, 4)
    base = np.arange(128, dtype=np.int16) % 11 - 5
    base[base == 0] = 1
    inp["query"][0, :, :] = base.astype(np.int8)
    keys = inp["key"].view(np.int8).reshape(-1, 128)
    keys[:32] = (-base).astype(np.int8)
    keys[5] = base.astype(np.int8)                 # one correlated key
    _, _, sc = ora.row_detail(inp, 0, 0, 32)
    assert sc[5] > 0
    assert np.all(np.delete(sc, 5) == 0.0)


def test_weight_outside_relu_and_scale_inside(ora):
    """W multiplies after the ReLU (a negative W gives a negative score);
    the dequant scales multiply before it (a negative ScaleQ turns a positive
    dot into a zero term)."""
    spec = synth.small(batch=1, s1=1, aslk=[16], block_size=16, sparse_count=4, table="identity")
    inp = synth.make_inputs(spec, 6)
    inp["query"][:] = 0
    inp["query"][0, 3, 0] = 10
    keys = inp["key"].view(np.int8).reshape(-1, 128)
    keys[:16] = 0
    keys[:16, 0] = 2                               # dot_3 = 20 for every key
    inp["k_scale"][:] = 1.0
    inp["weights"][:] = 0
    inp["weights"][0, 3] = -0.5
    inp["q_scale"][0, 3] = 0.25
    _, _, sc = ora.row_detail(inp, 0, 0, 16)
    assert np.all(sc == -0.5 * 0.25 * 20)
    inp["weights"][0, 3] = 0.5
    inp["q_scale"][0, 3] = -0.25
    _, _, sc = ora.row_detail(inp, 0, 0, 16)
    assert np.all(sc == 0.0)


def test_linearity_in_weights_and_key_scale(ora):
    spec = synth.small(batch=1, s1=1, aslk=[50], block_size=16, sparse_count=4)
    inp = synth.make_inputs(spec, 12)
    inp["k_scale"][:] = np.maximum(inp["k_scale"], np.float16(0.01))  # halving stays exact (no subnormals)
    _, _, s0 = ora.row_detail(inp, 0, 0, 50)
    inp["weights"] *= np.float16(2.0)
    _, _, s1 = ora.row_detail(inp, 0, 0, 50)
    assert np.array_equal(s1, 2 * s0)
    inp["weights"] /= np.float16(2.0)
    inp["k_scale"] *= np.float16(0.5)
    _, _, s2 = ora.row_detail(inp, 0, 0, 50)
    assert np.array_equal(s2, 0.5 * s0)
    assert np.all(s0 >= 0)


def test_single_head_special_case_fp32(ora):
    """FLOAT8_e4m3fn with FLOAT32 scales, only head h weighted:
    score_j = W_h * ReLU(SQ_h * SK_j * dot_hj), with the dots summed exactly
    (math.fsum of the exact e4m3 products) and fp32 inputs that fp16 cannot
    represent (weights, ScaleQ and ScaleK with 24 significant bits)."""
    spec = synth.small(qk=synth.FP8, batch=2, s1=1, aslk=[70, 40], block_size=32, sparse_count=8)
    inp = synth.make_inputs(spec, 21)
    rng = np.random.default_rng(5)
    inp["q_scale"][:] = (1.0 + rng.integers(1, 1 << 23, size=inp["q_scale"].shape) * 2.0 ** -23).astype(np.float32)
    inp["k_scale"][:] = (rng.uniform(0.0, 10.0, size=inp["k_scale"].shape)).astype(np.float32)
    for r, b, h in ((0, 0, 37), (1, 1, 2)):
        n = int(inp["aslk"][b])
        inp["weights"][:] = 0
        inp["weights"][r, h] = np.float32(1.0 + 2.0 ** -20)
        keys, sk = gather_batch(inp, b, n)
        q = query_values(inp, r)
        dots = np.array([math.fsum(q[h] * keys[j]) for j in range(n)])
        sq = float(inp["q_scale"][r, h])
        ref = (1.0 + 2.0 ** -20) * np.maximum(0.0, (sq * sk) * dots)
        _, _, sc = ora.row_detail(inp, r, 0, n)
        np.testing.assert_allclose(sc, ref, rtol=1e-15, atol=0)
        assert np.any(dots < 0) and np.all(sc[dots < 0] == 0)
        assert np.any(sc > 0)


def test_nonnegative_inputs_reduce_to_gemv_fp32(ora):
    """FLOAT8_e4m3fn q, k >= 0 and FLOAT32 scales / weights >= 0: ReLU is the
    identity and score_j = SK_j * K_j . (sum_g W_g SQ_g Q_g), one
    matrix-vector product (numpy.matmul in fp64)."""
    spec = synth.small(qk=synth.FP8, batch=1, s1=2, aslk=[96], block_size=32, sparse_count=8)
    inp = synth.make_inputs(spec, 22)
    inp["query"][:] &= 0x7F     # clear the sign bit: |x| (uniform(-8, 8) never makes the NaN code)
    inp["key"][:] &= 0x7F
    rng = np.random.default_rng(6)
    inp["weights"][:] = rng.uniform(0.0, 0.01, size=inp["weights"].shape).astype(np.float32)
    keys, sk = gather_batch(inp, 0, 96)
    for r in (0, 1):
        q = query_values(inp, r)
        wq = inp["weights"][r].astype(np.float64) * inp["q_scale"][r].astype(np.float64)
        ref = sk * np.matmul(keys, np.matmul(wq, q))
        _, _, sc = ora.row_detail(inp, r, 0, 96)
        np.testing.assert_allclose(sc, ref, rtol=1e-12)


def test_linearity_fp32(ora):
    """FLOAT32 weights and key scales enter linearly: doubling W doubles
    every score, halving ScaleK halves it (exact in fp64)."""
    spec = synth.small(qk=synth.FP8, batch=1, s1=1, aslk=[50], block_size=16, sparse_count=4)
    inp = synth.make_inputs(spec, 23)
    _, _, s0 = ora.row_detail(inp, 0, 0, 50)
    inp["weights"] *= np.float32(2.0)
    _, _, s1 = ora.row_detail(inp, 0, 0, 50)
    assert np.array_equal(s1, 2 * s0)
    inp["weights"] /= np.float32(2.0)
    inp["k_scale"] *= np.float32(0.5)
    _, _, s2 = ora.row_detail(inp, 0, 0, 50)
    assert np.array_equal(s2, 0.5 * s0)
    assert np.all(s0 >= 0) and np.any(s0 > 0)
