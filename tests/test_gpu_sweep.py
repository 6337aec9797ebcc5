"""Extended seeded sweep of random problems against the oracle (GPU).

Hundreds of random problems drawn by the same generator as the parity tests'
random cases (dtype, layout, ragged and empty lengths, query counts, every
mode, cmp_ratio 1 to 16, block sizes 16 to 512, sparse_count 1 to 2048,
padded strides), half of them with a random pre/next_tokens window and, for
every other one, score-ordered output; every problem also runs without a host
plan (lengths and query counts on the device) and must equal the planned run
bit for bit where the tiles match.  Every row is checked against the oracle.

The sweep takes a few minutes, so it runs only when QLI_SWEEP is set (for
example QLI_SWEEP=400 for 400 problems); otherwise it is skipped.
"""
import dataclasses
import os

import numpy as np
import pytest

import synth
from tests._gpu import device_inputs, log, run_gpu
from tests.test_gpu_parity import by_score, check_windowed, qli_mod, random_spec

pytestmark = pytest.mark.gpu

N = int(os.environ.get("QLI_SWEEP", "0"))


@pytest.mark.skipif(N <= 0, reason="extended sweep: set QLI_SWEEP=<problems> to run it")
@pytest.mark.parametrize("i", range(max(N, 1)))
def test_sweep(ora, i):
    import torch
    rng = np.random.default_rng(90000 + i)
    spec = random_spec(50000 + i)
    windowed = rng.random() < 0.5
    if windowed:
        spec = dataclasses.replace(spec, pre_tokens=int(rng.choice([0, 1, 5, 64, 700, 4000, synth.INT64_MAX])),
                                   next_tokens=int(rng.choice([0, 2, 100, synth.INT64_MAX])))
    inp = synth.make_inputs(spec, 1000 + i)
    p = inp["problem"]
    log("sweep %d: %s" % (i, spec))
    dev = device_inputs(inp)
    gidx, gval, _ = run_gpu(inp, dev)
    check_windowed(ora, inp, gidx, gval)
    if i % 2:
        sidx, sval, _ = run_gpu(dict(inp, problem=dict(p, sort_output=1)), dev)
        want_i, want_v = by_score(gidx, gval)
        assert np.array_equal(sidx, want_i) and np.array_equal(sval, want_v)
    # every problem also without a host plan
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
        assert np.array_equal(idx, gidx) and np.array_equal(val, gval)
    check_windowed(ora, inp, idx, val)


@pytest.mark.skipif(N <= 0, reason="extended sweep: set QLI_SWEEP=<problems> to run it")
@pytest.mark.parametrize("i", range(max(N // 4, 1)))
def test_sweep_consumer(i):
    """The sparse-attention consumer on random problems (head count, layout,
    lengths, block size, list length, holes punched into the lists, padded
    strides, softmax scale) against its fp64 oracle within the parity rule of
    its own tests."""
    import oracle.attention as oa
    from tests import test_gpu_attention as ga
    rng = np.random.default_rng(70000 + i)
    for attempt in range(50):  # problems the fp64 oracle finishes in about a second
        spec = dataclasses.replace(random_spec(60000 + 50 * i + attempt), qk=synth.INT8, stride_pad=0)
        inp = synth.make_inputs(spec, 2000 + i)
        a = synth.attention_inputs(inp, int(rng.choice([16, 32, 64, 128])), 3000 + i,
                                   kv_stride_pad=int(rng.choice([0, 0, 8, 40])),
                                   scale=float(rng.choice([1.0 / np.sqrt(128), 0.3, 2.0])))
        if int((a["indices"] >= 0).sum()) * a["heads"] <= 4_000_000:
            break
    holes = rng.random(a["indices"].shape) < 0.1
    a["indices"][holes] = -1
    log("consumer sweep %d: heads %d, %s" % (i, a["heads"], spec))
    ga.compare(oa.get(), a)
