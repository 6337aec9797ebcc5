"""The allocation-free bounded run (qli_run_bounded_static, its workspace a
static device array of the library) against qli_run_bounded with a caller
workspace: calls in a row on one GPU, the second smaller than the first, the
third under a token window, each bit-identical to the workspace variant and
within the parity rule of the oracle on every row."""
import numpy as np
import pytest

import synth
from tests._gpu import check_row, check_structure, device_inputs, log, rtol_of

pytestmark = pytest.mark.gpu

CALLS = [
    # (spec holding the bound in every batch, bound, device key lengths)
    (synth.small(batch=4, s1=2, aslk=[30000] * 4, block_size=64, sparse_count=1024, sparse_mode=3),
     30000, [30000, 12000, 9000, 500]),            # two-pass rows: segments, then merges
    (synth.small(qk=synth.FP8, batch=2, s1=1, aslk=[3000] * 2, block_size=32, sparse_count=256),
     3000, [2999, 700]),                           # smaller: one pass, fp8
    (synth.small(batch=3, s1=4, aslk=[20000] * 3, block_size=64, sparse_count=512, sparse_mode=3,
                 pre_tokens=3000, next_tokens=0),
     20000, [20000, 9000, 2500]),                  # a token window: each row's range from its position
]


def test_static_workspace_matches_caller_workspace(ora):
    import torch
    import sparse_attention_token_paged_amd as qli
    qli.load()
    for n, (spec, bound, lens) in enumerate(CALLS):
        inp = synth.make_inputs(spec, 31 + n)
        p = inp["problem"]
        log("static workspace call %d: %s lens %s" % (n, spec.name, lens))
        dev = device_inputs(inp)
        aslk = torch.tensor(lens, dtype=torch.int32, device="cuda")
        bix = qli.BoundedIndexer(p, bound)
        a_idx, a_val = bix.alloc_outputs()
        bix.run(aslk, dev["query"], dev["key"], dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
                a_idx, a_val)
        b_idx = torch.full_like(a_idx, -7)
        b_val = torch.full_like(a_val, 3.0)
        rc = qli.qli_run_bounded_static(qli.Problem.from_dict(p), bound, aslk, dev["query"], dev["key"],
                                        dev["weights"], dev["q_scale"], dev["k_scale"], dev["block_table"],
                                        b_idx, b_val, qli.current_stream())
        assert rc == qli.QLI_OK, qli.qli_status_string(rc)
        torch.cuda.synchronize()
        a_idx, a_val, b_idx, b_val = (t.cpu().numpy() for t in (a_idx, a_val, b_idx, b_val))
        assert np.array_equal(a_idx, b_idx) and np.array_equal(a_val, b_val), "call %d differs" % n
        sub = dict(inp, aslk=np.asarray(lens, dtype=np.int32))
        # each row's range [lo, hi) (lo = 0 without a window); positions relative to lo
        lo, hi = ora.row_range(p["layout_query"], p["batch"], p["s1"], p["sparse_mode"], p["cmp_ratio"], None,
                               sub["aslk"], p["pre_tokens"], p["next_tokens"])
        rel = np.where(b_idx >= 0, b_idx - lo[:, None], -1)
        check_structure(rel, b_val, hi - lo, p["sparse_count"])
        rc, _, _, sc = ora.indexer(sub, scores_cols=max(1, int(hi.max())))
        assert rc == 0
        for r in range(hi.size):
            check_row(r, int(hi[r] - lo[r]), p["sparse_count"], rel[r], b_val[r], sc[r, lo[r]:hi[r]], rtol_of(inp))
