"""The allocation-free bounded run (qli_run_bounded_static, its workspace a
static device array of the library) against qli_run_bounded with a caller
workspace: two calls in a row on one GPU, the second smaller than the first,
each bit-identical to the workspace variant and within the parity rule of the
oracle on every row."""
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
        vis = ora.row_visible(p["layout_query"], p["batch"], p["s1"], p["sparse_mode"], p["cmp_ratio"], None,
                              sub["aslk"])
        check_structure(b_idx, b_val, vis, p["sparse_count"])
        rc, _, _, sc = ora.indexer(sub, scores_cols=int(vis.max()))
        assert rc == 0
        for r in range(vis.size):
            check_row(r, int(vis[r]), p["sparse_count"], b_idx[r], b_val[r], sc[r, :vis[r]], rtol_of(inp))
