"""Host-side tests of the C ABI (no GPU needed): the library loads and
exports every entry point include/qli.h declares, qli_plan enforces each
constraint of the VllmQuantLightningIndexer page with the documented status
code, and the plan covers every visible (row, key) pair exactly once with
the visible counts the oracle computes."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="session")
def qli():
    import sparse_attention_token_paged_amd as q
    from sparse_attention_token_paged_amd import build as b
    if b.stale():
        b.build()
    q.load()
    return q


def declared_functions():
    text = open(os.path.join(ROOT, "include", "qli.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qli_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(qli):
    names = declared_functions()
    assert set(names) == set(qli.EXPORTED)
    lib = ctypes.CDLL(qli.LIBRARY)
    for n in names:
        assert hasattr(lib, n), n


def test_only_c_abi_symbols_exported(qli):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", qli.LIBRARY], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert {s for s in syms if s.startswith("qli")} == set(declared_functions())
    assert not [s for s in syms if s.startswith("_ZN3qli")]


def test_status_strings(qli):
    assert qli.qli_status_string(0) == "ok"
    for c in range(1, 6):
        assert qli.qli_status_string(c) not in ("ok", "unknown status")
    assert qli.qli_status_string(99) == "unknown status"


def base_problem(**kw):
    inp = synth.make_inputs(synth.small(**kw), 0)
    return inp


def plan_rc(qli, inp, **over):
    p = dict(inp["problem"], **over)
    rc, _, _ = qli.qli_plan(qli.Problem.from_dict(p), inp["aslq"], inp["aslk"])
    return rc


@pytest.mark.parametrize("field,value,code", [
    ("num_heads_q", 32, 1), ("num_heads_k", 2, 1), ("head_dim", 64, 1),
    ("layout_query", 2, 1), ("qk_dtype", 2, 1), ("scale_dtype", 1, 2),
    ("block_size", 24, 1), ("block_size", 8, 1), ("block_size", 1040, 1),
    ("sparse_count", 0, 1), ("sparse_count", 2049, 1), ("sparse_mode", 1, 1), ("sparse_mode", 2, 1),
    ("cmp_ratio", 3, 1), ("cmp_ratio", 0, 1), ("cmp_ratio", 256, 1),
    ("pre_tokens", -1, 1), ("next_tokens", -1, 1), ("query_quant_mode", 1, 2), ("key_quant_mode", 1, 2),
    ("return_value", 2, 1), ("sort_output", 2, 1), ("reserved0", 1, 1), ("key_block_stride", 100, 1), ("key_block_stride", 64 * 128 + 8, 2),
    ("batch", -1, 1), ("num_blocks", 0, 1), ("max_blocks_per_seq", 0, 1)])
def test_plan_validation(qli, field, value, code):
    inp = base_problem()
    assert plan_rc(qli, inp) == 0
    assert plan_rc(qli, inp, **{field: value}) == code


def test_plan_length_validation(qli):
    inp = base_problem(aslk=[300, 200], block_size=64)
    assert plan_rc(qli, inp, max_blocks_per_seq=4) == 1           # 300 entries need 5 blocks
    rc, _, _ = qli.qli_plan(qli.Problem.from_dict(inp["problem"]), None, np.array([300, -1], np.int32))
    assert rc == 1                                                  # negative key length
    rc, _, _ = qli.qli_plan(qli.Problem.from_dict(inp["problem"]), np.array([1, 3], np.int32), inp["aslk"])
    assert rc == 1                                                  # BSND count above S1
    rc, _, _ = qli.qli_plan(qli.Problem.from_dict(inp["problem"]), None, None)
    assert rc == 1                                                  # key lengths are required
    tnd = synth.make_inputs(synth.small(layout=synth.TND, s1=6, aslq=[4, 6]), 0)
    for bad in ([4, 3], [4, 7], [-1, 6]):
        rc, _, _ = qli.qli_plan(qli.Problem.from_dict(tnd["problem"]), np.array(bad, np.int32), tnd["aslk"])
        assert rc == 1, bad
    rc, _, _ = qli.qli_plan(qli.Problem.from_dict(tnd["problem"]), None, tnd["aslk"])
    assert rc == 1                                                  # TND needs the prefix sums


def test_maximum_key_length(qli):
    """A sequence holds at most 2^22 - 1 stored (compressed) entries, the
    range in which the kernels' reciprocal division is exact; one more is
    QLI_ERR_SIZE from the planner and the bounded entry points alike, with
    and without compression.  Only lengths are read, so no cache is needed."""
    p = base_problem()["problem"]
    for cmp in (1, 4):
        for n, want in (((1 << 22) - 1, qli.QLI_OK), (1 << 22, qli.QLI_ERR_SIZE)):
            q = dict(p, batch=1, s1=1, block_size=1024, num_blocks=4096, max_blocks_per_seq=4096,
                     sparse_count=2048, sparse_mode=0, cmp_ratio=cmp)
            prob = qli.Problem.from_dict(q)
            rc, _, ws = qli.qli_plan(prob, None, np.array([n * cmp], dtype=np.int32))
            assert rc == want, (cmp, n, rc)
            if rc == qli.QLI_OK:  # every score staged once, the merge region of 512 segment winners
                assert ws >= 4 * n
            rc, _ = qli.qli_bounded_workspace(prob, n * cmp)
            assert rc == want, (cmp, n, rc)


def test_plan_capacity(qli):
    inp = base_problem()
    lib = qli.load()
    prob = qli.Problem.from_dict(inp["problem"])
    nb, ws = ctypes.c_size_t(0), ctypes.c_size_t(0)
    ak = np.ascontiguousarray(inp["aslk"])
    assert lib.qli_plan(ctypes.byref(prob), None, ak.ctypes.data, None, 0, ctypes.byref(nb), ctypes.byref(ws)) == 0
    small = np.zeros(nb.value - 16, np.uint8)
    assert lib.qli_plan(ctypes.byref(prob), None, ak.ctypes.data, small.ctypes.data, small.size,
                        ctypes.byref(nb), ctypes.byref(ws)) == 3


# --- plan parsing (layout of qli_internal.h) ---------------------------------
HDR = np.dtype([("magic", "<u4"), ("version", "<u4"), ("fingerprint", "<u8"), ("plan_bytes", "<i8"),
                ("workspace_bytes", "<i8"), ("rows", "<i8"), ("visible_pairs", "<i8"), ("ws_scores", "<i8"),
                ("off_rows", "<i8"), ("off_items", "<i8"), ("off_select", "<i8"), ("kind", "<i4"),
                ("rows_per_item", "<i4"), ("n_items", "<i4"), ("n_select", "<i4"), ("chunk", "<i4"),
                ("max_vis", "<i4"), ("reserved1", "<i4"), ("max_cand", "<i4"), ("key_entries", "<i8"),
                ("table_entries", "<i8"), ("active_rows", "<i8"), ("ws_index_offset", "<i8"),
                ("reg_chunks", "<i4"), ("reg_rows", "<i4"), ("reg_maxv", "<i4"), ("n_select2", "<i4"),
                ("max_cand2", "<i4"), ("sort_output", "<i4"), ("reserved2", "<i4", 2),
                ("ws_values_offset", "<i8"), ("reserved3", "<i8")])
ROW = np.dtype([("batch", "<i4"), ("vis", "<i4"), ("ws_off", "<i8"), ("ncand", "<i4"), ("lo", "<i4")])
SEL = np.dtype([("src_off", "<i8"), ("dst_off", "<i8"), ("row", "<i4"), ("n", "<i4"), ("base", "<i4"),
                ("indexed", "<i4")])
SEGMENT = 8192  # candidates per first-pass selection of a long row
ITEM = np.dtype([("row0", "<i4"), ("nrows", "<i4"), ("batch", "<i4"), ("key0", "<i4"), ("nkeys", "<i4"),
                 ("flags", "<i4"), ("reserved", "<i4", 2), ("vis", "<i4", 4), ("cand_off", "<i8", 4),
                 ("lo", "<i4", 4)])


def parse(plan):
    h = np.frombuffer(plan[:HDR.itemsize].tobytes(), HDR)[0]
    rows = np.frombuffer(plan[h["off_rows"]:h["off_rows"] + ROW.itemsize * h["rows"]].tobytes(), ROW)
    items = np.frombuffer(plan[h["off_items"]:h["off_items"] + ITEM.itemsize * h["n_items"]].tobytes(), ITEM)
    nsel = int(h["n_select"]) + int(h["n_select2"])
    sel = np.frombuffer(plan[h["off_select"]:h["off_select"] + SEL.itemsize * nsel].tobytes(), SEL)
    return h, rows, items, sel


PLAN_CASES = [
    synth.small(),
    synth.small(batch=3, s1=4, aslk=[1000, 517, 77], block_size=48, sparse_count=256, sparse_mode=3),
    synth.small(batch=3, s1=3, aslk=[150, 40, 0], aslq=[3, 2, 3], block_size=32, sparse_count=64,
                sparse_mode=3, cmp_ratio=2),
    synth.small(layout=synth.TND, batch=3, s1=210, aslq=[70, 140, 200], aslk=[70, 100, 300], block_size=32,
                sparse_count=64, sparse_mode=3),
    synth.small(qk=synth.FP8, batch=5, s1=1, aslk=("uniform", 100, 9000), block_size=64, sparse_count=300),
    synth.small(batch=0, s1=4, aslk=[]),
    synth.small(layout=synth.TND, batch=0, s1=5, aslk=[], aslq=[]),
    synth.small(batch=16, s1=1, aslk=[70000 - 977 * i for i in range(16)], block_size=64, sparse_count=256),
    synth.small(batch=8, s1=2, aslk=[70000] * 8, block_size=32, sparse_count=256, sparse_mode=3),
    synth.small(batch=5, s1=3, aslk=[3000] * 5, block_size=64, sparse_count=256, sparse_mode=3),
    synth.small(batch=4, s1=1, aslk=[900] * 4, block_size=16, sparse_count=1000),
    # pre_tokens / next_tokens windows: decode rows, prefill rows, long staged rows
    synth.small(batch=3, s1=4, aslk=[5000, 700, 90], block_size=64, sparse_count=256, sparse_mode=3,
                pre_tokens=1000, next_tokens=0),
    synth.small(batch=2, s1=40, aslk=[3000, 2500], block_size=32, sparse_count=64, sparse_mode=0,
                cmp_ratio=2, pre_tokens=300, next_tokens=50),
    synth.small(batch=2, s1=2, aslk=[70000, 65000], block_size=128, sparse_count=512, sparse_mode=3,
                pre_tokens=30000, next_tokens=synth.INT64_MAX),
    synth.small(layout=synth.TND, batch=2, s1=30, aslq=[12, 30], aslk=[500, 4000], block_size=32,
                sparse_count=128, sparse_mode=3, cmp_ratio=4, pre_tokens=777, next_tokens=0),
]


@pytest.mark.parametrize("equal", [False, True])
def test_plan_items_of_ragged_batches_fill_the_slots(qli, equal):
    """64 one-row batches of 4k..64k keys (the ragged fp8 decode shape): each
    batch's entries are cut into near-equal runs of 128-entry blocks, none
    longer than the chunk, and the free decode slots (768) go to the batches
    with the longest items, so every slot holds an item.  Equal batches keep
    whole chunks and a remainder."""
    spec = synth.small(qk=synth.FP8, batch=2, s1=1, aslk=[100, 100], block_size=64, sparse_count=2048)
    p = dict(synth.make_inputs(spec, 1)["problem"], batch=64, max_blocks_per_seq=1024, num_blocks=1 << 16)
    rng = np.random.default_rng(7)
    aslk = np.full(64, 50000, np.int32) if equal else rng.integers(4096, 65537, size=64).astype(np.int32)
    rc, plan, _ = qli.qli_plan(qli.Problem.from_dict(p), None, aslk)
    assert rc == 0
    h, rows, items, _ = parse(plan)
    chunk = int(h["chunk"])
    assert items["nkeys"].max() <= chunk
    for b in range(64):
        it = np.sort(items[items["batch"] == b], order="key0")
        n = it["nkeys"]
        assert it["key0"][0] == 0 and np.array_equal(it["key0"][1:], np.cumsum(n)[:-1])
        assert n.sum() == aslk[b]
        if equal:
            assert np.all(n[:-1] == chunk)
        else:
            assert np.all(n[:-1] % 128 == 0) and (len(n) < 3 or n[:-1].max() - n[:-1].min() <= 128)
    if not equal:
        assert h["n_items"] == DECODE_SLOTS                         # every slot holds an item
        assert sum(-(-int(v) // chunk) for v in aslk) < DECODE_SLOTS  # whole chunks would leave some free


@pytest.mark.parametrize("spec", PLAN_CASES, ids=range(len(PLAN_CASES)))
def test_plan_covers_each_visible_pair_once(qli, ora, spec):
    inp = synth.make_inputs(spec, 3)
    p = inp["problem"]
    rc, plan, ws = qli.qli_plan(qli.Problem.from_dict(p), inp["aslq"], inp["aslk"])
    assert rc == 0
    h, rows, items, sel = parse(plan)
    assert h["magic"] == 0x504C4951
    nrows = p["batch"] * p["s1"] if p["layout_query"] == 0 else p["s1"]
    assert h["rows"] == nrows
    if nrows:
        lo, hi = ora.row_range(p["layout_query"], p["batch"], p["s1"], p["sparse_mode"], p["cmp_ratio"],
                               inp["aslq"], inp["aslk"], p["pre_tokens"], p["next_tokens"])
    else:
        lo = hi = np.zeros(0, np.int64)
    assert np.array_equal(rows["vis"], hi) and np.array_equal(rows["lo"], lo)
    vis = hi - lo                                   # visible counts
    assert h["visible_pairs"] == vis.sum()
    cover = [np.zeros(v, np.int32) for v in hi]     # entries [0, hi); those below lo must stay uncovered
    padded = np.zeros(nrows, np.int32)
    for it in items:
        for r in range(it["row0"], it["row0"] + it["nrows"]):
            if it["flags"] & 1:
                padded[r] += 1
            if it["nkeys"]:
                assert rows[r]["batch"] == it["batch"]
                e = min(it["key0"] + it["nkeys"], hi[r])
                if e > it["key0"]:
                    cover[r][it["key0"]:e] += 1
                if h["kind"] == 0 and it["nkeys"]:   # decode items carry the rows' ranges
                    u = r - it["row0"]
                    assert (it["vis"][u], it["lo"][u]) == (hi[r], lo[r])
                    if rows[r]["ws_off"] >= 0:
                        assert it["cand_off"][u] == rows[r]["ws_off"] + it["key0"] - lo[r]
        assert it["nkeys"] <= h["chunk"] and (it["key0"] % 64 == 0)
    assert all(np.all(c[lo[r]:] == 1) for r, c in enumerate(cover))
    if h["reg_chunks"] > 0:
        # regular decode plans: an item's batch, keys and rows follow from its position
        rc_, chunk_, s1_, mv_ = int(h["reg_chunks"]), int(h["chunk"]), int(h["reg_rows"]), int(h["reg_maxv"])
        assert h["kind"] == 0 and p["layout_query"] == 0 and s1_ == p["s1"] and len(items) == p["batch"] * rc_
        for i, it in enumerate(items):
            b, c = divmod(i, rc_)
            assert it["batch"] == b and it["key0"] == c * chunk_ and it["nkeys"] == min(chunk_, mv_ - c * chunk_)
            assert it["row0"] == b * s1_ and it["nrows"] == s1_
            assert max(int(hi[r]) for r in range(b * s1_, (b + 1) * s1_)) == mv_
    assert np.all(padded == 1)
    k = p["sparse_count"]
    selected = [r for r in range(nrows) if vis[r] > k]
    # a selected row stages every score it sees; the others none
    ncand = {r: int(vis[r]) for r in selected}
    assert [int(x) for x in rows["ncand"]] == [ncand.get(r, 0) for r in range(nrows)]
    pad4 = lambda n: (n + 3) // 4 * 4  # 16-byte aligned candidate regions
    offs = [int(rows[r]["ws_off"]) for r in selected]
    assert offs == list(np.cumsum([0] + [pad4(ncand[r]) for r in selected])[:-1])
    # The selection table: pass 1 = short rows (final) and segments of long rows,
    # pass 2 = one merge per long row over its segments' winners.
    n1, n2 = int(h["n_select"]), int(h["n_select2"])
    p1, p2 = sel[:n1], sel[n1:]
    long_rows = [r for r in selected if ncand[r] > SEGMENT]
    assert list(p2["row"]) == long_rows and np.all(p2["dst_off"] == -1) and np.all(p2["indexed"] == 1)
    region_end = sum(pad4(ncand[r]) for r in selected)
    merge_off = region_end
    i1 = 0
    for r in selected:
        n = ncand[r]
        if n <= SEGMENT:
            e = p1[i1]
            i1 += 1
            assert (e["row"], e["n"], e["src_off"], e["dst_off"], e["base"], e["indexed"]) == \
                (r, n, rows[r]["ws_off"], -1, lo[r], 0)
            continue
        dst, m = merge_off, 0
        for s0 in range(0, n, SEGMENT):
            e = p1[i1]
            i1 += 1
            sn = min(SEGMENT, n - s0)
            assert (e["row"], e["n"], e["src_off"], e["dst_off"], e["base"], e["indexed"]) == \
                (r, sn, rows[r]["ws_off"] + s0, dst + m, lo[r] + s0, 0)
            m += min(k, sn)
        fin = p2[long_rows.index(r)]
        assert fin["src_off"] == merge_off and fin["n"] == m
        merge_off += pad4(m)
    assert i1 == n1
    assert np.all(sel["src_off"] % 4 == 0)
    assert int(h["max_cand"]) == max([int(e["n"]) for e in p1], default=0)
    assert int(h["max_cand2"]) == max([int(e["n"]) for e in p2], default=0)
    # key indices of the merge regions [region_end, merge_off) follow every score, 16-byte aligned:
    # the index of candidate e sits at byte ws_index_offset + 4e
    a16 = (4 * merge_off + 15) // 16 * 16
    if n2 > 0:
        assert int(h["ws_index_offset"]) == a16 - 4 * region_end
        assert ws == a16 + 4 * (merge_off - region_end)
    else:
        assert ws == 4 * merge_off
    sel = selected
    if h["kind"] == 0:
        # decode items: inline visible counts, and candidate slots that tile each row's range
        slots = {r: [] for r in sel}
        for it in items:
            for u in range(it["nrows"]):
                r = it["row0"] + u
                assert it["vis"][u] == hi[r]
                if it["nkeys"] and r in slots:
                    a = max(int(it["key0"]), int(lo[r]))
                    n = min(int(it["key0"] + it["nkeys"]), int(hi[r])) - a
                    if n > 0:   # cand_off is the slot of entry key0; the row's own slots start at lo
                        slots[r].append((int(it["cand_off"][u]) + a - int(it["key0"]), n))
                elif it["nkeys"]:
                    assert it["cand_off"][u] == -1
        for r, c in slots.items():
            c.sort()
            pos = int(rows[r]["ws_off"])
            for off, n in c:
                assert off == pos
                pos += n
            assert pos == int(rows[r]["ws_off"]) + int(rows[r]["ncand"])
    info = qli.qli_plan_info_get(plan)
    assert info.rows == nrows and info.visible_pairs == vis.sum() and info.select_rows == len(sel)
    assert info.active_rows == int((vis > 0).sum())
    # per batch, the entries some row sees: [smallest lo, largest hi) over rows that see any
    spans = []
    for b in range(p["batch"]):
        rs = [r for r in range(nrows) if rows[r]["batch"] == b and vis[r] > 0]
        if rs:
            spans.append((min(int(lo[r]) for r in rs), max(int(hi[r]) for r in rs)))
    bs = p["block_size"]
    assert info.key_entries == sum(e - a for a, e in spans)
    assert info.table_entries == sum((e - 1) // bs - a // bs + 1 for a, e in spans)


def test_run_rejects_bad_arguments_without_launching(qli):
    inp = base_problem()
    prob = qli.Problem.from_dict(inp["problem"])
    rc, plan, ws = qli.qli_plan(prob, inp["aslq"], inp["aslk"])
    assert rc == 0
    fake = 1 << 40  # never dereferenced: every call below fails validation first
    args = [fake] * 9
    other = qli.Problem.from_dict(dict(inp["problem"], sparse_count=65))
    assert qli.qli_run(other, plan, fake, *args) == qli.QLI_ERR_PLAN
    bad = plan.copy()
    bad[0] ^= 0xFF
    assert qli.qli_run(prob, bad, fake, *args) == qli.QLI_ERR_PLAN
    assert qli.qli_run(prob, plan, None, *args) == qli.QLI_ERR_ARG
    a = list(args)
    a[7] = None                                                     # sparse_indices
    assert qli.qli_run(prob, plan, fake, *a) == qli.QLI_ERR_ARG
    a = list(args)
    a[8] = None                                                     # sparse_values with return_value=1
    assert qli.qli_run(prob, plan, fake, *a) == qli.QLI_ERR_ARG
    a = list(args)
    a[0] = None                                                     # query
    assert qli.qli_run(prob, plan, fake, *a) == qli.QLI_ERR_ARG
    invalid = qli.Problem.from_dict(dict(inp["problem"], sparse_mode=1))
    assert qli.qli_run(invalid, plan, fake, *args) == qli.QLI_ERR_ARG
    # stage selection: only 1, 2 and 3 are valid
    for stages in (0, 4, -1):
        assert qli.qli_run_stage(prob, plan, fake, *args, stages) == qli.QLI_ERR_ARG
    # debug range checks
    assert qli.qli_run_debug(prob, plan, fake, *args, 2, 1, 8, fake, fake) == qli.QLI_ERR_ARG
    assert qli.qli_run_debug(prob, plan, fake, *args, 0, 99, 8, fake, fake) == qli.QLI_ERR_ARG
    assert qli.qli_run_debug(prob, plan, fake, *args, 0, 1, 8, None, fake) == qli.QLI_ERR_ARG


def test_empty_problem_runs_without_device(qli):
    """Zero rows: validation passes and nothing is launched."""
    inp = synth.make_inputs(synth.small(batch=0, s1=4, aslk=[]), 0)
    prob = qli.Problem.from_dict(inp["problem"])
    rc, plan, ws = qli.qli_plan(prob, None, np.zeros(0, np.int32))
    assert rc == 0 and ws == 0
    assert qli.qli_run(prob, plan, 1 << 40, *([None] * 9)) == qli.QLI_OK


# --- bounded decode (no host plan) --------------------------------------------
ITEM_BYTES = 96
DECODE_SLOTS = 768   # decode workgroups resident at once (3 per CU x 256 CUs)


def bounded_workspace_expected(p, max_len):
    """Bounded BSND: the scores' layout below, then for decode problems (S1 <= 4)
    of more than 256 batches the item table the device builds (16-byte aligned;
    room for every item any lengths can give: max(slots + B, B * ceil(entries /
    4096)) items of 96 bytes) and its 16-byte count.  Up to 256 batches the
    scoring kernel splits the work itself and needs no table."""
    base = bounded_scores_expected(p, max_len)
    rows, b = p["batch"] * p["s1"], p["batch"]
    if rows == 0 or p["s1"] > 4 or b <= 256:
        return base
    span = window_span(p, max_len // p["cmp_ratio"], p["s1"], True)
    cap = max(DECODE_SLOTS + b, b * max(1, -(-span // 4096)))
    return (base + 15) // 16 * 16 + ITEM_BYTES * cap + 16


def bounded_scores_expected(p, max_len):
    """Workspace of the bounded scores, from their layout: rows that may see more
    than k entries keep every score (16-byte aligned row stride); rows longer than
    one selection segment also keep each segment's k winners for the merge, with
    their key indices in an int32 region after every score (merge regions only)."""
    rows, k = p["batch"] * p["s1"], p["sparse_count"]
    nmax = window_span(p, max_len // p["cmp_ratio"], 1, False)  # entries one row may see
    if rows == 0 or nmax <= k:
        return 0
    pad4 = lambda n: (n + 3) // 4 * 4
    nseg = -(-nmax // SEGMENT)
    merges = rows * pad4(nseg * k) if nseg > 1 else 0
    total = rows * pad4(nmax) + merges
    return ((4 * total + 15) // 16 * 16) + 4 * merges if nseg > 1 else 4 * total


TND_IN_KERNEL_BATCHES = 128  # up to this many batches the kernels derive the row partition themselves


def bounded_tnd_workspace_expected(p, max_len):
    """TND: the BSND layout over T rows; for more than 128 batches then
    (16-byte aligned) the row and group tables: rows_end[B], group_start[B + 1],
    group_batch[T // 4 + B + 2] (4-row groups; each table padded to 4
    elements) and row_batch[T], int32."""
    b, t = p["batch"], p["s1"]
    base = bounded_scores_expected(dict(p, batch=1, s1=t), max_len)
    if b <= TND_IN_KERNEL_BATCHES:
        return base
    up4 = lambda n: (n + 3) // 4 * 4
    return (base + 15) // 16 * 16 + 4 * (up4(b) + up4(b + 1) + up4(t // 4 + b + 2) + t)


@pytest.mark.parametrize("b,t,k,max_len", [(3, 40, 256, 5000), (1, 7, 2048, 100), (5, 300, 64, 20000),
                                           (128, 300, 64, 20000), (129, 300, 64, 20000), (129, 7, 2048, 100),
                                           (4096, 9000, 256, 5000)])
def test_bounded_tnd_workspace(qli, b, t, k, max_len):
    spec = synth.small(layout=synth.TND, batch=b, s1=t, aslq=[t] * b, aslk=[max(max_len, 1)] * b, block_size=64,
                       sparse_count=k, sparse_mode=3)
    p = synth.make_inputs(spec, 1)["problem"]
    rc, ws = qli.qli_bounded_workspace(qli.Problem.from_dict(p), max_len)
    assert rc == 0 and ws == bounded_tnd_workspace_expected(p, max_len)


@pytest.mark.parametrize("batch", [3, 300])
@pytest.mark.parametrize("s1,k,cmp,max_len", [(1, 512, 1, 1000), (4, 2048, 1, 8192), (2, 256, 4, 70000),
                                                (3, 100, 1, 0), (1, 2048, 1, 140000), (8, 256, 1, 3000),
                                                (13, 2048, 1, 20000), (64, 512, 2, 10000)])
def test_bounded_workspace(qli, batch, s1, k, cmp, max_len):
    spec = synth.small(batch=3, s1=s1, aslk=[max(max_len, 1)] * 3, block_size=64, sparse_count=k,
                       sparse_mode=3, cmp_ratio=cmp)
    p = dict(synth.make_inputs(spec, 1)["problem"], batch=batch)   # the workspace depends on the fields only
    rc, ws = qli.qli_bounded_workspace(qli.Problem.from_dict(p), max_len)
    assert rc == 0 and ws == bounded_workspace_expected(p, max_len)


def test_bounded_rejects_without_launching(qli):
    spec = synth.small(batch=2, s1=2, aslk=[5000, 5000], block_size=64, sparse_count=256, sparse_mode=3)
    p = synth.make_inputs(spec, 1)["problem"]
    prob = qli.Problem.from_dict(p)
    bound = 5000
    fake = 1 << 40  # never dereferenced: every call below fails validation first
    args = [fake] * 10
    assert qli.qli_bounded_workspace(prob, -1)[0] == qli.QLI_ERR_ARG
    blocks = p["max_blocks_per_seq"]
    assert qli.qli_bounded_workspace(prob, (blocks + 1) * 64)[0] == qli.QLI_ERR_ARG  # beyond the block table
    tnd = qli.Problem.from_dict(dict(p, layout_query=synth.TND))
    assert qli.qli_bounded_workspace(tnd, bound) == (qli.QLI_OK, bounded_tnd_workspace_expected(
        dict(p, layout_query=synth.TND), bound))
    assert qli.qli_run_bounded(tnd, bound, *args) == qli.QLI_ERR_UNSUPPORTED     # TND needs the query lengths
    assert qli.qli_run_bounded_tnd(prob, bound, fake, *args) == qli.QLI_ERR_UNSUPPORTED  # BSND
    assert qli.qli_run_bounded_tnd(tnd, bound, None, *args) == qli.QLI_ERR_ARG   # actual_seq_lengths_query
    assert qli.qli_run_bounded_tnd(tnd, bound, fake + 2, *args) == qli.QLI_ERR_ARG
    many = qli.Problem.from_dict(dict(p, layout_query=synth.TND, batch=4097))
    assert qli.qli_bounded_workspace(many, bound)[0] == qli.QLI_ERR_UNSUPPORTED
    wide = qli.Problem.from_dict(dict(p, s1=5))  # 4-row position groups: supported, same workspace layout
    assert qli.qli_bounded_workspace(wide, bound) == (qli.QLI_OK, bounded_workspace_expected(dict(p, s1=5), bound))
    a = list(args)
    a[0] = None                                                     # actual_seq_lengths_key
    assert qli.qli_run_bounded(prob, bound, *a) == qli.QLI_ERR_ARG
    a = list(args)
    a[8] = None                                                     # sparse_indices
    assert qli.qli_run_bounded(prob, bound, *a) == qli.QLI_ERR_ARG
    a = list(args)
    a[1] = fake + 4                                                 # query not 16-byte aligned
    assert qli.qli_run_bounded(prob, bound, *a) == qli.QLI_ERR_ARG
    assert qli.qli_run_bounded(qli.Problem.from_dict(dict(p, sparse_mode=1)), bound, *args) == qli.QLI_ERR_ARG


# Producer entry points: argument checks return before anything is launched
# (the fake device addresses below are never dereferenced).
A16, A8 = 0x10000, 0x20000


def test_quantize_query_rejects_bad_arguments(qli):
    f = qli.qli_quantize_query
    assert f(2, 4, A16, A16, A16) == qli.QLI_ERR_UNSUPPORTED
    assert f(0, -1, A16, A16, A16) == qli.QLI_ERR_ARG
    assert f(0, 0, None, None, None) == qli.QLI_OK  # nothing to do, nothing launched
    assert f(0, 4, None, A16, A16) == qli.QLI_ERR_ARG
    assert f(0, 4, A16, None, A16) == qli.QLI_ERR_ARG
    assert f(0, 4, A16, A16, None) == qli.QLI_ERR_ARG
    assert f(0, 4, A16 + 8, A16, A16) == qli.QLI_ERR_ARG   # x must be 16-byte aligned
    assert f(0, 4, A16, A16 + 4, A16) == qli.QLI_ERR_ARG   # codes 8-byte aligned
    assert f(0, 4, A16, A16, A16 + 1) == qli.QLI_ERR_ARG   # fp16 scales 2-byte aligned
    assert f(1, 4, A16, A16, A16 + 2) == qli.QLI_ERR_ARG   # fp32 scales 4-byte aligned


def test_append_keys_rejects_bad_arguments(qli):
    def call(qk=0, n=8, x=A16, bidx=A16, pos=A16, bt=A16, batches=2, mb=4, nb=8, bs=32, stride=0,
             kc=A16, ks=A16):
        return qli.qli_append_keys(qk, n, x, bidx, pos, bt, batches, mb, nb, bs, stride, kc, ks)
    assert call(qk=3) == qli.QLI_ERR_UNSUPPORTED
    for bs in (0, 8, 24, 1040):
        assert call(bs=bs) == qli.QLI_ERR_ARG, bs
    assert call(nb=0) == qli.QLI_ERR_ARG
    assert call(mb=0) == qli.QLI_ERR_ARG
    assert call(batches=-1) == qli.QLI_ERR_ARG
    assert call(stride=32 * 128 - 16) == qli.QLI_ERR_ARG   # below block_size * 128
    assert call(stride=32 * 128 + 8) == qli.QLI_ERR_ARG    # not a multiple of 16
    assert call(n=-1) == qli.QLI_ERR_ARG
    assert call(n=0, x=None, bidx=None, pos=None, bt=None, kc=None, ks=None) == qli.QLI_OK
    for k in ("x", "bidx", "pos", "bt", "kc", "ks"):
        assert call(**{k: None}) == qli.QLI_ERR_ARG, k
    assert call(x=A16 + 4) == qli.QLI_ERR_ARG
    assert call(kc=A16 + 8) == qli.QLI_ERR_ARG
    assert call(qk=1, ks=A16 + 2) == qli.QLI_ERR_ARG


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with a message, before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout.strip()


def test_bounded_static_rejects_without_launching(qli):
    """qli_run_bounded_static: every argument check returns before the library
    touches a device (the fake addresses are never dereferenced)."""
    spec = synth.small(batch=2, s1=2, aslk=[5000, 5000], block_size=64, sparse_count=256, sparse_mode=3)
    p = synth.make_inputs(spec, 1)["problem"]
    prob = qli.Problem.from_dict(p)
    fake = 1 << 40
    args = [fake] * 9
    f = qli.qli_run_bounded_static
    tnd = qli.Problem.from_dict(dict(p, layout_query=synth.TND))
    assert f(tnd, 5000, *args) == qli.QLI_ERR_UNSUPPORTED
    assert f(prob, -1, *args) == qli.QLI_ERR_ARG
    a = list(args)
    a[0] = None                                                     # actual_seq_lengths_key
    assert f(prob, 5000, *a) == qli.QLI_ERR_ARG
    a = list(args)
    a[7] = None                                                     # sparse_indices
    assert f(prob, 5000, *a) == qli.QLI_ERR_ARG
    a = list(args)
    a[1] = fake + 4                                                 # query not 16-byte aligned
    assert f(prob, 5000, *a) == qli.QLI_ERR_ARG
    # beyond the 32 MiB static workspace: 64 rows of 140000 staged scores
    big = dict(p, batch=64, s1=1, max_blocks_per_seq=140000 // 64 + 1, sparse_count=512, sparse_mode=0)
    rc, ws = qli.qli_bounded_workspace(qli.Problem.from_dict(big), 140000)
    assert rc == qli.QLI_OK and ws > 32 << 20
    assert f(qli.Problem.from_dict(big), 140000, *args) == qli.QLI_ERR_SIZE
    # the fp8 decode shape at its longest (64 x 65536 entries, k = 512) fits
    rc, ws = qli.qli_bounded_workspace(qli.Problem.from_dict(big), 65536)
    assert rc == qli.QLI_OK and ws <= 32 << 20


def test_sparse_attention_rejects_without_launching(qli):
    """The consumer's scalar and pointer checks return before any launch (the
    fake addresses are never dereferenced)."""
    base = dict(batch=2, s1=4, layout_query=synth.BSND, num_heads=64, head_dim=128, num_blocks=10,
                block_size=64, max_blocks_per_seq=5, kv_block_stride=0, sparse_count=2048, softmax_scale=0.088,
                return_lse=1)
    P = lambda **kw: qli.AttnProblem.from_dict(dict(base, **kw))
    fake = 1 << 40
    args = [None, fake, fake, fake, fake, fake, fake, fake, fake]   # aslq, q, k, v, table, indices, ws, out, lse
    f = qli.qli_sparse_attention
    def expected_ws(rows, k, heads):
        """Rows split so that every workgroup fits one round of two per CU, at
        least 256 entries each (32-entry stages): fp32 partials O[128], max and
        sum per split and head."""
        ns = max(1, min(512 // rows, -(-k // 256)))
        chunk = -(-(-(-k // ns)) // 32) * 32
        ns = -(-k // chunk)
        return 0 if ns == 1 else rows * ns * heads * 130 * 4
    for rows, k in ((8, 2048), (8, 256), (96, 2048), (300, 2048), (1, 100), (33, 1000)):
        rc, ws = qli.qli_sparse_attention_workspace(P(batch=rows, s1=1, sparse_count=k))
        assert rc == qli.QLI_OK and ws == expected_ws(rows, k, 64), (rows, k)
    assert expected_ws(8, 2048, 64) == 8 * 8 * 64 * 130 * 4 and expected_ws(96, 2048, 64) == 96 * 5 * 64 * 130 * 4
    for kw, code in [(dict(num_heads=48), qli.QLI_ERR_UNSUPPORTED), (dict(head_dim=64), qli.QLI_ERR_UNSUPPORTED),
                     (dict(block_size=40), qli.QLI_ERR_ARG), (dict(block_size=2048), qli.QLI_ERR_ARG),
                     (dict(sparse_count=0), qli.QLI_ERR_ARG), (dict(sparse_count=2049), qli.QLI_ERR_ARG),
                     (dict(softmax_scale=0.0), qli.QLI_ERR_ARG), (dict(softmax_scale=float("inf")), qli.QLI_ERR_ARG),
                     (dict(kv_block_stride=100), qli.QLI_ERR_ARG), (dict(kv_block_stride=64 * 128 + 4),
                                                                     qli.QLI_ERR_UNSUPPORTED),
                     (dict(layout_query=2), qli.QLI_ERR_ARG), (dict(return_lse=2), qli.QLI_ERR_ARG),
                     (dict(reserved1=1), qli.QLI_ERR_ARG), (dict(num_blocks=0), qli.QLI_ERR_ARG)]:
        assert f(P(**kw), *args) == code, kw
        assert qli.qli_sparse_attention_workspace(P(**kw))[0] == code, kw
    a = list(args)
    a[1] = None                                                      # q
    assert f(P(), *a) == qli.QLI_ERR_ARG
    a = list(args)
    a[1] = fake + 2                                                  # q not 16-byte aligned
    assert f(P(), *a) == qli.QLI_ERR_ARG
    a = list(args)
    a[8] = None                                                      # lse with return_lse = 1
    assert f(P(), *a) == qli.QLI_ERR_ARG
    a = list(args)
    a[6] = None                                                      # workspace needed (split rows)
    assert f(P(), *a) == qli.QLI_ERR_ARG
    assert f(P(layout_query=synth.TND, s1=8), *args) == qli.QLI_ERR_ARG   # TND needs the prefix sums
    assert f(P(batch=0), *args) == qli.QLI_OK                        # no rows: nothing to launch
    rc, ws = qli.qli_sparse_attention_workspace(P(batch=300))        # enough rows: one workgroup per row
    assert rc == qli.QLI_OK and ws == 0


BEYOND = 1 << 40  # a window side at least this long bounds nothing


def window_span(p, nmax, rows, aligned):
    """Bounded runs under a pre_tokens / next_tokens window: the most entries
    `rows` consecutive query rows of a batch see together, (pre + next' + rows)
    // cmp + 1 with next' = 0 under mode 3 (the causal cut binds first), plus
    127 when the items start at a multiple of 128 below the first of them;
    never more than nmax, and nmax without a window."""
    pre, nxt = p.get("pre_tokens", synth.INT64_MAX), p.get("next_tokens", synth.INT64_MAX)
    if pre == synth.INT64_MAX and nxt == synth.INT64_MAX:
        return nmax
    nxt = 0 if p["sparse_mode"] == 3 else nxt
    if pre >= BEYOND or nxt >= BEYOND:
        return nmax
    return min(nmax, (pre + nxt + rows) // p["cmp_ratio"] + 1 + (127 if aligned else 0))


@pytest.mark.parametrize("mode", [3, 0])
@pytest.mark.parametrize("pre,nxt", [(500, synth.INT64_MAX), (synth.INT64_MAX, 9), (0, 0), (3000, 40),
                                     (100000, 0), (BEYOND, 7)])
@pytest.mark.parametrize("s1,batch", [(2, 2), (4, 300), (9, 3)])
def test_bounded_windowed_workspace(qli, mode, pre, nxt, s1, batch):
    """Bounded runs take a pre_tokens / next_tokens window: each row's scores
    need only the window's entries, so the row stride, the selection segments
    and the device item table follow the window's span."""
    spec = synth.small(batch=3, s1=s1, aslk=[20000] * 3, block_size=64, sparse_count=256, sparse_mode=mode,
                       pre_tokens=pre, next_tokens=nxt)
    p = dict(synth.make_inputs(spec, 1)["problem"], batch=batch)
    rc, ws = qli.qli_bounded_workspace(qli.Problem.from_dict(p), 20000)
    assert rc == qli.QLI_OK and ws == bounded_workspace_expected(p, 20000)
    if pre < 20000 and (mode == 3 or nxt < 20000):  # the rows see fewer entries than without a window
        assert ws < bounded_workspace_expected(dict(p, pre_tokens=synth.INT64_MAX, next_tokens=synth.INT64_MAX),
                                               20000)
    tnd = dict(p, layout_query=synth.TND, batch=min(batch, 3), s1=s1 * 3)
    rc, ws = qli.qli_bounded_workspace(qli.Problem.from_dict(tnd), 20000)
    assert rc == qli.QLI_OK and ws == bounded_tnd_workspace_expected(tnd, 20000)


def test_window_span_bounds_every_row(ora):
    """The spans above bound what the oracle's windows give (visible ranges
    computed independently, in C, from the page's reading of the window): every
    row's count of entries, and the entries of every decode batch (S1 <= 4 rows)
    and 4-row group from its first entry rounded down to 128, over seeded
    random problems (modes, cmp_ratio, windows, lengths)."""
    rng = np.random.default_rng(5)
    for _ in range(400):
        mode, cmp = int(rng.choice([0, 3])), int(rng.choice([1, 2, 4, 16, 128]))
        pre = int(rng.choice([0, 1, 5, 100, 1000, 7000, synth.INT64_MAX]))
        nxt = int(rng.choice([0, 1, 3, 50, 4000, synth.INT64_MAX]))
        s1, batch = int(rng.integers(1, 13)), int(rng.integers(1, 4))
        aslk = rng.integers(0, 20000, size=batch).astype(np.int32)
        p = dict(sparse_mode=mode, cmp_ratio=cmp, pre_tokens=pre, next_tokens=nxt)
        nmax = int(aslk.max()) // cmp
        lo, hi = ora.row_range(0, batch, s1, mode, cmp, None, aslk, pre, nxt)
        assert (hi - lo).max() <= window_span(p, nmax, 1, False)
        for size in ([s1] if s1 <= 4 else []) + [4]:
            for b in range(batch):
                for g0 in range(0, s1, size):
                    rr = slice(b * s1 + g0, b * s1 + min(g0 + size, s1))
                    seen = hi[rr] > lo[rr]
                    if seen.any():
                        start = lo[rr][seen].min() // 128 * 128
                        assert hi[rr][seen].max() - start <= window_span(p, nmax, size, True), (p, s1, aslk)


@pytest.mark.parametrize("return_value", [1, 0])
def test_sorted_output_workspace(qli, return_value):
    """sort_output keeps the plan's tables; without returned values the
    workspace grows by a [rows, k] fp32 region, 16-byte aligned at its end."""
    inp = base_problem(batch=3, s1=4, aslk=[5000, 700, 90], block_size=64, sparse_count=256, sparse_mode=3)
    p = dict(inp["problem"], return_value=return_value)
    rc0, plan0, ws0 = qli.qli_plan(qli.Problem.from_dict(p), inp["aslq"], inp["aslk"])
    rc1, plan1, ws1 = qli.qli_plan(qli.Problem.from_dict(dict(p, sort_output=1)), inp["aslq"], inp["aslk"])
    assert rc0 == rc1 == 0
    h0, h1 = parse(plan0)[0], parse(plan1)[0]
    assert h0["sort_output"] == 0 and h1["sort_output"] == 1
    rows, k = 12, 256
    if return_value:
        assert ws1 == ws0 and h1["ws_values_offset"] == -1
    else:
        assert h1["ws_values_offset"] == (ws0 + 15) // 16 * 16 and ws1 == h1["ws_values_offset"] + 4 * rows * k
    rc, bws0 = qli.qli_bounded_workspace(qli.Problem.from_dict(p), 5000)
    rc, bws1 = qli.qli_bounded_workspace(qli.Problem.from_dict(dict(p, sort_output=1)), 5000)
    assert bws1 == (bws0 if return_value else (bws0 + 15) // 16 * 16 + 4 * rows * k)
