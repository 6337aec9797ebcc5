"""The attention oracle's pins have teeth: each plausible mistake below is
planted in a copy of attention_oracle.c (on the CPU, in a temporary
directory), the copy is compiled, and at least one pin of
tests/test_oracle_attention.py must fail against it (in a child process, so
a planted out-of-range read that crashes counts as caught)."""
import os
import subprocess
import sys

import pytest

import oracle
import oracle.attention as oa

MUTANTS = [
    ("max not subtracted", "w = exp(logit[n++] - m);", "w = exp(logit[n++]);"),
    ("scale dropped", "logit[n] = scale * dot;", "logit[n] = dot;"),
    ("scale inverted", "logit[n] = scale * dot;", "logit[n] = dot / scale;"),
    ("value read from the key cache", "vj = entry(v_cache,", "vj = entry(k_cache,"),
    ("query head ignored", "const uint16_t *qh = q + (r * heads + h) * head_dim;",
     "const uint16_t *qh = q + (r * heads) * head_dim;"),
    ("block index", "block_table[(int64_t)b * max_blocks + j / block_size]",
     "block_table[(int64_t)b * max_blocks + j % block_size]"),
    ("block stride ignored", "cache + (int64_t)blk * stride", "cache + (int64_t)blk * block_size * head_dim"),
    ("padding slots attended", "                    if (j < 0)\n                        continue;\n", ""),
    ("lse without the log", "lse[r * heads + h] = m + log(l);", "lse[r * heads + h] = m + l;"),
    ("normalized by the count", "o[d] /= l;", "o[d] /= n;"),
    ("TND batch off by one", "if (r < aslq[b])", "if (r <= aslq[b])"),
    ("bf16 shift", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    ("empty-row lse", "lse[r * heads + h] = -INFINITY;", "lse[r * heads + h] = 0.0;"),
]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def caught(aor) -> bool:
    from tests import test_oracle_attention as t
    import synth
    pins = [t.test_bf16_decoding,
            lambda o: t.test_brute_force(o, synth.BSND), lambda o: t.test_brute_force(o, synth.TND),
            t.test_dense_causal_equals_sdpa, t.test_single_entry_and_zero_scale, t.test_list_order_and_padding,
            t.test_paging_and_layout_invariance, t.test_large_logits_stay_finite]
    for pin in pins:
        try:
            pin(aor)
        except Exception:
            return True
    return False


def pins_fail_in_child(lib_path: str) -> bool:
    code = ("import sys; sys.path.insert(0, %r); import oracle.attention as oa; "
            "from tests.test_oracle_attention_mutants import caught; "
            "sys.exit(3 if caught(oa.AttentionOracle(%r)) else 0)" % (ROOT, lib_path))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if res.returncode not in (0, 3) and res.returncode > 0:
        raise RuntimeError("pin battery could not run:\n" + res.stderr[-2000:])
    return res.returncode != 0


def test_unmutated_copy_passes_every_pin(tmp_path):
    src = tmp_path / "copy.c"
    src.write_text(open(oa.SOURCE).read())
    assert not pins_fail_in_child(oracle.compile_source(str(src), str(tmp_path / "copy.so")))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    text = open(oa.SOURCE).read()
    assert text.count(old) == 1, "mutation site not unique: %s" % name
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.compile_source(str(src), str(tmp_path / "mutant.so"))
    assert pins_fail_in_child(lib), "no pin caught the planted mistake: %s" % name
