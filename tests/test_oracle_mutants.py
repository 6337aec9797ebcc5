"""The oracle's pins have teeth: each plausible mistake below is planted in a
copy of qli_oracle.c (on the CPU, in a temporary directory), the copy is
compiled, and at least one pin test must fail against it.  Each copy runs
in a child process, so a mistake that crashes (an out-of-range block index)
counts as caught without taking the test runner down."""
import os
import subprocess
import sys

import pytest

import oracle
from tests import test_oracle_decode as dec
from tests import test_oracle_operator as op
from tests import test_oracle_scores as sco
from tests import test_oracle_topk as tk
from tests import test_oracle_visible as vis

MUTANTS = [
    ("relu dropped", "double relu = corr > 0.0 ? corr : 0.0;", "double relu = corr;"),
    ("weight dropped", "score += w * relu;", "score += relu;"),
    ("weight inside relu", "double corr = (sq * sk) * dot;", "double corr = (w * sq * sk) * dot;"),
    ("weight head index", "scale_value(p->weights, r * QLIO_HEADS + g,", "scale_value(p->weights, r * QLIO_HEADS + (g ^ 1),"),
    ("query scale of the wrong row", "scale_value(p->q_scale, r * QLIO_HEADS + g,", "scale_value(p->q_scale, g,"),
    ("key scale slot", "(int64_t)blk * pk->block_size + slot,", "slot,"),
    ("block index", "j / pk->block_size]", "j % pk->block_size]"),
    ("block stride ignored", "return pk->key + (int64_t)blk * pk->stride", "return pk->key + (int64_t)blk * pk->block_size * QLIO_DIM"),
    ("transposed query", "(r * QLIO_HEADS + g) * QLIO_DIM", "(g * QLIO_HEADS + r) * QLIO_DIM"),
    ("reversed key dims", "(int64_t)(int8_t)k[d]", "(int64_t)(int8_t)k[QLIO_DIM - 1 - d]"),
    ("fp8 read as int8", "    if (qk_dtype == 0) {\n        int64_t acc", "    if (1) {\n        int64_t acc"),
    ("causal off by one", "upto = skb - s1b + i + 1;", "upto = skb - s1b + i;"),
    ("negative causal count kept", "if (upto <= 0)\n        return 0;", "if (upto < -1000000)\n        return 0;"),
    ("ceil of compressed count", "int64_t stored = skb / cmp_ratio;", "int64_t stored = (skb + cmp_ratio - 1) / cmp_ratio;"),
    ("ties to the higher index", "return (x->idx > y->idx) - (x->idx < y->idx);", "return (x->idx < y->idx) - (x->idx > y->idx);"),
    ("ascending order", "if (x->score > y->score)\n        return -1;", "if (x->score < y->score)\n        return -1;"),
    ("e4m3 exponent bias", "ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 9)"),
    ("e4m3 subnormal scale", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("f16 subnormal scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("value padding", "ov[j] = -INFINITY;", "ov[j] = 0.0f;"),
    ("TND local index", "*i = r - start;", "*i = r;"),
    ("BSND query counts ignored", "int64_t n = p->aslq ? p->aslq[bb] : p->s1_or_t;", "int64_t n = p->s1_or_t;"),
    # the FLOAT32 scale / weight decoding of the FLOAT8_e4m3fn pairing
    ("fp32 element stride 2", "memcpy(&f, (const char *)base + 4 * i, 4);",
     "memcpy(&f, (const char *)base + 8 * i, 4);"),
    ("fp32 scales read as fp16", "if (scale_dtype == 0) {", "if (scale_dtype >= 0) {"),
    ("fp32 weight ignored", "double w = scale_value(p->weights, r * QLIO_HEADS + g, p->scale_dtype);",
     "double w = p->scale_dtype == 1 ? 1.0 : scale_value(p->weights, r * QLIO_HEADS + g, p->scale_dtype);"),
    ("fp32 values read as 1.0", "    return (double)f;\n}", "    return 1.0;\n}"),
    # pre_tokens / next_tokens windows
    ("window checks the last token only",
     "if (in_window(first, pos, pre_tokens, next_tokens) &&\n            in_window(last,",
     "if (in_window(last, pos, pre_tokens, next_tokens) &&\n            in_window(last,"),
    ("next_tokens ignored", "if (t > pos && t - pos > next_tokens)", "if (t > pos && t - pos > next_tokens && 0)"),
    ("pre_tokens off by one", "pos - t > pre_tokens", "pos - t >= pre_tokens"),
    ("window start dropped from the indices", "oi[j] = (int32_t)(lo + top[j]);", "oi[j] = (int32_t)top[j];"),
    ("window scores from entry 0", "sc[j] = score_one(&p, r, b, lo + j, NULL, 0);",
     "sc[j] = score_one(&p, r, b, j, NULL, 0);"),
]

PINS = [
    dec.test_e4m3fn_closed_forms,
    dec.test_e4m3fn_all_codes_match_torch,
    lambda o: None if o is None else dec.test_f16_all_codes_match_numpy(o),
    vis.test_visible_matches_token_brute_force,
    vis.test_row_visible_layouts,
    vis.test_long_context_edges,
    vis.test_window_matches_token_brute_force,
    vis.test_window_defaults_and_special_cases,
    lambda o: op.test_window_restricts_the_candidates(o, 3, 4, 7, 5),
    lambda o: op.test_window_restricts_the_candidates(o, 0, 2, 100, 30),
    sco.test_worked_example,
    sco.test_worked_example_fp8_f32,
    sco.test_single_head_special_case_fp32,
    sco.test_nonnegative_inputs_reduce_to_gemv_fp32,
    sco.test_linearity_fp32,
    lambda o: sco.test_int8_dots_brute_force(o, 0),
    lambda o: sco.test_int8_dots_brute_force(o, 48),
    sco.test_int8_dot_closed_forms,
    sco.test_fp8_dots_exact,
    sco.test_single_head_special_case,
    sco.test_nonnegative_inputs_reduce_to_gemv,
    sco.test_weight_outside_relu_and_scale_inside,
    lambda o: tk.test_topk_matches_stable_argsort(o, 100, 7),
    tk.test_all_equal_scores_take_lowest_indices,
    op.test_output_layout_and_padding,
    op.test_paging_invariance,
    op.test_tnd_equals_bsnd_for_equal_lengths,
    op.test_graph_mode_example_shape,
]


def caught(ora) -> bool:
    for pin in PINS:
        try:
            pin(ora)
        except Exception:
            return True
    return False


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def pins_fail_in_child(lib_path: str) -> bool:
    """Run the pin battery against one build in a fresh interpreter; True if
    any pin failed or the build crashed."""
    code = ("import sys; sys.path.insert(0, %r); import oracle; "
            "from tests.test_oracle_mutants import caught; "
            "sys.exit(3 if caught(oracle.Oracle(%r)) else 0)" % (ROOT, lib_path))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if res.returncode not in (0, 3) and res.returncode > 0:
        raise RuntimeError("pin battery could not run:\n" + res.stderr[-2000:])
    return res.returncode != 0


def test_unmutated_copy_passes_every_pin(tmp_path):
    src = tmp_path / "copy.c"
    src.write_text(open(oracle.SOURCE).read())
    assert not pins_fail_in_child(oracle.compile_source(str(src), str(tmp_path / "copy.so")))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    text = open(oracle.SOURCE).read()
    assert text.count(old) == 1, "mutation site not unique: %s" % name
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.compile_source(str(src), str(tmp_path / "mutant.so"))
    assert pins_fail_in_child(lib), "no pin caught the planted mistake: %s" % name
