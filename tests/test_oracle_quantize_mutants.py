"""The producer oracle's pins have teeth: each plausible mistake below is
planted in a copy of oracle/quantize.py (loaded as a separate module on the
CPU), and at least one pin of tests/test_oracle_quantize.py must fail
against it."""
import importlib.util
import os

import pytest

import oracle
from tests import test_oracle_quantize as pins

SOURCE = os.path.join(os.path.dirname(oracle.__file__), "quantize.py")

MUTANTS = [
    ("rint replaced by floor", "np.rint(x[i] * r)", "np.floor(x[i] * r)"),
    ("int8 clamp at -128", "np.clip(np.rint(x[i] * r), -127, 127)", "np.clip(np.rint(x[i] * r), -128, 127)"),
    ("int8 scale from 128", "(amax / np.float32(127.0))", "(amax / np.float32(128.0))"),
    ("int8 scale not capped", "s16[np.isinf(s16)] = np.float16(65504.0)", "pass"),
    ("fp8 scale from 240", "amax / np.float32(448.0)", "amax / np.float32(240.0)"),
    ("e4m3 ties to odd", "(hi % 2 == 0)", "(hi % 2 == 1)"),
    ("e4m3 sign dropped", "sign = np.signbit(y.ravel()).astype(np.uint8) << 7", "sign = np.zeros(y.size, np.uint8)"),
    ("bf16 decode shift", "astype(np.uint32) << 16)", "astype(np.uint32) << 15)"),
    ("append block from remainder", "bt[b * max_blocks + p // block_size]", "bt[b * max_blocks + p % block_size]"),
    ("append stride ignored", "key_cache[blk * stride + o * 128: blk * stride + o * 128 + 128]",
     "key_cache[blk * block_size * 128 + o * 128: blk * block_size * 128 + o * 128 + 128]"),
    ("append bound off by one", "p // block_size >= max_blocks", "p // block_size > max_blocks"),
]

PINS = [
    lambda: pins.test_bf16_decode_is_top_half_of_fp32(),
    lambda: pins.test_e4m3fn_encoder_matches_torch(),
    lambda: pins.test_e4m3fn_encoder_keeps_sign_of_zero(),
    lambda: [pins.test_single_spike_takes_the_extreme_code(q) for q in (0, 1)],
    lambda: [pins.test_zero_and_constant_rows(q) for q in (0, 1)],
    lambda: pins.test_int8_rounding_bound_and_clamp(),
    lambda: pins.test_e4m3_dequant_error_within_half_spacing(),
    lambda: [pins.test_sign_and_power_of_two_invariance(q) for q in (0, 1)],
    lambda: pins.test_int8_scale_saturates_at_fp16_max(),
    lambda: [pins.test_append_paging_invariance_and_skips(q) for q in (0, 1)],
]


def load_mutant(old: str, new: str):
    with open(SOURCE) as f:
        text = f.read()
    assert text.count(old) == 1, "mutation site must be unique: %r" % old
    spec = importlib.util.spec_from_loader("oracle._quantize_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    exec(compile(text.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


def test_original_passes_every_pin():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, old, new):
    monkeypatch.setattr(pins, "oq", load_mutant(old, new))
    caught = 0
    for pin in PINS:
        try:
            pin()
        except Exception:
            caught += 1
    assert caught > 0, "no pin catches the planted mistake: %s" % name
