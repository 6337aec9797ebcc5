"""Pins for the oracle's element decoding (int8 is the identity).

FLOAT8_e4m3fn and FLOAT16 are the q/k and scale dtypes of the
VllmQuantLightningIndexer page's parameter table.  The oracle decodes them
from the bit fields; here every code is compared with an independent
library conversion, plus closed-form values of the OCP E4M3FN definition.
"""
import math

import numpy as np

from tests._helpers import e4m3_table


def test_e4m3fn_all_codes_match_torch(ora):
    lib = e4m3_table()
    for code in range(256):
        v = ora.e4m3fn_value(code)
        if math.isnan(lib[code]):
            assert math.isnan(v), code
        else:
            assert v == lib[code], (code, v, lib[code])


def test_e4m3fn_closed_forms(ora):
    # bias 7, no infinities, max normal 448, min subnormal 2^-9, NaN S.1111.111
    assert ora.e4m3fn_value(0x38) == 1.0
    assert ora.e4m3fn_value(0xB8) == -1.0
    assert ora.e4m3fn_value(0x7E) == 448.0
    assert ora.e4m3fn_value(0xFE) == -448.0
    assert ora.e4m3fn_value(0x01) == 2.0 ** -9
    assert ora.e4m3fn_value(0x07) == 7 * 2.0 ** -9
    assert ora.e4m3fn_value(0x08) == 2.0 ** -6
    assert ora.e4m3fn_value(0x78) == 256.0          # exponent 15 is finite in FN
    assert math.isnan(ora.e4m3fn_value(0x7F)) and math.isnan(ora.e4m3fn_value(0xFF))
    assert ora.e4m3fn_value(0x00) == 0.0
    assert math.copysign(1.0, ora.e4m3fn_value(0x80)) == -1.0


def test_f16_all_codes_match_numpy(ora):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([ora.f16_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero and subnormal edge
    assert math.copysign(1.0, ora.f16_value(0x8000)) == -1.0
    assert ora.f16_value(0x0001) == 2.0 ** -24
    assert ora.f16_value(0x3C00) == 1.0
