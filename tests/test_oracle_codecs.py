"""Pins for the oracle's exact codecs against library casts and closed forms.

bf16 decode ("GLM on an A100, in Vx", section "INT4, FP8 and BF16": exact for
all 65,536 encodings, subnormals, infinities and NaN kept) and e4m3fn decode
("Self-contained GLM-5 serving stack", checkpoint IO: FP8 E4M3FN)."""
import math

import numpy as np
import torch


def test_bf16_all_encodings_match_torch_cast(oracle_mod):
    lib = oracle_mod._load()
    codes = np.arange(1 << 16, dtype=np.uint32)
    ref = torch.from_numpy(codes.astype(np.int32).astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([lib.oracle_bf16_to_double(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros are kept
    assert math.copysign(1.0, got[0x8000]) == -1.0 and got[0x8000] == 0.0


def test_bf16_closed_forms(oracle_mod):
    f = oracle_mod.bf16_to_double
    assert f(0x3F80) == 1.0
    assert f(0xBF80) == -1.0
    assert f(0x4049) == 3.140625
    assert f(0x0001) == 2.0 ** -133          # smallest subnormal: 1/128 * 2^-126
    assert f(0x0080) == 2.0 ** -126          # smallest normal
    assert f(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127
    assert f(0x7F80) == math.inf and f(0xFF80) == -math.inf
    assert math.isnan(f(0x7FC0)) and math.isnan(f(0x7F81))


def test_e4m3fn_all_encodings_match_torch_cast(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_mod.e4m3fn_to_double(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert nan.sum() == 2                     # 0x7F and 0xFF only
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3fn_closed_forms(oracle_mod):
    f = oracle_mod.e4m3fn_to_double
    assert f(0x7E) == 448.0                   # largest finite: 1.75 * 2^8
    assert f(0xFE) == -448.0
    assert f(0x01) == 2.0 ** -9               # smallest subnormal: 1/8 * 2^-6
    assert f(0x07) == 7 * 2.0 ** -9
    assert f(0x08) == 2.0 ** -6               # smallest normal
    assert f(0x38) == 1.0                     # exponent 7 = bias
    assert f(0x3C) == 1.5
    assert f(0x00) == 0.0 and math.copysign(1.0, f(0x80)) == -1.0
    assert math.isnan(f(0x7F)) and math.isnan(f(0xFF))
    # no infinity: 0x78..0x7E are ordinary values 256..448
    assert [f(c) for c in range(0x78, 0x7F)] == [256.0, 288.0, 320.0, 352.0, 384.0, 416.0, 448.0]
