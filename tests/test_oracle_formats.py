"""Pins for the oracle's binary16 / bfloat16 decode and RNE encode.

Independent references: numpy's float16 type (decode, and double -> half
conversion), the bfloat16 definition as the top half of a binary32, torch's
float32 -> bfloat16 conversion, and hand-built tie cases.
"""
import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _same(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_f16_decode_exhaustive():
    ours = oracle.decode(ALL, "f16")
    ref = ALL.view(np.float16).astype(np.float64)
    assert _same(ours, ref)
    # signed zeros keep their sign
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_bf16_decode_exhaustive():
    ours = oracle.decode(ALL, "bf16")
    ref = (ALL.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert _same(ours, ref)


def test_f16_encode_matches_numpy_random():
    rng = np.random.default_rng(0)
    mag = np.exp2(rng.uniform(-30, 17, size=200000))
    x = mag * rng.choice([-1.0, 1.0], size=mag.size)
    ours = oracle.encode(x, "f16")
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_encode_roundtrip_exhaustive():
    vals = oracle.decode(ALL, "f16")
    finite = np.isfinite(vals)
    back = oracle.encode(vals[finite], "f16")
    assert np.array_equal(back, ALL[finite])


@pytest.mark.parametrize("x,expect", [
    (1.0 + 2.0**-11, 1.0),                       # tie -> even fraction (0)
    (1.0 + 3 * 2.0**-11, 1.0 + 2.0**-9),         # tie -> even fraction (2)
    (1.0 + 2.0**-11 + 2.0**-30, 1.0 + 2.0**-10), # just above the tie rounds up
    (2.0**-25, 0.0),                             # half the smallest subnormal -> 0 (even)
    (3 * 2.0**-25, 2 * 2.0**-24),                # subnormal tie -> even
    (2.0**-14 - 2.0**-26, 2.0**-14),             # rounds up into the normal range
    (65519.99, 65504.0),                          # below the overflow threshold
    (65520.0, np.inf),                            # tie at the top rounds to infinity
    (-65520.0, -np.inf),
])
def test_f16_encode_ties_and_edges(x, expect):
    got = oracle.decode(oracle.encode(np.array([x]), "f16"), "f16")[0]
    assert got == expect


def test_bf16_encode_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    mag = np.exp2(rng.uniform(-120, 120, size=200000)).astype(np.float32)
    x32 = mag * rng.choice([-1.0, 1.0], size=mag.size).astype(np.float32)
    ours = oracle.encode(x32.astype(np.float64), "bf16")
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("x,expect", [
    (1.0 + 2.0**-8, 1.0),                        # tie -> even
    (1.0 + 3 * 2.0**-8, 1.0 + 2.0**-6),          # tie -> even
    (1.0 + 2.0**-8 + 2.0**-40, 1.0 + 2.0**-7),   # one rounding from the exact value rounds up
    (-(1.0 + 2.0**-8 + 2.0**-40), -(1.0 + 2.0**-7)),
])
def test_bf16_encode_single_rounding(x, expect):
    got = oracle.decode(oracle.encode(np.array([x]), "bf16"), "bf16")[0]
    assert got == expect


def test_nan_and_inf_encode():
    e = oracle.encode(np.array([np.nan, np.inf, -np.inf]), "f16")
    d = oracle.decode(e, "f16")
    assert np.isnan(d[0]) and d[1] == np.inf and d[2] == -np.inf
