"""Pins for the oracle's 16-bit float codecs.

The codecs are written from the IEEE-754 binary16 and bfloat16 definitions.
They are pinned against independent library conversions (numpy's float16 cast,
torch's bfloat16 cast), which implement the same round-to-nearest-even rule,
over every 16-bit pattern, every midpoint between neighbouring 16-bit values
(the ties) and a large sample of random float32 bit patterns.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, F16


def _all_f16_values():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return h


def _np_bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _same_bits_or_both_nan(got, want, dtype):
    emask = 0x7C00 if dtype == F16 else 0x7F80
    mmask = 0x03FF if dtype == F16 else 0x007F
    nan_got = ((got & emask) == emask) & ((got & mmask) != 0)
    nan_want = ((want & emask) == emask) & ((want & mmask) != 0)
    assert np.array_equal(nan_got, nan_want)
    ok = nan_got | (got == want)
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, f"first mismatches at {bad[:5]}: got {got[bad[:5]]}, want {want[bad[:5]]}"


def test_f16_decode_all_patterns(orc):
    h = _all_f16_values()
    got = orc.widen16(h, F16)
    want = h.view(np.float16).astype(np.float32)
    both_nan = np.isnan(got) & np.isnan(want)
    assert np.array_equal(got[~both_nan], want[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(want))


def test_bf16_decode_all_patterns(orc):
    h = _all_f16_values()
    got = orc.widen16(h, BF16)
    # bfloat16 is by definition the top half of a binary32 pattern
    want = (h.astype(np.uint32) << 16).view(np.float32)
    both_nan = np.isnan(got) & np.isnan(want)
    assert np.array_equal(got[~both_nan], want[~both_nan])


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_encode_roundtrips_every_value(orc, dtype):
    h = _all_f16_values()
    vals = orc.widen16(h, dtype)
    fin = np.isfinite(vals)
    back = orc.encode16(vals[fin], dtype)
    assert np.array_equal(back, h[fin])


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_encode_midpoints_round_to_even(orc, dtype):
    """Every midpoint between two neighbouring finite 16-bit values (exact in fp32)
    must round to the neighbour with the even mantissa."""
    h = np.arange(0, 0x7C00 if dtype == F16 else 0x7F80, dtype=np.uint32).astype(np.uint16)
    lo = orc.widen16(h[:-1], dtype).astype(np.float64)
    hi = orc.widen16(h[1:], dtype).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # exactly representable
    got = orc.encode16(mid, dtype)
    even = np.where(h[:-1] % 2 == 0, h[:-1], h[1:])
    assert np.array_equal(got, even)
    got_neg = orc.encode16(-mid, dtype)
    assert np.array_equal(got_neg, even | 0x8000)


def test_f16_encode_vs_numpy_random_patterns(orc):
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # concentrate half of them near the binary16 range
    u[::2] = (u[::2] & 0x807FFFFF) | (rng.integers(100, 145, size=u[::2].size).astype(np.uint32) << 23)
    f = u.view(np.float32)
    got = orc.encode16(f, F16)
    with np.errstate(over="ignore"):
        want = f.astype(np.float16).view(np.uint16)
    _same_bits_or_both_nan(got, want, F16)


def test_bf16_encode_vs_torch_random_patterns(orc):
    rng = np.random.default_rng(6)
    u = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    got = orc.encode16(f, BF16)
    want = _np_bf16_bits(f)
    _same_bits_or_both_nan(got, want, BF16)


def test_encode_special_values(orc):
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 2**-24, 2**-25,
                     2**-25 * 1.0000001, 2**-14, 1e-8], dtype=np.float32)
    got = orc.encode16(vals, F16)
    want = [0x0000, 0x8000, 0x7C00, 0xFC00, 0x7BFF, 0x7BFF, 0x7C00, 0x0001, 0x0000, 0x0001,
            0x0400, 0x0000]
    assert [int(g) for g in got] == want
    # bf16: 1e-8 is a normal bfloat16 number (the page's scale floor)
    b = orc.f32_to_bf16_bits(1e-8)
    assert b == int(_np_bf16_bits(np.array([1e-8], np.float32))[0])
    assert 0 < orc.bf16_bits_to_f32(b) < 1.01e-8
