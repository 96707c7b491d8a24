"""The quantizer kernels round w / s through an fp64 product instead of an fp32
division: fl32(w / s) == RN32(RN64(w * RN64(1 / s))) whenever s is an fp16 or
bf16 value (at most 11 significant bits) and w an fp32 value.  numpy's float32
division is IEEE, and its float64 product and float64 -> float32 conversion
round to nearest even, so the identity can be checked on the CPU over many
pairs, including the adversarial ones: quotients at and within a few ulps of
half-integers and of fp32 rounding midpoints."""
import numpy as np
import pytest


def _fp64_route(w, s):
    r = 1.0 / s.astype(np.float64)
    return (w.astype(np.float64) * r).astype(np.float32)


def _scales(rng, n, kind):
    if kind == "f16":
        bits = rng.integers(0x0001, 0x7C00, size=n).astype(np.uint16)   # subnormal .. max
        return bits.view(np.float16).astype(np.float32)
    bits = rng.integers(0x0080, 0x7F80, size=n).astype(np.uint32)       # bf16 normals
    return (bits << 16).view(np.float32)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_random_pairs(kind):
    rng = np.random.default_rng(11)
    n = 2_000_000
    s = _scales(rng, n, kind)
    x = rng.uniform(-200, 200, size=n)
    with np.errstate(over="ignore"):
        w = (x * s.astype(np.float64)).astype(np.float32)
    ok = np.isfinite(w) & (w != 0)
    w, s = w[ok], s[ok]
    assert np.array_equal(_fp64_route(w, s), w / s)


@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_near_half_and_midpoints(kind):
    rng = np.random.default_rng(12)
    n = 400_000
    s = _scales(rng, n, kind)
    s = s[(s > 1e-30) & (s < 1e30)]
    n = s.size
    h = rng.integers(-160, 160, size=n) + 0.5
    # w a few fp32 ulps around h * s: quotients at, just above and just below h
    with np.errstate(over="ignore"):
        base = (h * s.astype(np.float64)).astype(np.float32)
    k = rng.integers(-3, 4, size=n).astype(np.int32)
    w = (base.view(np.int32) + k).view(np.float32)
    # and weights whose quotient sits next to an fp32 midpoint (25-bit values)
    m = rng.integers(2**24, 2**25, size=n) | 1
    e = rng.integers(-30, 8, size=n).astype(np.float64)
    with np.errstate(over="ignore"):
        w2 = (m * np.exp2(e - 24) * s.astype(np.float64)).astype(np.float32)
    for ww in (w, w2):
        ok = np.isfinite(ww) & (ww != 0)
        assert np.array_equal(_fp64_route(ww[ok], s[ok]), ww[ok] / s[ok])


def test_rounded_codes_tie_to_even():
    """Exact half-integer quotients survive the fp64 route unchanged, so the
    following round-to-integer still breaks ties to even."""
    s = np.float32(2.0**-6)
    w = (np.array([0.5, 1.5, 2.5, -0.5, -2.5, 7.5], np.float64) * s).astype(np.float32)
    q = np.rint(_fp64_route(w, np.full(w.shape, s, np.float32)))
    assert list(q) == [0, 2, 2, -0, -2, 8]
