"""Exact pins of the quantizer's scale form and scale floor (readings R7 and R2 of oracle/lmh_oracle.c).

Page "radiance_lmhead_int4.py", ``quantize_int4_rows``: the group scale is the
fp32 product of amax with the ratio r / QMAX (a Python double quotient, cast to
fp32 when torch multiplies it into the fp32 tensor), clamped from below at
1e-8 (an fp32 clamp), then rounded to the 16-bit scale type.  Config text of
the tiny head says "fp16 scales = amax/7"; reading R7 takes the module's
literal form, whose 16-bit result differs from RN16(fl32(amax / 7)) for about
one group in 16000.  Reading R2 keeps the page's floor for bf16 scales and uses
the smallest fp16 subnormal (2^-24) for fp16 scales, where 1e-8 underflows.

The expected bits are derived here in exact rational arithmetic, with a
round-to-nearest-even written from the definition of a binary floating-point
format (p significant bits, smallest normal exponent emin, subnormals below),
not from the oracle's C code.  numpy's IEEE fp32 arithmetic is only used to
find inputs where the page's form and the plausible mistakes disagree; every
expected value comes from the Fraction derivation.  A planted-mistake run
compiles altered copies of the oracle source and checks that these pins fail
on each of them.
"""
import ctypes
import functools
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

from oracle import BF16, F16, F32, MSE_RATIOS

QMAX = {4: 7, 8: 127}
# (significant bits, smallest normal exponent) of each binary format
FMT = {"f64": (53, -1022), "f32": (24, -126), F16: (11, -14), BF16: (8, -126)}


def rne(x: Fraction, fmt) -> Fraction:
    """x rounded to the nearest value of the format, ties to an even significand."""
    p, emin = FMT[fmt]
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    e = max(e, emin)  # subnormals share the spacing of the smallest binade
    quantum = Fraction(2) ** (e - p + 1)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def bits16(v: Fraction, sdt) -> int:
    """16-bit pattern of a value that the scale type represents exactly."""
    if sdt == F16:
        h = np.float16(float(v))
        assert Fraction(float(h)) == v
        return int(h.view(np.uint16))
    f = np.float32(float(v))
    assert Fraction(float(f)) == v
    u = int(f.view(np.uint32))
    assert u & 0xFFFF == 0
    return u >> 16


def floor_of(sdt) -> Fraction:
    # bf16: the page's clamp(min=1e-8) on an fp32 tensor (the double 1e-8 cast
    # to fp32); fp16: 2^-24, the smallest positive fp16 value (R2)
    return rne(Fraction(1e-8), "f32") if sdt == BF16 else Fraction(1, 2**24)


def page_scale(amax: float, r: float, bits: int, sdt) -> Fraction:
    """RN16(max(fl32(amax * fl32(RN64(r / qmax))), floor)) in exact arithmetic."""
    c = rne(rne(Fraction(r) / QMAX[bits], "f64"), "f32")
    s32 = rne(Fraction(amax) * c, "f32")
    s32 = max(s32, floor_of(sdt))
    return rne(s32, sdt)


def mistaken_scales(amax: float, r: float, bits: int, sdt):
    """The plausible misreadings of the scale expression, same floor and rounding."""
    a, qm, fl = Fraction(amax), QMAX[bits], floor_of(sdt)
    forms = {
        # fl32(amax * r) / qmax, both steps rounded to fp32
        "mul_first": rne(rne(a * Fraction(r), "f32") / qm, "f32"),
        # the exact value amax * r / qmax rounded once to fp32
        "one_rounding": rne(a * Fraction(r) / qm, "f32"),
        # the ratio rounded to fp32 before the division by qmax
        "ratio_f32_then_div": rne(a * rne(Fraction(r), "f32") / qm, "f32"),
    }
    if r == 1.0:
        forms["amax_div_qmax"] = rne(a / qm, "f32")  # the config text's "amax/7"
    return {k: rne(max(v, fl), sdt) for k, v in forms.items()}


def _np_page(amax, r, bits, sdt):
    """The page's form in numpy fp32 (only to search for discriminating inputs)."""
    c = np.float32(r / QMAX[bits])
    s = np.maximum(amax * c, np.float32(1e-8) if sdt == BF16 else np.float32(2.0**-24))
    return s.astype(np.float16).astype(np.float32) if sdt == F16 else _bf16_round(s)


def _np_alts(amax, r, bits, sdt):
    """Misreadings of the scale in numpy (only to search for inputs)."""
    fl = np.float32(1e-8) if sdt == BF16 else np.float32(2.0**-24)
    qm = np.float32(QMAX[bits])
    alts = [(amax * np.float32(r)) / qm,                                   # multiply first
            (amax.astype(np.float64) * r / QMAX[bits]).astype(np.float32),  # one rounding
            amax * (np.float32(r) / qm)]                                    # fp32 ratio
    out = []
    for s in alts:
        s = np.maximum(s, fl)
        out.append(s.astype(np.float16).astype(np.float32) if sdt == F16 else _bf16_round(s))
    return out


def _bf16_round(s):
    u = s.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def discriminating_amax(r, bits, sdt, want=6, seed=0):
    """amax values (fp32) whose page-form scale differs from a misreading's."""
    rng = np.random.default_rng([seed, bits, int(sdt), int(r * 100)])
    found = []
    for _ in range(40):
        # spread over several binades of realistic weights (1e-3 .. 1)
        amax = (10.0 ** rng.uniform(-3, 0, 400_000)).astype(np.float32)
        page = _np_page(amax, r, bits, sdt)
        diff = np.nonzero(np.any([page != a for a in _np_alts(amax, r, bits, sdt)], axis=0))[0]
        for i in diff:
            a = float(amax[i])
            ps = page_scale(a, r, bits, sdt)
            if any(m != ps for m in mistaken_scales(a, r, bits, sdt).values()):
                found.append(a)
            if len(found) >= want:
                return found
    return found


@functools.lru_cache(maxsize=None)
def _cases(bits, sdt):
    """(ratio, amax) pairs: the discriminating inputs of every ratio, plus
    random ones for every ratio (for r = 0.8 no misreading above ever differs
    at 16 bits: 0.8 / qmax is close enough to its fp32 value that every fp32
    result near an fp16 or bf16 rounding midpoint comes out the same)."""
    out = []
    for r in MSE_RATIOS:
        for a in discriminating_amax(r, bits, sdt, want=4):
            out.append((r, a))
    rng = np.random.default_rng([3, bits, int(sdt)])
    for r in MSE_RATIOS:
        for a in (10.0 ** rng.uniform(-3, 0, 4)).astype(np.float32):
            out.append((r, float(a)))
    return tuple(out)


def _discriminating(bits, sdt):
    return {r for r, a in _cases(bits, sdt)
            if any(m != page_scale(a, r, bits, sdt) for m in mistaken_scales(a, r, bits, sdt).values())}


def _quantize_groups(quant, amaxes, r, bits, sdt):
    """One group of 64 columns per amax: the maximum at column 5, smaller
    entries elsewhere (so amax is the group's largest magnitude)."""
    G = 64
    w = np.zeros((len(amaxes), G), dtype=np.float32)
    for i, a in enumerate(amaxes):
        w[i, 5] = a if i % 2 == 0 else -a
        w[i, 9] = np.float32(a) * np.float32(0.5)
        w[i, 40] = -np.float32(a) * np.float32(0.25)
    q, s = quant(w, bits, G, sdt, (r,))
    return s[:, 0]


# ---------------------------------------------------------------- R7 pins

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", [F16, BF16])
def test_scale_form_is_the_pages_literal_expression(orc, bits, sdt):
    cases = _cases(bits, sdt)
    # the ratios 1.0 .. 0.85 each contribute inputs on which a misreading
    # gives other bits (the config text's amax/7 among them for r = 1.0)
    assert {1.0, 0.95, 0.9, 0.85} <= _discriminating(bits, sdt)
    for r in MSE_RATIOS:
        amaxes = [a for rr, a in cases if rr == r]
        got = _quantize_groups(orc.quantize, amaxes, r, bits, sdt)
        for a, g in zip(amaxes, got):
            want = bits16(page_scale(a, r, bits, sdt), sdt)
            assert int(g) == want, (r, a, hex(int(g)), hex(want))


@pytest.mark.parametrize("sdt", [F16, BF16])
def test_amax_over_7_differs_from_the_page_form(sdt):
    """The config text's amax/7 and the module's amax*(1/7) give different fp16
    and bf16 scales on some groups, so the reading matters (R7)."""
    amaxes = discriminating_amax(1.0, 4, sdt, want=3, seed=7)
    assert amaxes
    for a in amaxes:
        m = mistaken_scales(a, 1.0, 4, sdt)
        assert any(v != page_scale(a, 1.0, 4, sdt) for v in m.values())


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", [F16, BF16])
def test_mse_scale_is_one_of_the_five_page_scales(orc, bits, sdt):
    """Under the 5-ratio search every stored scale equals, bit for bit, the page
    form of one of the ratios, and the recorded pick names that ratio."""
    rng = np.random.default_rng([11, bits, int(sdt)])
    w = (rng.standard_normal((48, 128)) * 0.02).astype(np.float32)
    w[rng.random(w.shape) < 0.01] *= 8
    q, s, pick = orc.quantize(w, bits, 64, sdt, MSE_RATIOS, return_pick=True)
    amax = np.abs(w).reshape(48, 2, 64).max(-1)
    for v in range(48):
        for g in range(2):
            r = MSE_RATIOS[int(pick[v, g])]
            assert int(s[v, g]) == bits16(page_scale(float(amax[v, g]), r, bits, sdt), sdt)


# ---------------------------------------------------------------- R2 pins

def test_bf16_floor_is_the_pages_clamp(orc):
    """A tiny bf16-scale group takes bf16(fl32(1e-8)): the page's clamp value
    rounded to bf16 (R2)."""
    want = bits16(rne(rne(Fraction(1e-8), "f32"), BF16), BF16)
    assert want == 0x322C  # 1.0011717677e-08, the bf16 neighbour of 1e-8
    for bits in (4, 8):
        for amax in (1e-12, 3e-9, 1e-20):
            got = _quantize_groups(orc.quantize, [amax], 1.0, bits, BF16)[0]
            assert int(got) == want, (bits, amax, hex(int(got)))


def test_fp16_floor_is_the_smallest_subnormal(orc):
    """A tiny fp16-scale group takes 2^-24, fp16 bits 0x0001 (R2)."""
    for bits in (4, 8):
        for amax in (1e-9, 2e-10, 1e-30):
            got = _quantize_groups(orc.quantize, [amax], 1.0, bits, F16)[0]
            assert int(got) == 0x0001, (bits, amax, hex(int(got)))


def test_floor_boundary(orc):
    """Just above the floor the product itself is rounded (no clamp); the
    derivation decides both sides."""
    for sdt in (F16, BF16):
        c = rne(rne(Fraction(1, 7), "f64"), "f32")
        a_floor = floor_of(sdt) / c
        for f in (0.5, 0.99, 1.01, 2.0, 5.0):
            a = float(np.float32(float(a_floor) * f))
            got = _quantize_groups(orc.quantize, [a], 1.0, 4, sdt)[0]
            assert int(got) == bits16(page_scale(a, 1.0, 4, sdt), sdt), (sdt, f)


# ---------------------------------------------------------------- planted mistakes

_MUTANTS = {
    # the config text's "amax/7" instead of amax * fl32(r/qmax)
    "amax_div_qmax": ("float s32 = amax * c;", "float s32 = amax * (float)ratios[i] / (float)qmax;"),
    # the ratio multiplied in first, then divided by qmax
    "mul_first": ("float s32 = amax * c;", "float s32 = (amax * (float)ratios[i]) / (float)qmax;"),
    # no floor at all
    "no_floor": ("if (s32 < floor_s) s32 = floor_s;", ""),
    # the page's 1e-8 floor for fp16 scales as well
    "bf16_floor_everywhere": ("(float)ldexp(1.0, -24)", "1e-8f"),
}


def _build_mutant(tmp_path, name):
    src = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "oracle", "lmh_oracle.c")
    text = open(src).read()
    old, new = _MUTANTS[name]
    # the change goes into the symmetric quantizer only
    lo, hi = text.index("int orc_quantize("), text.index("int orc_quantize_asym(")
    body = text[lo:hi]
    assert body.count(old) == 1, f"planted mistake {name}: anchor not found once"
    path = tmp_path / f"orc_{name}.c"
    path.write_text(text[:lo] + body.replace(old, new) + text[hi:])
    so = tmp_path / f"liborc_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", str(so), str(path), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.orc_quantize.restype = i32
    lib.orc_quantize.argtypes = [vp, i32, i64, i64, i32, i64, i32, vp, i32, vp, vp, vp]

    def quant(w, bits, G, sdt, ratios):
        w = np.ascontiguousarray(w, dtype=np.float32)
        V, K = w.shape
        q = np.empty((V, K), dtype=np.int8)
        s = np.empty((V, K // G), dtype=np.uint16)
        r = np.ascontiguousarray(np.array(ratios, dtype=np.float64))
        rc = lib.orc_quantize(w.ctypes.data, F32, V, K, bits, G, sdt, r.ctypes.data, len(r),
                              q.ctypes.data, s.ctypes.data, None)
        assert rc == 0
        return q, s

    return quant


def _pins_hold(quant):
    """The R7 and R2 pins above, run against another quantizer."""
    for bits in (4, 8):
        for sdt in (F16, BF16):
            for r, a in _cases(bits, sdt):
                if int(_quantize_groups(quant, [a], r, bits, sdt)[0]) != \
                        bits16(page_scale(a, r, bits, sdt), sdt):
                    return False
    if int(_quantize_groups(quant, [1e-12], 1.0, 4, BF16)[0]) != 0x322C:
        return False
    if int(_quantize_groups(quant, [1e-9], 1.0, 4, F16)[0]) != 0x0001:
        return False
    return True


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the planted mistakes")
@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_planted_mistakes_fail_the_pins(tmp_path, name):
    assert not _pins_hold(_build_mutant(tmp_path, name)), name


def test_pins_hold_on_the_oracle(orc):
    assert _pins_hold(orc.quantize)
