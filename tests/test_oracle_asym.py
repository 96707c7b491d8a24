"""Pins for the oracle's asymmetric (zero-point) form: the quantizer
oracle.quantize_asym, the packed form pack_zp/unpack_zp, logits_zp and
embed_zp (w ~ (n - z) * s with unsigned codes n and a per-group zero point z;
the module page's kernel subtracts a fixed 8 from every nibble, the asymmetric
checkpoint on the other page has a per-group value there; reading R21 of oracle/lmh_oracle.c).

None of these re-types the oracle's formula.  They check:
  * a known answer: groups built on an exact grid (k - z0) * s0 that include
    both ends of the code range come back as (k, s0, z0);
  * invariants that the mathematics fixes: code range, zero kept exact, the
    reconstruction error bound derived from the 16-bit rounding of s,
    monotone codes, every code a nearest level of (s, z) in exact rationals,
    z a nearest integer to -lo/s, s*qr within rounding of hi - lo;
  * reductions: z = 8 / 128 with n = q + 8 / q + 128 gives the symmetric
    oracle's logits and embedding rows bit for bit; logits_zp equals the
    dense-logits oracle on the dequantized table; embed_zp equals logits_zp
    on one-hot inputs;
  * the packed bytes of a hand-built example at hand-derived offsets.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import BF16, F16, F32

QR = {4: 15, 8: 255}
U16 = {F16: Fraction(1, 2**11), BF16: Fraction(1, 2**8)}  # unit roundoff of the scale type


def _f(x) -> Fraction:
    return Fraction(float(x))


def _skewed(V, K, seed):
    """Gaussian weights with a per-row offset, so groups are lopsided."""
    w = synth.random_weight((V, K), 0.02, seed, ())
    off = np.random.default_rng(seed + 100).uniform(-0.03, 0.03, size=(V, 1)).astype(np.float32)
    return (w + off).astype(np.float32)


def _grid_case(bits, sdt, G, seed):
    """Rows built on an exact grid: w = (k - z0) * s0 with both k = 0 and k = qr present."""
    rng = np.random.default_rng(seed)
    qr = QR[bits]
    V = 12
    s0_f = rng.uniform(1e-4, 3e-2, size=V).astype(np.float32)
    if sdt == F16:
        s0_f = s0_f.astype(np.float16).astype(np.float32)
    else:
        s0_f = torch.from_numpy(s0_f).to(torch.bfloat16).float().numpy()
    z0 = rng.integers(0, qr + 1, size=V)
    z0[0], z0[1] = 0, qr                       # one-sided groups: all >= 0, all <= 0
    k = rng.integers(0, qr + 1, size=(V, G))
    k[:, 0], k[:, 1] = 0, qr
    w = ((k - z0[:, None]).astype(np.float32) * s0_f[:, None]).astype(np.float32)
    # exact in fp32: an integer of <= 9 bits times a 16-bit value
    assert all(_f(w[v, j]) == (int(k[v, j]) - int(z0[v])) * _f(s0_f[v])
               for v in range(V) for j in range(G))
    return w, k, z0, s0_f


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", [F16, BF16])
def test_exact_grid_groups_are_recovered(orc, bits, sdt):
    G = 64
    w, k, z0, s0 = _grid_case(bits, sdt, G, seed=bits * 10 + sdt)
    n, s, z = orc.quantize_asym(w, bits, G, sdt)
    assert np.array_equal(n, k.astype(np.uint8))
    assert np.array_equal(z[:, 0], z0.astype(np.uint8))
    assert np.array_equal(orc.widen16(s, sdt)[:, 0], s0)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", [F16, BF16])
def test_one_sided_groups_extend_the_range_to_zero(orc, bits, sdt):
    # w = k * s0 with k in [kmin, qr], kmin > 0 (no zero element): the range
    # [0, qr * s0] still includes zero, so s = s0, z = 0 and n = k; mirrored
    # (w = (k - qr) * s0, k in [0, kmax]) it gives z = qr
    qr = QR[bits]
    G = 32
    rng = np.random.default_rng(bits + 3 * sdt)
    s0 = np.float32(2.0**-7 * 1.5)
    k = rng.integers(qr // 3, qr + 1, size=(2, G))
    k[:, 0] = qr
    w = np.empty((2, G), dtype=np.float32)
    w[0] = (k[0] * s0).astype(np.float32)
    w[1] = (-k[1] * s0).astype(np.float32)
    n, s, z = orc.quantize_asym(w, bits, G, sdt)
    assert (orc.widen16(s, sdt)[:, 0] == s0).all()
    assert z[0, 0] == 0 and z[1, 0] == qr
    assert np.array_equal(n[0], k[0].astype(np.uint8))
    assert np.array_equal(n[1], (qr - k[1]).astype(np.uint8))


def test_rounded_down_scale_clamps_zero_point_and_codes(orc):
    # int8, bf16 scales (8 significant bits), hi = 0, lo = -255.97: the exact
    # scale 255.97 / 255 = 1.0038... rounds down to 1.0 (the next bf16 value is
    # 1.0078125), so -lo / s = 255.97 rounds to 256, past the code range: z
    # clamps to 255, and w = lo gives rint(-255.97) + 255 = -1, clamped to 0
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = -255.97
    w[0, 1] = -100.0
    n, s, z = orc.quantize_asym(w, 8, 32, BF16)
    assert orc.widen16(s, BF16)[0, 0] == 1.0
    assert z[0, 0] == 255
    assert n[0, 0] == 0 and n[0, 1] == 155 and (n[0, 2:] == 255).all()


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", [F16, BF16])
def test_range_zero_groups_and_zero_exact(orc, bits, sdt):
    w = _skewed(40, 256, 1)
    w[3] = 0.0
    w[7, 64:128] = 0.0
    w[9, 5] = 0.0                                 # an exact zero inside a live group
    w[10, :64] = np.abs(w[10, :64])               # one-sided groups
    w[11, :64] = -np.abs(w[11, :64])
    n, s, z = orc.quantize_asym(w, bits, 64, sdt)
    qr = QR[bits]
    assert n.max() <= qr and z.max() <= qr
    assert (s[3] == 0).all() and (z[3] == 0).all() and (n[3] == 0).all()
    assert s[7, 1] == 0 and z[7, 1] == 0 and (n[7, 64:128] == 0).all()
    assert n[9, 5] == z[9, 0]                     # zero dequantizes to exactly zero
    assert z[10, 0] == 0                          # lo = 0
    assert z[11, 0] == qr                         # hi = 0 and -lo/s rounds to qr
    assert n[10, :64].max() == qr and n[11, :64].min() == 0


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", [F16, BF16])
def test_error_bound_and_monotone_codes(orc, bits, sdt):
    V, K, G = 48, 512, 64
    w = _skewed(V, K, 2)
    n, s, z = orc.quantize_asym(w, bits, G, sdt)
    qr = QR[bits]
    sv = orc.widen16(s, sdt).astype(np.float64)
    s_el = np.repeat(sv, G, axis=1)
    z_el = np.repeat(z.astype(np.float64), G, axis=1)
    wd = w.astype(np.float64)
    err = np.abs((n.astype(np.float64) - z_el) * s_el - wd)
    lo = np.minimum(wd.reshape(V, -1, G).min(-1), 0.0)
    hi = np.maximum(wd.reshape(V, -1, G).max(-1), 0.0)
    # s/2 from rounding, plus what the 16-bit rounding of s can push past the ends
    bound = s_el * 0.5 + np.repeat((hi - lo) * float(U16[sdt]) * 1.001, G, axis=1) + 1e-30
    assert (err <= bound).all()
    # codes are non-decreasing in w inside a group
    for v in range(V):
        for g in range(K // G):
            order = np.argsort(w[v, g * G:(g + 1) * G], kind="stable")
            assert (np.diff(n[v, g * G:(g + 1) * G][order].astype(int)) >= 0).all()


def _nearest(t: Fraction, lo: int, hi: int):
    """Integers in [lo, hi] nearest to t (exact)."""
    best, out = None, []
    for c in range(lo, hi + 1):
        d = abs(c - t)
        if best is None or d < best:
            best, out = d, [c]
        elif d == best:
            out.append(c)
    return out


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", [F16, BF16])
def test_codes_zero_points_and_scales_brute_force(orc, bits, sdt):
    V, K, G = 6, 64, 32
    w = _skewed(V, K, 3)
    w[2, :32] *= 8.0
    n, s, z = orc.quantize_asym(w, bits, G, sdt)
    qr = QR[bits]
    sv = orc.widen16(s, sdt)
    eps = Fraction(1, 2**20)
    for v in range(V):
        for g in range(K // G):
            grp = [_f(x) for x in w[v, g * G:(g + 1) * G]]
            lo, hi = min(min(grp), 0), max(max(grp), 0)
            sf, zg = _f(sv[v, g]), int(z[v, g])
            # s * qr is (hi - lo) up to the 16-bit rounding of s
            assert abs(sf * qr - (hi - lo)) <= (hi - lo) * (U16[sdt] + Fraction(1, 2**22))
            # z is a nearest integer to -lo / s in [0, qr]
            t = -lo / sf
            cz = _nearest(t, 0, qr)
            if abs(t - (t.numerator // t.denominator) - Fraction(1, 2)) > eps:
                assert zg in cz, (v, g)
            for j, wf in enumerate(grp):
                # n - z is a nearest integer to w / s among the representable codes
                t = wf / sf
                cands = _nearest(t, -zg, qr - zg)
                if abs(t - (t.numerator // t.denominator) - Fraction(1, 2)) > eps:
                    assert int(n[v, g * G + j]) - zg in cands, (v, g, j)


def test_ties_go_to_even(orc):
    # hi - lo = 15 * 2^-6 exactly, so s = 2^-6 (fp16 and fp32 exact) and z = 4:
    # w / s = -3.5 -> -4 (even), 2.5 -> 2 (even), 0.5 -> 0
    s0 = 2.0**-6
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0], w[0, 1] = -4 * s0, 11 * s0
    w[0, 2], w[0, 3], w[0, 4] = -3.5 * s0, 2.5 * s0, 0.5 * s0
    n, s, z = orc.quantize_asym(w, 4, 32, F16)
    assert orc.widen16(s, F16)[0, 0] == s0 and z[0, 0] == 4
    assert list(n[0, :5]) == [0, 15, 0, 6, 4]


def test_16bit_weights_widen_exactly(orc):
    w = _skewed(16, 128, 4)
    h = w.astype(np.float16)
    a = orc.quantize_asym(h, 4, 32, F16)
    b = orc.quantize_asym(h.astype(np.float32), 4, 32, F16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    bb = torch.from_numpy(w).to(torch.bfloat16)
    a = orc.quantize_asym(bb.view(torch.int16).numpy().view(np.uint16), 8, 64, BF16, w_dtype=BF16)
    b = orc.quantize_asym(bb.float().numpy(), 8, 64, BF16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---- packed form ------------------------------------------------------------------

@pytest.mark.parametrize("bits,K,G,V", [(4, 256, 64, 70), (4, 512, 128, 64), (8, 128, 32, 129),
                                        (8, 256, 256, 1)])
def test_zp_roundtrip_ragged(orc, bits, K, G, V):
    rng = np.random.default_rng(V + K)
    n = rng.integers(0, QR[bits] + 1, size=(V, K)).astype(np.uint8)
    s = rng.integers(0, 0x7C00, size=(V, K // G)).astype(np.uint16)
    z = rng.integers(0, QR[bits] + 1, size=(V, K // G)).astype(np.uint8)
    blob = orc.pack_zp(n, s, z, bits, G)
    vpad = (V + 63) // 64 * 64
    assert len(blob) == vpad * K * bits // 8 + vpad * (K // G) * 3
    n2, s2, z2 = orc.unpack_zp(blob, V, K, bits, G)
    assert np.array_equal(n, n2) and np.array_equal(s, s2) and np.array_equal(z, z2)


@pytest.mark.parametrize("bits", [4, 8])
def test_zp_codes_and_scales_share_the_symmetric_layout(orc, bits):
    # with V a multiple of 64 (no padding rows) the code and scale regions are
    # the symmetric blob of q = n - 8 (int4) / n - 128 (int8), byte for byte
    V, K, G = 128, 256, 64
    rng = np.random.default_rng(bits)
    n = rng.integers(0, QR[bits] + 1, size=(V, K)).astype(np.uint8)
    s = rng.integers(0, 0x7C00, size=(V, K // G)).astype(np.uint16)
    z = rng.integers(0, QR[bits] + 1, size=(V, K // G)).astype(np.uint8)
    q = (n.astype(np.int16) - (8 if bits == 4 else 128)).astype(np.int8)
    sym = orc.pack(q, s, bits, G)
    zp = orc.pack_zp(n, s, z, bits, G)
    assert np.array_equal(zp[:len(sym)], sym)
    assert len(zp) == len(sym) + V * (K // G)


def test_zp_region_hand_bytes(orc):
    # V = 70 (two 64-row blocks), K = 128, G = 64: NG = 2.  The zero-point
    # region starts after 128 * 64 code bytes (int4) and 128 * 2 * 2 scale
    # bytes.  Block b, group g, row r sits at (b*2 + g)*64 + 4*(r % 16) + r // 16.
    V, K, G = 70, 128, 64
    n = np.zeros((V, K), dtype=np.uint8)
    s = np.zeros((V, 2), dtype=np.uint16)
    z = np.zeros((V, 2), dtype=np.uint8)
    z[0, 0], z[16, 0], z[32, 0], z[48, 0] = 1, 2, 3, 4    # one lane's word: bytes 0..3
    z[1, 0] = 5                                          # byte 4
    z[17, 1] = 6                                         # (0*2+1)*64 + 4*1 + 1 = 69
    z[64, 0] = 7                                         # (1*2+0)*64 + 0 = 128
    z[69, 1] = 9                                         # (1*2+1)*64 + 4*5 + 0 = 212
    blob = orc.pack_zp(n, s, z, 4, G)
    base = 128 * 64 + 128 * 2 * 2
    region = blob[base:]
    assert len(region) == 128 * 2
    want = np.zeros(256, dtype=np.uint8)
    want[[0, 1, 2, 3, 4, 69, 128, 212]] = [1, 2, 3, 4, 5, 6, 7, 9]
    assert np.array_equal(region, want)
    # padding rows: code 0, scale 0, zero point 0
    assert (blob[:base] == 0).all()


# ---- logits and embedding rows ------------------------------------------------------

def _table(V, K, G, bits, sdt, seed):
    rng = np.random.default_rng(seed)
    n = rng.integers(0, QR[bits] + 1, size=(V, K)).astype(np.uint8)
    lo, hi = (0x0001, 0x5800) if sdt == F16 else (0x3000, 0x4400)
    s = rng.integers(lo, hi, size=(V, K // G)).astype(np.uint16)
    z = rng.integers(0, QR[bits] + 1, size=(V, K // G)).astype(np.uint8)
    return n, s, z


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", [F16, BF16])
def test_logits_zp_with_fixed_zero_point_is_symmetric(orc, bits, sdt):
    V, K, G = 33, 256, 64
    rng = np.random.default_rng(5)
    q = rng.integers(-8 if bits == 4 else -128, 8 if bits == 4 else 128, size=(V, K)).astype(np.int8)
    _, s, _ = _table(V, K, G, bits, sdt, 6)
    zc = 8 if bits == 4 else 128
    n = (q.astype(np.int16) + zc).astype(np.uint8)
    z = np.full((V, K // G), zc, dtype=np.uint8)
    x = rng.standard_normal((3, K)).astype(np.float16)
    bias = rng.standard_normal(V).astype(np.float32)
    assert np.array_equal(orc.logits_zp(x, n, s, z, sdt, G, bias), orc.logits(x, q, s, sdt, G, bias))
    rows = [32, 0, 5, 5]
    assert np.array_equal(orc.logits_zp(x, n, s, z, sdt, G, rows=rows),
                          orc.logits(x, q, s, sdt, G, rows=rows))
    ids = [4, -1, 32, 7]
    for od in (F32, F16, BF16):
        assert np.array_equal(orc.embed_zp(n, s, z, sdt, G, ids, od),
                              orc.embed(q, s, sdt, G, ids, od))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", [F16, BF16])
def test_logits_zp_is_dense_logits_of_the_dequantized_table(orc, bits, sdt):
    V, K, G = 21, 128, 32
    n, s, z = _table(V, K, G, bits, sdt, 7)
    sv = orc.widen16(s, sdt).astype(np.float64)
    wdq = (n.astype(np.float64) - np.repeat(z, G, axis=1)) * np.repeat(sv, G, axis=1)
    w32 = wdq.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), wdq)   # exact in fp32
    x = np.random.default_rng(8).standard_normal((4, K)).astype(np.float16)
    assert np.array_equal(orc.logits_zp(x, n, s, z, sdt, G), orc.dense_logits(x, w32))


def test_logits_zp_exact_rationals(orc):
    V, K, G = 5, 64, 16
    n, s, z = _table(V, K, G, 4, F16, 9)
    x = np.random.default_rng(10).standard_normal((2, K)).astype(np.float16)
    y = orc.logits_zp(x, n, s, z, F16, G)
    sv = orc.widen16(s, F16)
    for m in range(2):
        for v in range(V):
            terms = [_f(x[m, k]) * (int(n[v, k]) - int(z[v, k // G])) * _f(sv[v, k // G])
                     for k in range(K)]
            exact = sum(terms)
            mag = sum(abs(t) for t in terms)
            assert abs(_f(y[m, v]) - exact) <= mag * K * Fraction(1, 2**52)


@pytest.mark.parametrize("sdt", [F16, BF16])
def test_embed_zp_equals_one_hot_logits_zp(orc, sdt):
    V, K, G = 37, 64, 32
    n, s, z = _table(V, K, G, 4, sdt, 11)
    table = orc.logits_zp(np.eye(K, dtype=np.float16), n, s, z, sdt, G).T
    got = orc.embed_zp(n, s, z, sdt, G, np.arange(V), F32)
    assert np.array_equal(got.astype(np.float64), table)
    out = orc.embed_zp(n, s, z, sdt, G, [-1, V, 3], F32)
    assert (out[:2] == 0).all() and np.array_equal(out[2], got[3])
    assert orc.embed_zp(n, s, z, sdt, G, [], F16).shape == (0, K)
    h = orc.embed_zp(n, s, z, sdt, G, np.arange(V), F16)
    with np.errstate(over="ignore"):
        assert np.array_equal(h, got.astype(np.float16).view(np.uint16))


def test_bad_arguments_rejected(orc):
    w = np.zeros((4, 64), dtype=np.float32)
    with pytest.raises(Exception):
        orc.quantize_asym(w, 5, 32, F16)
    with pytest.raises(Exception):
        orc.quantize_asym(w, 4, 48, F16)
    with pytest.raises(Exception):
        orc.pack_zp(np.zeros((4, 64), np.uint8), np.zeros((4, 2), np.uint16),
                    np.zeros((4, 2), np.uint8), 4, 48)
