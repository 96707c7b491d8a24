"""Pins for the oracle's logits (exact products, fp64 sums) and dense logits.

  * brute force in exact rationals on tiny inputs (every product and sum exact);
  * numpy float64 dequantize-then-matmul (the "dequant + F.linear" path of vLLM
    PR #48870, Purpose) on a slice of the tiny head;
  * invariants: all-zero rows give exactly 0, y(2x) = 2 y(x), bias adds per row,
    a row subset equals the matching columns of the full result.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import BF16, F16, F32, MSE_RATIOS


def _frac16(bits, dtype, orc):
    return [Fraction(float(v)) for v in orc.widen16(np.asarray(bits, np.uint16), dtype).ravel()]


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("xdt,sdt", [(F16, F16), (BF16, BF16), (F16, BF16)])
def test_logits_exact_rationals(orc, G, xdt, sdt):
    rng = np.random.default_rng(G + 10 * xdt + sdt)
    M, V, K = 2, 5, 64
    q = rng.integers(-8, 8, size=(V, K)).astype(np.int8)
    sf = (rng.random((V, K // G)) * 0.01 + 1e-4).astype(np.float32)
    s = orc.encode16(sf, sdt)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    x = orc.encode16(xf, xdt)
    bias = rng.standard_normal(V).astype(np.float32)
    y = orc.logits(x, q, s, sdt, G, bias=bias, x_dtype=xdt)
    xs = _frac16(x, xdt, orc)
    ss = _frac16(s, sdt, orc)
    for m in range(M):
        for v in range(V):
            terms = [xs[m * K + k] * int(q[v, k]) * ss[v * (K // G) + k // G] for k in range(K)]
            exact = sum(terms) + Fraction(float(bias[v]))
            mag = sum(abs(t) for t in terms) + abs(Fraction(float(bias[v])))
            assert abs(Fraction(y[m, v]) - exact) <= mag * Fraction(1, 10**15)


@pytest.fixture(scope="module")
def tiny_slice(orc):
    w = synth.WORKLOADS["tiny_w4g64_50304x512"]
    r0 = w.V - 2048  # the last 2048 rows include the 64 all-zero padding rows
    W = synth.weight(w, r0, w.V)
    q, s = orc.quantize(W, w.bits, w.group, F16)
    x = synth.activations(w, 3)
    return w, q, s, x


def test_logits_vs_numpy_dequant_matmul(orc, tiny_slice):
    w, q, s, x = tiny_slice
    y = orc.logits(x, q, s, F16, w.group)
    sv = np.repeat(orc.widen16(s, F16).astype(np.float64), w.group, axis=1)
    wd = q.astype(np.float64) * sv
    x64 = x.astype(np.float64)
    ref = x64 @ wd.T
    mag = np.abs(x64) @ np.abs(wd).T
    assert (np.abs(y - ref) <= 1e-12 * mag + 1e-300).all()


def test_logits_invariants(orc, tiny_slice):
    w, q, s, x = tiny_slice
    y = orc.logits(x, q, s, F16, w.group)
    assert (y[:, -64:] == 0.0).all()  # all-zero rows -> exactly zero logits
    assert np.abs(y[:, :-64]).min() > 0
    x2 = (x.astype(np.float32) * 2).astype(np.float16)
    assert np.array_equal(orc.logits(x2, q, s, F16, w.group), 2 * y)
    rows = [5, 0, 2047, 1000, 5]
    assert np.array_equal(orc.logits(x, q, s, F16, w.group, rows=rows), y[:, rows])
    b = np.linspace(-1, 1, q.shape[0]).astype(np.float32)
    yb = orc.logits(x, q, s, F16, w.group, bias=b)
    assert np.allclose(yb - y, b.astype(np.float64)[None, :], rtol=0, atol=1e-12)


def test_dense_logits_exact_rationals_and_numpy(orc):
    rng = np.random.default_rng(3)
    M, V, K = 2, 4, 48
    x = rng.standard_normal((M, K)).astype(np.float16)
    wf = (rng.standard_normal((V, K)) * 0.02).astype(np.float32)
    for wdt, warr in [(F16, wf.astype(np.float16)), (BF16, orc.encode16(wf, BF16)), (F32, wf)]:
        y = orc.dense_logits(x, warr, w_dtype=wdt)
        wv = warr.astype(np.float64) if wdt != BF16 else orc.widen16(warr, BF16).astype(np.float64)
        for m in range(M):
            for v in range(V):
                terms = [Fraction(float(x[m, k])) * Fraction(float(wv[v, k])) for k in range(K)]
                mag = sum(abs(t) for t in terms)
                assert abs(Fraction(y[m, v]) - sum(terms)) <= mag * Fraction(1, 10**15)
        ref = x.astype(np.float64) @ wv.T
        assert np.allclose(y, ref, rtol=1e-13, atol=0)


def test_quantized_logits_track_dense_logits(orc):
    """Quantisation error stays small relative to the logits: the int8 per-row head
    of the review comment on vLLM PR #48870 (fp16 weight, M = 1) on a 512-row slice."""
    w = synth.WORKLOADS["w8row_151936x2048"]
    W = synth.weight(w, 0, 512)
    q, s = orc.quantize(W, 8, w.group, F16)
    x = synth.activations(w, 1)
    yq = orc.logits(x, q, s, F16, w.group)
    yd = orc.dense_logits(x, W)
    rel = np.abs(yq - yd).max() / np.abs(yd).max()
    assert 1e-5 < rel < 2e-2
    # int4 with the MSE search on the bf16 head distribution
    w5 = synth.WORKLOADS["w4g128mse_248064x5120"]
    W5 = synth.weight(w5, 0, 256)
    q5, s5 = orc.quantize(W5, 4, 128, BF16, MSE_RATIOS, w_dtype=BF16)
    x5 = synth.activations(w5, 1)
    y5q = orc.logits(x5, q5, s5, BF16, 128, x_dtype=BF16)
    y5d = orc.dense_logits(x5, W5, x_dtype=BF16, w_dtype=BF16)
    rel5 = np.abs(y5q - y5d).max() / np.abs(y5d).max()
    assert 1e-3 < rel5 < 0.3
