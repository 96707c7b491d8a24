"""Pins for the oracle's top-K selection and exact rescoring (vLLM PR #48870, review
comment point 2; reading R5 of oracle/lmh_oracle.c: value descending then index ascending; the top-1 is
the first maximum of the scattered vector)."""
import numpy as np
import pytest

from oracle import BF16, F16, F32


def _ref_topk(y, k):
    return sorted(range(len(y)), key=lambda i: (-float(y[i]), i))[:k]


@pytest.mark.parametrize("k", [1, 4, 8, 16])
def test_topk_vs_sorted_with_ties(orc, k):
    rng = np.random.default_rng(k)
    for trial in range(5):
        y = rng.integers(-5, 6, size=300).astype(np.float32) * np.float32(0.25)  # many ties
        assert list(orc.topk(y, k)) == _ref_topk(y, k)
    y = rng.standard_normal(1000).astype(np.float32)
    assert list(orc.topk(y, k)) == _ref_topk(y, k)


def test_topk_edge_cases(orc):
    y = np.array([3.0, -1.0, 3.0, 2.0], dtype=np.float32)
    assert list(orc.topk(y, 4)) == [0, 2, 3, 1]
    assert list(orc.topk(y, 1)) == [0]
    with pytest.raises(ValueError):
        orc.topk(y, 5)
    with pytest.raises(ValueError):
        orc.topk(y, 0)


@pytest.mark.parametrize("wdt", [F16, BF16, F32])
def test_rescore_values_and_top1(orc, wdt):
    rng = np.random.default_rng(7 + wdt)
    M, V, K, k = 3, 400, 96, 8
    x = rng.standard_normal((M, K)).astype(np.float16)
    wf = (rng.standard_normal((V, K)) * 0.05).astype(np.float32)
    if wdt == F16:
        w, wv = wf.astype(np.float16), wf.astype(np.float16).astype(np.float64)
    elif wdt == BF16:
        w = orc.encode16(wf, BF16)
        wv = orc.widen16(w, BF16).astype(np.float64)
    else:
        w, wv = wf, wf.astype(np.float64)
    exact = x.astype(np.float64) @ wv.T
    # "quantized" logits: the exact ones plus a perturbation that reorders the top
    y = (exact + rng.standard_normal(exact.shape) * 0.05).astype(np.float32)
    y[1, 17] = y[1].max() + 1.0  # a spurious winner that rescoring must demote
    idx, val, top1 = orc.topk_rescore(y, k, x, w, w_dtype=wdt)
    for m in range(M):
        assert list(idx[m]) == _ref_topk(y[m], k)
        assert np.allclose(val[m], exact[m, idx[m]], rtol=1e-13, atol=1e-15)
        scat = y[m].astype(np.float64).copy()
        scat[idx[m]] = val[m]
        assert top1[m] == int(np.argmax(scat))
    assert top1[1] != 17 or exact[1, 17] >= exact[1].max()
