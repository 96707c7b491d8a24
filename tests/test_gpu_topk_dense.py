"""GPU top-K exact rescoring and the dense 16-bit control GEMV against the oracle.

Top-K: the selected indices and their order must equal the oracle's selection on
the GPU's own logits (bit-exact, reading R5 of oracle/lmh_oracle.c); rescored values must lie within the
fp32 summation bound gamma_K * sum_k |x w| of the fp64 dot product; the top-1 must
equal the oracle's argmax of the scattered row wherever that is unambiguous."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, OD, TD, gpu, need_gpu, to_dev

pytestmark = gpu


def _gamma(n):
    u = 2.0**-24
    return n * u / (1 - n * u)


@pytest.mark.parametrize("wdt,xdt", [("f16", "f16"), ("bf16", "bf16"), ("f32", "f16")])
# V spans one to a few hundred 2048-entry blocks (fewer lists than T and more),
# topk = 64 takes the first pass's block-wide threshold, K = 100 the
# unvectorised rescoring
@pytest.mark.parametrize("V,K,topk,M", [(5000, 256, 8, 1), (9000, 512, 16, 3), (300, 96, 1, 2),
                                         (4097, 128, 64, 2), (70, 64, 64, 1), (3001, 100, 8, 2),
                                         (100000, 64, 16, 1), (200000, 32, 32, 2),
                                         (400000, 32, 8, 1), (600000, 32, 8, 1)])
def test_topk_rescore_vs_oracle(wdt, xdt, V, K, topk, M):
    need_gpu()
    wf = synth.random_weight((V, K), 0.05, V + K)
    w = wf.astype(np.float16) if wdt == "f16" else (synth.to_bf16_bits(wf) if wdt == "bf16" else wf)
    x = synth.random_x(M, K, seed=topk, dtype=xdt)
    # quantized-like logits: exact logits plus noise, with planted exact ties
    exact = oracle.dense_logits(x, w, x_dtype=OD[xdt], w_dtype=OD[wdt])
    rng = np.random.default_rng(V)
    y0 = (exact + rng.standard_normal(exact.shape) * 0.02).astype(np.float32)
    y0[:, 10] = y0[:, 11] = y0.max(axis=1)  # a tie at the top: lower index first
    y = torch.from_numpy(y0).to(DEV)
    idx, val, top1 = lmh.topk_rescore(to_dev(x, xdt), to_dev(w, wdt), y, topk)
    torch.cuda.synchronize()
    oi, ov, ot = oracle.topk_rescore(y0, topk, x, w, x_dtype=OD[xdt], w_dtype=OD[wdt])
    gi = idx.cpu().numpy().astype(np.int64)
    gv = val.cpu().numpy().astype(np.float64)
    assert np.array_equal(gi, oi), "selection or order differs"
    xa = np.abs(oracle.widen16(x, OD[xdt]) if xdt == "bf16" else x.astype(np.float64))
    wa = np.abs(oracle.widen16(w, OD[wdt]) if wdt == "bf16" else w.astype(np.float64))
    for m in range(M):
        bound = _gamma(K) * (xa[m][None, :] * wa[oi[m]]).sum(axis=1)
        assert (np.abs(gv[m] - ov[m]) <= bound + 1e-30).all()
    # the scattered row
    yn = y.cpu().numpy()
    for m in range(M):
        assert np.array_equal(yn[m, gi[m]], gv[m].astype(np.float32))
        keep = np.ones(V, bool)
        keep[gi[m]] = False
        assert np.array_equal(yn[m, keep], y0[m, keep])
        # top-1: the first maximum of the GPU's own scattered row, and the oracle's
        # top-1 unless the exact and rounded winners are within rounding of each other
        assert top1[m].item() == int(np.argmax(yn[m]))
        srt = np.sort(np.concatenate([ov[m], y0[m, keep].astype(np.float64)]))
        if srt[-1] - srt[-2] > 1e-5:
            assert top1[m].item() == ot[m]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("V,K,M", [(1000, 2048, 1), (517, 1024, 2), (64, 520, 4), (3, 8, 1)])
def test_dense_control_vs_oracle(dt, V, K, M):
    need_gpu()
    wf = synth.random_weight((V, K), 0.02, V * 3 + K)
    w = wf.astype(np.float16) if dt == "f16" else synth.to_bf16_bits(wf)
    x = synth.random_x(M, K, seed=V, dtype=dt)
    y = lmh.dense_logits(to_dev(x, dt), to_dev(w, dt))
    torch.cuda.synchronize()
    y_or = oracle.dense_logits(x, w, x_dtype=OD[dt], w_dtype=OD[dt])
    xa = np.abs(oracle.widen16(x, OD[dt]) if dt == "bf16" else x.astype(np.float64))
    wa = np.abs(oracle.widen16(w, OD[dt]) if dt == "bf16" else w.astype(np.float64))
    bound = _gamma(K + 64) * (xa @ wa.T)
    assert (np.abs(y.cpu().numpy() - y_or) <= bound + 1e-30).all()
