"""The oracle's row-parallel calls give the single-thread results bit for bit
(every row's arithmetic is independent of how the rows are split)."""
import numpy as np
import pytest

import synth
from oracle import BF16, F16, MSE_RATIOS


@pytest.mark.parametrize("threads", [2, 3, 7])
def test_threaded_quantize_and_logits_equal_single_thread(orc, threads):
    w = synth.random_weight((1000, 256), 0.02, 5, (998, 999))
    for bits, G, sdt, ratios in ((4, 64, F16, (1.0,)), (8, 128, BF16, MSE_RATIOS)):
        q1, s1, p1 = orc.quantize(w, bits, G, sdt, ratios, return_pick=True, threads=1)
        qt, st, pt = orc.quantize(w, bits, G, sdt, ratios, return_pick=True, threads=threads)
        assert np.array_equal(q1, qt) and np.array_equal(s1, st) and np.array_equal(p1, pt)
        x = (np.random.default_rng(1).standard_normal((3, 256))).astype(np.float16)
        y1 = orc.logits(x, q1, s1, sdt, G, threads=1)
        yt = orc.logits(x, q1, s1, sdt, G, threads=threads)
        assert np.array_equal(y1, yt)
        rows = np.array([999, 3, 500, 0, 64, 63], dtype=np.int64)
        assert np.array_equal(orc.logits(x, q1, s1, sdt, G, rows=rows, threads=threads),
                              y1[:, rows])
