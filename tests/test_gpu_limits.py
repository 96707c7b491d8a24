"""The largest sizes the library accepts, against the oracle: K = 65536 (the
longest row; every kernel that takes it, both code widths, one scale per row
as well as 128-column groups, fp16 and bf16 activations) and M = 65535 (the
most activation rows; the three MFMA kernels, which must give identical
bits, compared with each other on every row and with the oracle on rows
that cross the tile boundaries).  Also the quantizer and the packers at
K = 65536, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, OD, TD, abs_terms, bits16, check_logits, gpu, need_gpu, to_dev

pytestmark = gpu

KMAX, MMAX = 65536, 65535
GEMV, MFMA, LDS, XRES, SPLITK = (lmh.PATH_GEMV, lmh.PATH_MFMA, lmh.PATH_MFMA_LDS,
                                 lmh.PATH_MFMA_XRES, lmh.PATH_MFMA_SPLITK)


def _head(V, K, bits, G, seed):
    w = synth.random_weight((V, K), 0.02, seed)
    w[::7, ::97] *= 8.0  # outliers
    q, s = oracle.quantize(w, bits, G, OD["f16"], threads=8)
    return q, s, torch.from_numpy(oracle.pack(q, s, bits, G)).to(DEV)


def _logits(x, xdt, blob, V, K, bits, G, path):
    y = lmh.logits(to_dev(x, xdt), blob, V, K, bits, G, torch.float16, path=path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("bits,G", [(4, 128), (4, KMAX), (8, 64), (8, KMAX)])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_longest_rows(bits, G, xdt):
    """K = 65536 (512 int4 or 1024 int8 superchunks per row; the split-K
    kernel's waves run its two-buffer ring over 64 or 128 of them)."""
    need_gpu()
    V, K = 130, KMAX
    q, s, blob = _head(V, K, bits, G, seed=bits + G % 1000)
    for M, paths in ((1, (0, MFMA, LDS, SPLITK)), (7, (0, MFMA, LDS, SPLITK)), (40, (0, MFMA, LDS))):
        x = synth.random_x(M, K, seed=M, dtype=xdt)
        y_or = oracle.logits(x, q, s, OD["f16"], G, x_dtype=OD[xdt], threads=8)
        y_abs = abs_terms(x, xdt, q, s, OD["f16"], G)
        for path in paths:
            y = _logits(x, xdt, blob, V, K, bits, G, path)
            check_logits(y, y_or, y_abs, K, G, what=f"M={M} path={path}")
        for path in (XRES, GEMV):  # beyond these kernels' limits (K <= 1024; M * K <= 32768)
            with pytest.raises(lmh.LmheadError):
                _logits(x, xdt, blob, V, K, bits, G, path)


def test_gemv_at_its_largest_row_product():
    """The GEMV's limit M * K <= 32768: one row of 32768 columns and four of
    8192, with fp16 and bf16 activations."""
    need_gpu()
    bits, G, V = 4, 128, 200
    for M, K in ((1, 32768), (4, 8192)):
        q, s, blob = _head(V, K, bits, G, seed=K)
        for xdt in ("f16", "bf16"):
            x = synth.random_x(M, K, seed=M + K, dtype=xdt)
            y = _logits(x, xdt, blob, V, K, bits, G, GEMV)
            y_or = oracle.logits(x, q, s, OD["f16"], G, x_dtype=OD[xdt], threads=8)
            check_logits(y, y_or, abs_terms(x, xdt, q, s, OD["f16"], G), K, G,
                         what=f"M={M} K={K} {xdt}")


@pytest.mark.parametrize("bits,G", [(4, 64), (8, 128)])
def test_most_activation_rows(bits, G):
    """M = 65535 (1024 activation-resident tiles of 64 rows, the last one
    short by a row): the three MFMA kernels bit-identical on every row,
    and the oracle on rows around the first and last tiles' edges and a
    seeded sample between."""
    need_gpu()
    V, K = 130, 256
    q, s, blob = _head(V, K, bits, G, seed=bits * 7 + 1)
    x = synth.random_x(MMAX, K, seed=11)
    xd = to_dev(x, "f16")
    outs = {}
    for path in (0, MFMA, LDS, XRES):
        y = lmh.logits(xd, blob, V, K, bits, G, torch.float16, path=path)
        torch.cuda.synchronize()
        outs[path] = y.cpu().numpy()
    assert lmh.auto_path(MMAX, K, bits, G) == XRES
    for path in (MFMA, LDS, 0):
        assert np.array_equal(outs[path].view(np.uint32), outs[XRES].view(np.uint32)), path
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(0, 70), np.arange(MMAX - 70, MMAX),
                                     rng.integers(0, MMAX, 400)]))
    y_or = oracle.logits(x[rows], q, s, OD["f16"], G, x_dtype=OD["f16"], threads=8)
    y_abs = abs_terms(x[rows], "f16", q, s, OD["f16"], G)
    check_logits(outs[XRES][rows], y_or, y_abs, K, G, what=f"M={MMAX}")


@pytest.mark.parametrize("bits,G", [(4, 128), (4, KMAX), (8, KMAX)])
@pytest.mark.parametrize("clip", ["rtn", "mse"])
def test_quantize_and_pack_longest_rows(bits, G, clip):
    """Quantizer (bit-exact codes and scales), packer and fused quantize+pack
    (byte-exact blobs) at K = 65536; one group per row streams the row once
    per pass."""
    need_gpu()
    V, K = 70, KMAX
    w = synth.random_weight((V, K), 0.02, bits + G % 1000)
    w[3, 100:200] *= 20.0  # outliers: the clip search moves
    ratios = oracle.MSE_RATIOS if clip == "mse" else oracle.RTN_RATIOS
    qo, so = oracle.quantize(w, bits, G, OD["bf16"], ratios, threads=8)
    wd = to_dev(w, "f32")
    q, s = lmh.quantize(wd, bits, G, TD["bf16"], clip)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(s), so)
    assert np.array_equal(q.cpu().numpy(), qo)
    blob_or = oracle.pack(qo, so, bits, G)
    packed = lmh.pack(q, s, bits, G)
    fused = lmh.quantize_pack(wd, bits, G, TD["bf16"], clip)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), blob_or)
    assert np.array_equal(fused.cpu().numpy(), blob_or)
