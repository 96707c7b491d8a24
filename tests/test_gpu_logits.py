"""GPU logits (GEMV and the four MFMA kernels) against the fp64 oracle on small heads
that still span several row blocks, several superchunks per wave and a ragged tail."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, OD, TD, abs_terms, bits16, check_logits, gpu, need_gpu, to_dev

pytestmark = gpu

GEMV, MFMA, LDS, XRES = lmh.PATH_GEMV, lmh.PATH_MFMA, lmh.PATH_MFMA_LDS, lmh.PATH_MFMA_XRES
SPLITK = lmh.PATH_MFMA_SPLITK


def _head(V, K, bits, G, sdt, seed, zero_rows=()):
    w = synth.random_weight((V, K), 0.02, seed, zero_rows)
    w[::17, ::13] *= 8.0  # outliers
    q, s = oracle.quantize(w, bits, G, OD[sdt])
    blob = oracle.pack(q, s, bits, G)
    return q, s, torch.from_numpy(blob).to(DEV)


def _run(xnp, xdt, blob, V, K, bits, G, sdt, path, bias=None, ldy=None):
    x = to_dev(xnp, xdt)
    M = xnp.shape[0]
    ldy = ldy or V
    out = torch.full((M, ldy), float("nan"), dtype=torch.float32, device=DEV)
    b = None if bias is None else torch.from_numpy(bias).to(DEV)
    lmh.logits(x, blob, V, K, bits, G, TD[sdt], bias=b, out=out, path=path)
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    if ldy > V:
        assert np.isnan(y[:, V:]).all(), "columns past V were written"
    return y[:, :V]


CASES = [  # bits, G, K
    (4, 32, 512), (4, 64, 1024), (4, 128, 512), (4, 256, 1024), (4, 1024, 1024),
    (8, 32, 256), (8, 64, 512), (8, 128, 1024), (8, 512, 512),
]


@pytest.mark.parametrize("bits,G,K", CASES)
@pytest.mark.parametrize("xdt,sdt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "bf16")])
@pytest.mark.parametrize("path,Ms", [(GEMV, (1, 2, 3, 4)), (MFMA, (1, 5, 16, 17, 40, 67)),
                                     (LDS, (1, 5, 64, 65, 130)), (XRES, (1, 7, 64, 65, 130)),
                                     (SPLITK, (1, 3, 9, 16))])
def test_logits_small_vs_oracle(bits, G, K, xdt, sdt, path, Ms):
    need_gpu()
    V = 64 * 5 + 37
    q, s, blob = _head(V, K, bits, G, sdt, seed=K + G + bits, zero_rows=(3, V - 1))
    worst = 0.0
    for M in Ms:
        x = synth.random_x(M, K, seed=M, dtype=xdt)
        y = _run(x, xdt, blob, V, K, bits, G, sdt, path)
        y_or = oracle.logits(x, q, s, OD[sdt], G, x_dtype=OD[xdt])
        y_abs = abs_terms(x, xdt, q, s, OD[sdt], G)
        worst = max(worst, check_logits(y, y_or, y_abs, K, G, what=f"M={M} path={path}"))
    print(f"bits={bits} G={G} K={K} x={xdt} s={sdt} path={path}: max row rel err {worst:.2e}")


@pytest.mark.parametrize("path,M", [(GEMV, 1), (GEMV, 3), (MFMA, 8), (MFMA, 33), (LDS, 20), (LDS, 70),
                                    (XRES, 3), (XRES, 29), (XRES, 70), (SPLITK, 5), (SPLITK, 13)])
def test_bias_and_row_stride(path, M):
    need_gpu()
    V, K, bits, G = 200, 512, 4, 64
    q, s, blob = _head(V, K, bits, G, "f16", seed=5)
    bias = synth.random_weight((1, V), 1.0, 6)[0]
    x = synth.random_x(M, K, seed=9)
    y = _run(x, "f16", blob, V, K, bits, G, "f16", path, bias=bias, ldy=V + 45)
    y_or = oracle.logits(x, q, s, oracle.F16, G, bias=bias)
    y_abs = abs_terms(x, "f16", q, s, oracle.F16, G)
    check_logits(y, y_or, y_abs, K, G, what="bias", bias=bias)


@pytest.mark.parametrize("bits,G", [(4, 64), (4, 128), (8, 128), (8, 32)])
@pytest.mark.parametrize("path", [GEMV, MFMA, LDS, XRES, SPLITK])
def test_one_hot_exposes_layout(bits, G, path):
    """x = e_k gives y[v] = q[v,k] * s[v, k/G] exactly (one exact product): any
    misplaced nibble, byte, slot or scale shows up bit for bit."""
    need_gpu()
    V, K = 130, 256
    q, s, blob = _head(V, K, bits, G, "f16", seed=11)
    sv = oracle.widen16(s, oracle.F16).astype(np.float64)
    ks = [0, 1, 7, 8, 31, 32, 63, 64, 100, 127, 128, 200, 255]
    for i in range(0, len(ks), 4):
        kk = ks[i:i + 4]
        x = np.zeros((len(kk), K), dtype=np.float16)
        for m, k in enumerate(kk):
            x[m, k] = 1.0
        y = _run(x, "f16", blob, V, K, bits, G, "f16", path)
        for m, k in enumerate(kk):
            want = q[:, k].astype(np.float64) * sv[:, k // G]
            assert np.array_equal(y[m].astype(np.float64), want), f"column {k}"


@pytest.mark.parametrize("path,M", [(GEMV, 1), (GEMV, 4), (MFMA, 16), (MFMA, 64), (LDS, 64), (LDS, 128),
                                    (XRES, 64), (XRES, 200), (SPLITK, 11), (SPLITK, 16)])
def test_invariants_zero_rows_scaling_determinism(path, M):
    need_gpu()
    V, K, bits, G = 320, 512, 4, 64
    zero = (0, 64, 200, 319)
    q, s, blob = _head(V, K, bits, G, "f16", seed=13, zero_rows=zero)
    x = synth.random_x(M, K, seed=21)
    y1 = _run(x, "f16", blob, V, K, bits, G, "f16", path)
    y2 = _run(x, "f16", blob, V, K, bits, G, "f16", path)
    assert np.array_equal(y1, y2), "two identical calls differ"
    assert (y1[:, list(zero)] == 0).all()
    x2 = (x.astype(np.float32) * 2).astype(np.float16)
    y3 = _run(x2, "f16", blob, V, K, bits, G, "f16", path)
    assert np.array_equal(y3, 2 * y1), "y(2x) != 2 y(x)"


@pytest.mark.parametrize("bits,G,K", [(4, 128, 2048), (4, 128, 3072), (4, 128, 5120), (4, 64, 4096),
                                      (4, 1024, 3072), (8, 128, 2048), (8, 64, 3072), (8, 2048, 2048)])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_gemv_wide_rows(bits, G, K, xdt):
    """The GEMV on rows of 2048..5120 columns: waves with 2..5 superchunks of
    the K split (the two-buffer ring with an even and an odd count, the serial
    mode of the 3- and 4-row variants), groups inside and across waves."""
    need_gpu()
    V = 330
    sdt = "bf16" if xdt == "bf16" else "f16"
    q, s, blob = _head(V, K, bits, G, sdt, seed=K + G + bits)
    for M in (1, 2, 3, 4):
        x = synth.random_x(M, K, seed=M + 7, dtype=xdt)
        y = _run(x, xdt, blob, V, K, bits, G, sdt, GEMV)
        y_or = oracle.logits(x, q, s, OD[sdt], G, x_dtype=OD[xdt])
        y_abs = abs_terms(x, xdt, q, s, OD[sdt], G)
        check_logits(y, y_or, y_abs, K, G, what=f"K={K} G={G} bits={bits} M={M} {xdt}")


def test_gemv_and_mfma_agree():
    need_gpu()
    V, K, bits, G = 600, 1024, 4, 64
    q, s, blob = _head(V, K, bits, G, "f16", seed=17)
    for M in (1, 2, 3, 4):
        x = synth.random_x(M, K, seed=30 + M)
        a = _run(x, "f16", blob, V, K, bits, G, "f16", GEMV)
        b = _run(x, "f16", blob, V, K, bits, G, "f16", MFMA)
        scale = np.abs(a).max()
        assert np.abs(a - b).max() <= 1e-5 * scale


@pytest.mark.parametrize("bits,G", [(4, 32), (4, 64), (4, 256), (8, 64), (8, 128)])
def test_mfma_kernels_bit_identical(bits, G):
    """The register-fed, LDS-staged and activation-resident MFMA kernels run
    the same per-group MFMA chains and the same fp32 scale FMAs in the same
    order: bit-identical, across activation-tile boundaries and a ragged
    vocabulary tail."""
    need_gpu()
    V, K = 64 * 9 + 21, 512
    q, s, blob = _head(V, K, bits, G, "f16", seed=41 + G)
    for M in (17, 32, 64, 100, 129):
        x = synth.random_x(M, K, seed=50 + M)
        a = _run(x, "f16", blob, V, K, bits, G, "f16", MFMA)
        b = _run(x, "f16", blob, V, K, bits, G, "f16", LDS)
        assert np.array_equal(a, b), f"M={M}"
        c = _run(x, "f16", blob, V, K, bits, G, "f16", XRES)
        assert np.array_equal(a, c), f"M={M} (activation-resident)"


@pytest.mark.parametrize("bits,G,K", [(4, 32, 512), (4, 64, 1024), (4, 256, 1024), (4, 128, 3072),
                                      (4, 64, 768), (4, 128, 384), (8, 64, 320), (8, 64, 512),
                                      (8, 128, 2048), (8, 1024, 1024)])
def test_splitk_agrees_with_mfma_kernels(bits, G, K):
    """The split-K kernel adds the same exact per-group products and fp32
    scale FMAs as the other MFMA kernels, only its K partial sums associate
    differently: per element within the fp32 summation bound of the oracle
    and within a few fp32 ulps of max|y| of the register-fed kernel; splits
    of 1, 2, 4 and 8 waves (superchunk counts 4..48), one- and two-buffer
    loads, one to sixteen rows, a ragged vocabulary tail."""
    need_gpu()
    V = 64 * 7 + 29
    q, s, blob = _head(V, K, bits, G, "f16", seed=61 + G + K)
    for M in (1, 3, 9, 16):
        x = synth.random_x(M, K, seed=70 + M)
        a = _run(x, "f16", blob, V, K, bits, G, "f16", MFMA)
        b = _run(x, "f16", blob, V, K, bits, G, "f16", SPLITK)
        y_or = oracle.logits(x, q, s, oracle.F16, G, x_dtype=oracle.F16)
        y_abs = abs_terms(x, "f16", q, s, oracle.F16, G)
        check_logits(b, y_or, y_abs, K, G, what=f"split-K M={M}")
        assert np.abs(a - b).max() <= 1e-5 * np.abs(a).max(), f"M={M}"


@pytest.mark.parametrize("V,K,bits,G", [(1, 128, 4, 64), (63, 128, 4, 32), (65, 256, 4, 128),
                                        (130, 384, 4, 128), (200, 64, 8, 32), (64, 128, 8, 128)])
def test_splitk_small_heads_and_dead_waves(V, K, bits, G):
    """Split-K on heads of one to a few row blocks: K splits of 1, 2 and 4
    waves (several blocks per workgroup, most waves finding no block), a
    ragged last block, bias and a padded row stride, fp32 and fp16 output."""
    need_gpu()
    q, s, blob = _head(V, K, bits, G, "f16", seed=V + K)
    bias = synth.random_weight((1, V), 1.0, 3)[0]
    for M in (1, 2, 7, 16):
        x = synth.random_x(M, K, seed=M + V)
        y = _run(x, "f16", blob, V, K, bits, G, "f16", SPLITK, bias=bias, ldy=V + 5)
        y_or = oracle.logits(x, q, s, oracle.F16, G, x_dtype=oracle.F16, bias=bias)
        check_logits(y, y_or, abs_terms(x, "f16", q, s, oracle.F16, G), K, G, what=f"M={M}",
                     bias=bias)
        y16 = lmh.logits(to_dev(x, "f16"), blob, V, K, bits, G, torch.float16, path=SPLITK,
                         bias=torch.from_numpy(bias).to(DEV), out_dtype=torch.float16)
        torch.cuda.synchronize()
        assert torch.equal(y16.cpu(), torch.from_numpy(np.ascontiguousarray(y)).half()), f"fp16 M={M}"


def test_bf16_activations_large_and_small_rows():
    """bf16 rows far outside the fp16 range (and tiny ones) are handled by the
    power-of-two row scale."""
    need_gpu()
    V, K, bits, G = 256, 512, 4, 128
    q, s, blob = _head(V, K, bits, G, "bf16", seed=19)
    xf = synth.random_weight((3, K), 1.0, 23)
    xf[0] *= 1e6
    xf[1] *= 1e-6
    xf[2, 5] = 3e4
    x = synth.to_bf16_bits(xf)
    for path in (GEMV, MFMA, LDS, XRES, SPLITK):
        y = _run(x, "bf16", blob, V, K, bits, G, "bf16", path)
        y_or = oracle.logits(x, q, s, oracle.BF16, G, x_dtype=oracle.BF16)
        y_abs = abs_terms(x, "bf16", q, s, oracle.BF16, G)
        check_logits(y, y_or, y_abs, K, G, what=f"bf16 extremes path={path}")


def test_empty_calls_launch_nothing():
    need_gpu()
    x = torch.zeros((0, 128), dtype=torch.float16, device=DEV)
    blob = torch.zeros(lmh.packed_bytes(64, 128, 4, 64), dtype=torch.uint8, device=DEV)
    y = lmh.logits(x, blob, 64, 128, 4, 64, torch.float16)
    assert y.shape == (0, 64)


def _ulp16(y: np.ndarray, odt: str) -> np.ndarray:
    """Spacing of the 16-bit format at |y| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(y), 1e-30)))
    return np.exp2(e - (10 if odt == "f16" else 7))


@pytest.mark.parametrize("odt", ["f16", "bf16"])
@pytest.mark.parametrize("path,M", [(GEMV, 1), (GEMV, 3), (MFMA, 5), (MFMA, 17), (LDS, 20), (LDS, 70),
                                    (XRES, 20), (XRES, 40), (XRES, 130), (SPLITK, 9), (SPLITK, 16)])
@pytest.mark.parametrize("bits,G", [(4, 64), (8, 128)])
def test_16bit_logits_output(odt, path, M, bits, G):
    """16-bit logits are the fp32 result rounded once to nearest even (bit-exact
    against converting the same kernel's fp32 output), so they stay within the
    fp32 bound plus half a 16-bit ulp of the oracle; bias and strided rows too."""
    need_gpu()
    V, K = 64 * 5 + 13, 512
    q, s, blob = _head(V, K, bits, G, "f16", seed=bits + G + M)
    x = synth.random_x(M, K, seed=60 + M)
    bias = synth.random_weight((1, V), 0.5, 7)[0]
    y32 = _run(x, "f16", blob, V, K, bits, G, "f16", path, bias=bias)
    ldy = V + 24
    out = torch.full((M, ldy), 7.0, dtype=TD[odt], device=DEV)
    lmh.logits(to_dev(x, "f16"), blob, V, K, bits, G, torch.float16,
               bias=torch.from_numpy(bias).to(DEV), out=out[:, :V], path=path)
    torch.cuda.synchronize()
    assert (out[:, V:] == 7.0).all(), "columns past V were written"
    got = out[:, :V].float().cpu().numpy()
    want = torch.from_numpy(y32).to(TD[odt]).float().numpy()
    assert np.array_equal(got, want), f"not the rounded fp32 result at {np.argwhere(got != want)[:4]}"
    y_or = oracle.logits(x, q, s, oracle.F16, G, bias=bias, x_dtype=oracle.F16)
    y_abs = abs_terms(x, "f16", q, s, oracle.F16, G)
    slack = (K + K // G + 16) * 2.0**-24 * y_abs + np.abs(bias)[None, :] * 2.0**-23
    assert (np.abs(got - y_or) <= slack + 0.5 * _ulp16(y_or, odt) * (1 + 2.0**-10) + 1e-30).all()


def test_16bit_output_overflow_to_inf():
    """fp16 logits beyond 65504 round to +-inf, as the conversion of the fp32 value does."""
    need_gpu()
    V, K, bits, G = 200, 256, 4, 64
    q, s, blob = _head(V, K, bits, G, "f16", seed=3)
    x = synth.random_x(2, K, seed=5)
    bias = np.zeros(V, dtype=np.float32)
    bias[::3] = 7.0e4                      # past the fp16 range
    bias[1::7] = -6.6e4
    y32 = _run(x, "f16", blob, V, K, bits, G, "f16", GEMV, bias=bias)
    y16 = lmh.logits(to_dev(x, "f16"), blob, V, K, bits, G, torch.float16, path=GEMV,
                     bias=torch.from_numpy(bias).to(DEV), out_dtype=torch.float16)
    torch.cuda.synchronize()
    want = torch.from_numpy(y32).half()
    assert torch.isinf(want).any(), "test input did not reach the fp16 range limit"
    assert torch.equal(y16.cpu(), want)
