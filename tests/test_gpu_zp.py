"""Zero-point (asymmetric) heads on the GPU against the oracle: quantizer bit-exact
(n, s, z), packer and fused quantize + pack byte-exact, embedding rows bit-exact,
and logits within the acceptance bars of the symmetric path on every kernel.

The acceptance bound per element uses sum_k |x (n - z) s|, the same fp32
summation bound as for symmetric heads (products x * (n - z) are exact)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, OD, TD, bits16, check_logits, gpu, need_gpu, to_dev

pytestmark = gpu

ZP = lmh.ZP
QR = {4: 15, 8: 255}
GEMV, MFMA, LDS, XRES = lmh.PATH_GEMV, lmh.PATH_MFMA, lmh.PATH_MFMA_LDS, lmh.PATH_MFMA_XRES
SPLITK = lmh.PATH_MFMA_SPLITK


def _weights(V, K, wdt, seed, zero_rows=()):
    """Lopsided Gaussian groups (per-row offsets), outliers, an all-zero group,
    tiny groups (the scale floor) and one-sided rows."""
    w = synth.random_weight((V, K), 0.02, seed, zero_rows)
    off = np.random.default_rng(seed + 1).uniform(-0.03, 0.03, size=(V, 1)).astype(np.float32)
    w = (w + off).astype(np.float32)
    for r in zero_rows:
        w[r] = 0.0
    w[V // 3, : K // 2] *= 9.0
    w[V // 2, 32:64] = 0.0
    w[min(5, V - 1), :32] *= 1e-7
    if V > 9:
        w[8] = np.abs(w[8])
        w[9] = -np.abs(w[9])
    if wdt == "f16":
        return w.astype(np.float16)
    if wdt == "bf16":
        return synth.to_bf16_bits(w)
    return w


def _dq(n, s, z, sdt, G):
    """Dequantized table (n - z) * s, exact in fp32."""
    sv = oracle.widen16(s, OD[sdt]).astype(np.float64)
    w = (n.astype(np.float64) - np.repeat(z, G, axis=1)) * np.repeat(sv, G, axis=1)
    return w.astype(np.float32)


def _abs_terms(x, xdt, wdq):
    """sum_k |x (n - z) s| per (m, row): the dense oracle on |x| and |W|."""
    xa = x & np.uint16(0x7FFF) if xdt == "bf16" else np.abs(x)
    return oracle.dense_logits(xa, np.abs(wdq), x_dtype=OD[xdt], w_dtype=oracle.F32)


def _s_dev(s, sdt):
    return torch.from_numpy(s.view(np.int16)).view(TD[sdt]).to(DEV)


# ---- quantizer and packer ----------------------------------------------------------

@pytest.mark.parametrize("wdt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits,G", [(4, 32), (4, 64), (4, 128), (4, 256), (8, 32), (8, 128),
                                    (8, 512)])
@pytest.mark.parametrize("sdt", ["f16", "bf16"])
def test_quantize_zp_bit_exact(wdt, bits, G, sdt):
    need_gpu()
    V, K = 131, 512
    w = _weights(V, K, wdt, seed=bits * 100 + G, zero_rows=(0, V - 1))
    n, s, z = lmh.quantize_zp(to_dev(w, wdt), bits, G, TD[sdt])
    torch.cuda.synchronize()
    no, so, zo = oracle.quantize_asym(w, bits, G, OD[sdt], w_dtype=OD[wdt])
    assert np.array_equal(bits16(s), so), f"scales differ at {np.argwhere(bits16(s) != so)[:5]}"
    assert np.array_equal(z.cpu().numpy(), zo), "zero points differ"
    ng = n.cpu().numpy()
    assert np.array_equal(ng, no), f"codes differ at {np.argwhere(ng != no)[:5]}"


def test_quantize_zp_hand_cases():
    """The oracle pins' known answers: ties to even, and the int8 / bf16 group
    whose rounded-down scale pushes z and one code to their clamps."""
    need_gpu()
    s0 = 2.0**-6
    w = np.zeros((2, 32), dtype=np.float32)
    w[0, :5] = np.array([-4, 11, -3.5, 2.5, 0.5], np.float32) * np.float32(s0)
    n, s, z = lmh.quantize_zp(to_dev(w, "f32"), 4, 32, torch.float16)
    assert list(n[0, :5].cpu().numpy()) == [0, 15, 0, 6, 4] and int(z[0, 0]) == 4
    assert (n[1] == 0).all() and int(z[1, 0]) == 0 and int(bits16(s)[1, 0]) == 0
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0], w[0, 1] = -255.97, -100.0
    n, s, z = lmh.quantize_zp(to_dev(w, "f32"), 8, 32, torch.bfloat16)
    assert int(z[0, 0]) == 255 and int(n[0, 0]) == 0 and int(n[0, 1]) == 155
    assert (n[0, 2:] == 255).all()


@pytest.mark.parametrize("bits,K,G", [(4, 128, 32), (4, 512, 64), (4, 256, 256), (8, 64, 32),
                                      (8, 512, 512)])
@pytest.mark.parametrize("V", [1, 64, 65, 200])
def test_pack_zp_byte_exact(bits, K, G, V):
    need_gpu()
    rng = np.random.default_rng(V * 3 + K + bits)
    n = rng.integers(0, QR[bits] + 1, size=(V, K)).astype(np.uint8)
    s = rng.integers(0, 0x7C00, size=(V, K // G)).astype(np.uint16)
    z = rng.integers(0, QR[bits] + 1, size=(V, K // G)).astype(np.uint8)
    blob = lmh.pack_zp(torch.from_numpy(n).to(DEV), _s_dev(s, "f16"), torch.from_numpy(z).to(DEV),
                       bits, G)
    got = blob.cpu().numpy()
    want = oracle.pack_zp(n, s, z, bits, G)
    assert got.size == want.size
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"first differing bytes at {bad[:8]}"


@pytest.mark.parametrize("wdt", ["f32", "bf16"])
@pytest.mark.parametrize("bits,G", [(4, 32), (4, 64), (4, 128), (4, 256), (8, 64), (8, 128),
                                    (8, 256)])
@pytest.mark.parametrize("sdt", ["f16", "bf16"])
def test_quantize_pack_zp_byte_exact(wdt, bits, G, sdt):
    need_gpu()
    V, K = 131, 512
    w = _weights(V, K, wdt, seed=bits * 31 + G, zero_rows=(0,))
    got = lmh.quantize_pack(to_dev(w, wdt), bits | ZP, G, TD[sdt]).cpu().numpy()
    want = oracle.pack_zp(*oracle.quantize_asym(w, bits, G, OD[sdt], w_dtype=OD[wdt]), bits, G)
    assert got.size == want.size
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"first differing bytes at {bad[:8]}"


def test_quantize_pack_zp_chunked_and_two_step():
    """Row chunks in any order give the one-call blob, which equals the two-step
    pack_zp(quantize_zp(w)); clip search is refused for this form."""
    need_gpu()
    V, K, bits, G = 333, 512, 4, 64
    w = _weights(V, K, "f16", seed=3)
    wd = to_dev(w, "f16")
    whole = lmh.quantize_pack(wd, bits | ZP, G, torch.float16)
    n, s, z = lmh.quantize_zp(wd, bits, G, torch.float16)
    assert torch.equal(lmh.pack_zp(n, s, z, bits, G), whole)
    out = torch.full_like(whole, 0xA5)
    for r0 in list(range(0, V, 128))[::-1]:
        lmh.quantize_pack(wd[r0:r0 + 128], bits | ZP, G, torch.float16, V=V, row0=r0, out=out)
    assert torch.equal(out, whole)
    with pytest.raises(lmh.LmheadError):
        lmh.quantize_pack(wd, bits | ZP, G, torch.float16, "mse")


# ---- logits ---------------------------------------------------------------------------

def _zp_head(V, K, bits, G, sdt, seed, zero_rows=()):
    w = _weights(V, K, "f32", seed, zero_rows)
    n, s, z = oracle.quantize_asym(w, bits, G, OD[sdt])
    blob = torch.from_numpy(oracle.pack_zp(n, s, z, bits, G)).to(DEV)
    return n, s, z, blob


def _run(xnp, xdt, blob, V, K, bits, G, sdt, path, bias=None, ldy=None, out_dtype=torch.float32):
    x = to_dev(xnp, xdt)
    M = xnp.shape[0]
    ldy = ldy or V
    out = torch.full((M, ldy), float("nan"), dtype=out_dtype, device=DEV)
    b = None if bias is None else torch.from_numpy(bias).to(DEV)
    lmh.logits(x, blob, V, K, bits | ZP, G, TD[sdt], bias=b, out=out, path=path)
    torch.cuda.synchronize()
    y = out.float().cpu().numpy()
    if ldy > V:
        assert np.isnan(y[:, V:]).all(), "columns past V were written"
    return y[:, :V]


CASES = [  # bits, G, K
    (4, 32, 512), (4, 64, 1024), (4, 128, 512), (4, 256, 1024),
    (8, 32, 256), (8, 64, 512), (8, 128, 1024), (8, 512, 512),
]


@pytest.mark.parametrize("bits,G,K", CASES)
@pytest.mark.parametrize("xdt,sdt", [("f16", "f16"), ("bf16", "bf16")])
@pytest.mark.parametrize("path,Ms", [(GEMV, (1, 2, 4)), (MFMA, (1, 5, 17, 40)),
                                     (LDS, (3, 33, 65)), (XRES, (7, 65, 130)), (SPLITK, (3, 9, 16))])
def test_logits_zp_vs_oracle(bits, G, K, xdt, sdt, path, Ms):
    need_gpu()
    V = 64 * 5 + 37
    n, s, z, blob = _zp_head(V, K, bits, G, sdt, seed=K + G + bits, zero_rows=(3, V - 1))
    wdq = _dq(n, s, z, sdt, G)
    worst = 0.0
    for M in Ms:
        x = synth.random_x(M, K, seed=M + 7, dtype=xdt)
        y = _run(x, xdt, blob, V, K, bits, G, sdt, path)
        y_or = oracle.logits_zp(x, n, s, z, OD[sdt], G, x_dtype=OD[xdt])
        y_abs = _abs_terms(x, xdt, wdq)
        worst = max(worst, check_logits(y, y_or, y_abs, K, G, what=f"M={M} path={path}"))
    print(f"zp bits={bits} G={G} K={K} x={xdt} path={path}: max row rel err {worst:.2e}")


@pytest.mark.parametrize("bits,G", [(4, 64), (4, 128), (8, 128), (8, 32)])
@pytest.mark.parametrize("path", [GEMV, MFMA, LDS, XRES, SPLITK])
def test_logits_zp_one_hot_exposes_layout(bits, G, path):
    """x = e_k gives y[v] = (n[v,k] - z[v,k/G]) * s[v,k/G] exactly: a misplaced
    zero-point byte shows up bit for bit."""
    need_gpu()
    V, K = 130, 256
    n, s, z, blob = _zp_head(V, K, bits, G, "f16", seed=11)
    wdq = _dq(n, s, z, "f16", G).astype(np.float64)
    ks = [0, 1, 7, 8, 31, 32, 63, 64, 100, 127, 128, 200, 255]
    for i in range(0, len(ks), 4):
        kk = ks[i:i + 4]
        x = np.zeros((len(kk), K), dtype=np.float16)
        for m, k in enumerate(kk):
            x[m, k] = 1.0
        y = _run(x, "f16", blob, V, K, bits, G, "f16", path)
        for m, k in enumerate(kk):
            assert np.array_equal(y[m].astype(np.float64), wdq[:, k]), f"column {k}"


@pytest.mark.parametrize("bits,G", [(4, 64), (4, 128), (8, 128), (8, 32)])
def test_fixed_zero_point_is_the_symmetric_head_bit_for_bit(bits, G):
    """A zero-point blob with z = 8 / 128 and n = q + 8 / q + 128 gives exactly the
    symmetric blob's logits on every kernel (the unpacked operands are equal)."""
    need_gpu()
    V, K = 200, 512
    w = synth.random_weight((V, K), 0.02, 19)
    q, s = oracle.quantize(w, bits, G, oracle.F16)
    zc = 8 if bits == 4 else 128
    n = (q.astype(np.int16) + zc).astype(np.uint8)
    z = np.full((V, K // G), zc, dtype=np.uint8)
    sym = torch.from_numpy(oracle.pack(q, s, bits, G)).to(DEV)
    zpb = torch.from_numpy(oracle.pack_zp(n, s, z, bits, G)).to(DEV)
    for path, M in [(GEMV, 1), (GEMV, 3), (MFMA, 9), (LDS, 40), (XRES, 100), (SPLITK, 15)]:
        x = to_dev(synth.random_x(M, K, seed=M), "f16")
        ys = lmh.logits(x, sym, V, K, bits, G, torch.float16, path=path)
        yz = lmh.logits(x, zpb, V, K, bits | ZP, G, torch.float16, path=path)
        assert torch.equal(ys, yz), f"path {path} M={M}"


@pytest.mark.parametrize("bits,G", [(4, 64), (8, 128)])
def test_mfma_kernels_agree_bit_for_bit_zp(bits, G):
    need_gpu()
    V, K = 400, 1024
    n, s, z, blob = _zp_head(V, K, bits, G, "bf16", seed=23)
    for M in (5, 33, 70):
        x = synth.random_x(M, K, seed=M, dtype="bf16")
        ys = [_run(x, "bf16", blob, V, K, bits, G, "bf16", p) for p in (MFMA, LDS, XRES)]
        assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2]), f"M={M}"


@pytest.mark.parametrize("path,M", [(GEMV, 2), (MFMA, 8), (LDS, 20), (XRES, 70), (SPLITK, 12)])
def test_logits_zp_bias_stride_and_16bit_output(path, M):
    need_gpu()
    V, K, bits, G = 200, 512, 4, 64
    n, s, z, blob = _zp_head(V, K, bits, G, "f16", seed=5)
    bias = synth.random_weight((1, V), 1.0, 6)[0]
    x = synth.random_x(M, K, seed=9)
    y = _run(x, "f16", blob, V, K, bits, G, "f16", path, bias=bias, ldy=V + 45)
    y_or = oracle.logits_zp(x, n, s, z, oracle.F16, G, bias=bias)
    check_logits(y, y_or, _abs_terms(x, "f16", _dq(n, s, z, "f16", G)), K, G, what="bias",
                 bias=bias)
    for od in (torch.float16, torch.bfloat16):
        y16 = _run(x, "f16", blob, V, K, bits, G, "f16", path, bias=bias, out_dtype=od)
        want = torch.from_numpy(y).to(od).float().numpy()
        assert np.array_equal(y16, want), f"{od}: not the fp32 result rounded once"


def test_logits_topk_zp():
    """The one-call logits + exact top-K equals logits then rescoring, on a
    zero-point head."""
    need_gpu()
    V, K, bits, G = 3000, 512, 4, 64
    w = _weights(V, K, "f16", seed=29)
    wd = to_dev(w, "f16")
    blob = lmh.quantize_pack(wd, bits | ZP, G, torch.float16)
    x = to_dev(synth.random_x(3, K, seed=4), "f16")
    y = lmh.logits(x, blob, V, K, bits | ZP, G, torch.float16)
    idx0, val0, top0 = lmh.topk_rescore(x, wd, y, 8)
    out = torch.empty_like(y)
    idx1, val1, top1 = lmh.logits_topk(x, blob, V, K, bits | ZP, G, torch.float16, wd, 8, out=out)
    assert torch.equal(idx0, idx1) and torch.equal(val0, val1) and torch.equal(top0, top1)
    assert torch.equal(out, y)


# ---- embedding ------------------------------------------------------------------------

@pytest.mark.parametrize("bits,K,G", [(4, 256, 32), (4, 512, 128), (8, 128, 64), (8, 512, 512)])
@pytest.mark.parametrize("sdt", ["f16", "bf16"])
@pytest.mark.parametrize("odt", ["f32", "f16", "bf16"])
def test_embed_zp_bit_exact(bits, K, G, sdt, odt):
    need_gpu()
    V = 200
    n, s, z, blob = _zp_head(V, K, bits, G, sdt, seed=K + bits)
    # zero scales with n != z give -0 or +0 rows: the sign must survive
    ids = np.array([0, 5, V - 1, 63, 64, -1, V, 199, 8, 9, 3, 3], dtype=np.int32)
    out = lmh.embed(torch.from_numpy(ids).to(DEV), blob, V, K, bits | ZP, G, TD[sdt], TD[odt])
    torch.cuda.synchronize()
    want = oracle.embed_zp(n, s, z, OD[sdt], G, ids, OD[odt])
    got = out.cpu().numpy() if odt == "f32" else bits16(out)
    if odt == "f32":
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    else:
        assert np.array_equal(got, want)


# ---- full size -------------------------------------------------------------------------

def test_fullsize_zp_w4g64_sampled():
    """The 151936 x 1024 int4 g64 head in the zero-point form: the fused
    quantizer's bytes on sampled row blocks and the logits of sampled rows at
    M = 1, 32 and 256, in the benchmark's launch configuration."""
    need_gpu()
    wl = synth.WORKLOADS["w4g64_151936x1024"]
    W = synth.weight(wl)
    Wd = to_dev(W, wl.w_dtype)
    bits, G, V, K = wl.bits, wl.group, wl.V, wl.K
    blob = lmh.quantize_pack(Wd, bits | ZP, G, TD[wl.scale_dtype])
    torch.cuda.synchronize()
    rng = np.random.default_rng(41)
    blocks = np.unique(np.concatenate([rng.choice((V + 63) // 64, 10, replace=False),
                                       [0, (V - 1) // 64]]))
    rows = (blocks[:, None] * 64 + np.arange(64)[None, :]).ravel()
    rows = rows[rows < V]
    no, so, zo = oracle.quantize_asym(np.ascontiguousarray(W[rows]), bits, G, OD[wl.scale_dtype],
                                      w_dtype=OD[wl.w_dtype])
    bl = blob.cpu().numpy()
    NB, NG, NC = (V + 63) // 64, K // G, K // 128
    wreg, sreg = NB * 64 * K // 2, NB * 64 * NG * 2
    for b in blocks:
        sel = (rows >= b * 64) & (rows < b * 64 + 64)
        ob = oracle.pack_zp(no[sel], so[sel], zo[sel], bits, G)
        ow, osc = 64 * K // 2, 64 * NG * 2
        assert np.array_equal(bl[b * NC * 4096:(b + 1) * NC * 4096], ob[:ow]), f"block {b} codes"
        assert np.array_equal(bl[wreg + b * NG * 128:wreg + (b + 1) * NG * 128], ob[ow:ow + osc])
        assert np.array_equal(bl[wreg + sreg + b * NG * 64:wreg + sreg + (b + 1) * NG * 64],
                              ob[ow + osc:]), f"block {b} zero points"
    wdq = _dq(no, so, zo, wl.scale_dtype, G)
    for M in (1, 32, 256):
        x = synth.activations(wl, M)
        y = lmh.logits(to_dev(x, wl.x_dtype), blob, V, K, bits | ZP, G, TD[wl.scale_dtype])
        ys = y[:, torch.from_numpy(rows).to(DEV)].cpu().numpy()
        y_or = oracle.logits_zp(x, no, so, zo, OD[wl.scale_dtype], G, x_dtype=OD[wl.x_dtype])
        rel = check_logits(ys, y_or, _abs_terms(x, wl.x_dtype, wdq), K, G, what=f"zp M={M}")
        print(f"zp w4g64 M={M}: max row rel err on {len(rows)} sampled rows {rel:.2e}")
    del Wd, blob
    torch.cuda.empty_cache()
