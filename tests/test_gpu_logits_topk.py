"""GPU logits + top-K rescoring in one call (lmhead_logits_topk).

The single call must give exactly what the two separate calls give
(lmhead_logits, then lmhead_topk_rescore): the same indices in the same
order, bit-identical rescored values, top-1 and scattered logits, with or
without the logits stored.  The selection itself is checked against the
oracle's top-K of the GPU's own logits (reading R5 of oracle/lmh_oracle.c: value descending, then index ascending)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, OD, TD, gpu, need_gpu, to_dev

pytestmark = gpu


def _head(V, K, bits, G, seed):
    w = synth.random_weight((V, K), 0.02, seed)
    q, s = oracle.quantize(w, bits, G, oracle.F16)
    blob = torch.from_numpy(oracle.pack(q, s, bits, G)).to(DEV)
    return w, blob


def _separate(x, blob, V, K, bits, G, wref, topk, path):
    y = lmh.logits(x, blob, V, K, bits, G, torch.float16, path=path)
    idx, val, top1 = lmh.topk_rescore(x, wref, y, topk)
    return y, idx, val, top1


@pytest.mark.parametrize("bits,G,K", [(4, 64, 1024), (4, 128, 512), (8, 128, 1024), (4, 32, 256)])
@pytest.mark.parametrize("M", [1, 2, 5, 40])
@pytest.mark.parametrize("topk", [1, 8, 64])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_one_call_equals_separate_calls(bits, G, K, M, topk, xdt):
    need_gpu()
    V = 64 * 83 + 21  # 84 blocks, a ragged last one
    w, blob = _head(V, K, bits, G, seed=bits * 1000 + G + K)
    wref = torch.from_numpy(w.astype(np.float16)).to(DEV)
    x = to_dev(synth.random_x(M, K, seed=M + topk, dtype=xdt), xdt)
    y0, i0, v0, t0 = _separate(x, blob, V, K, bits, G, wref, topk, path=lmh.PATH_AUTO)
    y1 = torch.full((M, V + 7), float("nan"), device=DEV)[:, :V]
    i1, v1, t1 = lmh.logits_topk(x, blob, V, K, bits, G, torch.float16, wref, topk, out=y1)
    i2, v2, t2 = lmh.logits_topk(x, blob, V, K, bits, G, torch.float16, wref, topk, out=None)
    torch.cuda.synchronize()
    for i, v, t in ((i1, v1, t1), (i2, v2, t2)):
        assert torch.equal(i, i0), "selection differs"
        assert torch.equal(v, v0), "rescored values differ"
        assert torch.equal(t, t0), "top-1 differs"
    assert torch.equal(y1, y0), "logits (with the rescored values scattered in) differ"


def test_selection_is_the_oracle_top_k():
    """The indices are the oracle's top-K (value descending, index ascending)
    of the GPU's own quantized logits."""
    need_gpu()
    V, K, bits, G, topk = 64 * 300 + 17, 1024, 4, 64, 16
    w, blob = _head(V, K, bits, G, seed=91)
    wref = torch.from_numpy(w.astype(np.float16)).to(DEV)
    x = to_dev(synth.random_x(1, K, seed=5), "f16")
    y = lmh.logits(x, blob, V, K, bits, G, torch.float16)
    torch.cuda.synchronize()
    yq = y.cpu().numpy()
    idx, _, _ = lmh.logits_topk(x, blob, V, K, bits, G, torch.float16, wref, topk)
    torch.cuda.synchronize()
    want = oracle.topk(yq[0], topk)
    assert np.array_equal(idx.cpu().numpy()[0].astype(np.int64), want)


@pytest.mark.parametrize("V", [151936, 600000])
def test_full_size_rows_match_separate_calls(V):
    """A 151936 x 1024 int4 g64 head at M = 1, and a 600000-row one (pass 1
    then takes 4096-entry blocks to stay within 256 lists)."""
    need_gpu()
    K, bits, G = 1024, 4, 64
    gen = torch.Generator(device=DEV).manual_seed(V)
    Wd = torch.randn(V, K, device=DEV, generator=gen) * 0.02
    q, s = lmh.quantize(Wd, bits, G, torch.float16, "rtn")
    blob = lmh.pack(q, s, bits, G)
    wref = Wd.half()
    del q, s, Wd
    x = to_dev(synth.random_x(1, K, seed=3), "f16")
    y0, i0, v0, t0 = _separate(x, blob, V, K, bits, G, wref, 8, path=lmh.PATH_AUTO)
    i1, v1, t1 = lmh.logits_topk(x, blob, V, K, bits, G, torch.float16, wref, 8)
    torch.cuda.synchronize()
    assert torch.equal(i1, i0) and torch.equal(v1, v0) and torch.equal(t1, t0)


def _dev_head(V, K, bits, G, seed, zp=False, zero=False):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    Wd = torch.randn(V, K, device=DEV, generator=gen) * 0.02
    if zero:
        Wd.zero_()
    bb = bits | lmh.ZP if zp else bits
    blob = lmh.quantize_pack(Wd, bb, G, torch.float16)
    return Wd.half(), blob, bb


@pytest.mark.parametrize("V,topk", [(1, 1), (2, 1), (5, 4), (64, 8), (65, 16), (64 * 256, 16),
                                    (64 * 256 + 1, 1), (64 * 4096, 8), (64 * 4096 + 3, 8),
                                    (3000, 17)])
@pytest.mark.parametrize("zp", [False, True])
def test_decode_path_edges(V, topk, zp):
    """M = 1 runs the GEMV with its per-block top-K lists and one merge kernel
    (topk <= 16, at most 4096 row blocks; else the two-pass path): single and
    ragged blocks, V below a block, the largest merged list count and one
    block more, topk 16 and 17, with a bias and on zero-point heads.  The
    result equals the separate logits + rescoring calls bit for bit."""
    need_gpu()
    K, bits, G = 256, 4, 64
    wref, blob, bb = _dev_head(V, K, bits, G, seed=V + topk, zp=zp)
    gen = torch.Generator(device=DEV).manual_seed(7)
    bias = torch.randn(V, device=DEV, generator=gen)
    x = to_dev(synth.random_x(1, K, seed=topk, dtype="f16"), "f16")
    y0 = lmh.logits(x, blob, V, K, bb, G, torch.float16, bias=bias)
    i0, v0, t0 = lmh.topk_rescore(x, wref, y0, topk)
    y1 = torch.full((1, V + 5), float("nan"), device=DEV)[:, :V]
    i1, v1, t1 = lmh.logits_topk(x, blob, V, K, bb, G, torch.float16, wref, topk, bias=bias, out=y1)
    i2, v2, t2 = lmh.logits_topk(x, blob, V, K, bb, G, torch.float16, wref, topk, bias=bias)
    torch.cuda.synchronize()
    for i, v, t in ((i1, v1, t1), (i2, v2, t2)):
        assert torch.equal(i, i0) and torch.equal(v, v0) and torch.equal(t, t0)
    assert torch.equal(y1, y0)


@pytest.mark.parametrize("topk", [2, 8, 16])
def test_decode_path_clustered_blocks(topk):
    """Most of the row's top logits in a few 64-row blocks (those rows' weights
    scaled up), the rest spread: the merge then takes several entries from
    some lists (up to all of one) and one from others.  Equal to the separate
    calls bit for bit, and the selection is the oracle's top-K."""
    need_gpu()
    V, K, bits, G = 64 * 200 + 13, 512, 4, 64
    gen = torch.Generator(device=DEV).manual_seed(topk)
    Wd = torch.randn(V, K, device=DEV, generator=gen) * 0.02
    Wd[64 * 7: 64 * 7 + 5] *= 6.0          # five rows of block 7
    Wd[64 * 120 + 30: 64 * 120 + 64] *= 4.0  # the second half of block 120
    Wd[V - 3:] *= 5.0                        # the ragged last block
    blob = lmh.quantize_pack(Wd, bits, G, torch.float16)
    wref = Wd.half()
    for seed in range(4):
        x = to_dev(synth.random_x(1, K, seed=seed, dtype="f16"), "f16")
        y0 = lmh.logits(x, blob, V, K, bits, G, torch.float16)
        i0, v0, t0 = lmh.topk_rescore(x, wref, y0, topk)
        i1, v1, t1 = lmh.logits_topk(x, blob, V, K, bits, G, torch.float16, wref, topk)
        torch.cuda.synchronize()
        assert torch.equal(i1, i0) and torch.equal(v1, v0) and torch.equal(t1, t0), seed
        yq = lmh.logits(x, blob, V, K, bits, G, torch.float16).cpu().numpy()
        assert np.array_equal(i1.cpu().numpy()[0].astype(np.int64), oracle.topk(yq[0], topk)), seed


def test_decode_path_all_ties():
    """An all-zero head: every logit is 0, so the top-K are the first K indices
    (index ascending on ties) and the top-1 is row 0."""
    need_gpu()
    V, K, bits, G, topk = 64 * 37 + 9, 512, 4, 128, 16
    wref, blob, bb = _dev_head(V, K, bits, G, seed=1, zero=True)
    x = to_dev(synth.random_x(1, K, seed=2, dtype="bf16"), "bf16")
    idx, val, top1 = lmh.logits_topk(x, blob, V, K, bb, G, torch.float16, wref, topk)
    torch.cuda.synchronize()
    assert idx.cpu().numpy()[0].tolist() == list(range(topk))
    assert (val == 0).all() and int(top1[0]) == 0


@pytest.mark.parametrize("M,topk", [(1, 8), (64, 8), (64, 16)])
def test_rescoring_recovers_the_reference_top1(M, topk):
    """Whenever the unquantized weight's top-1 (lmhead_dense_logits: exact 16-bit
    products, fp32 sums) is among the quantized top-K and wins by a clear
    margin, the rescored top-1 is that row (the rescoring recomputes those K
    rows from the same weight)."""
    need_gpu()
    V, K, bits, G = 64 * 200 + 5, 512, 4, 64
    w, blob = _head(V, K, bits, G, seed=M + topk)
    wref = torch.from_numpy(w.astype(np.float16)).to(DEV)
    wl = synth.WORKLOADS["tiny_w4g64_50304x512"]
    x = to_dev(synth.decode_states(wl, 0, M), "f16")
    yq = lmh.logits(x, blob, V, K, bits, G, torch.float16)
    ref = torch.cat([lmh.dense_logits(x[i:i + 4], wref) for i in range(0, M, 4)])
    _, _, top1 = lmh.logits_topk(x, blob, V, K, bits, G, torch.float16, wref, topk)
    torch.cuda.synchronize()
    ref1 = torch.argmax(ref, dim=1)
    t2 = torch.topk(ref, 2, dim=1).values
    clear = (t2[:, 0] - t2[:, 1]) > 1e-3
    inset = (torch.topk(yq, topk, dim=1).indices == ref1[:, None]).any(dim=1)
    sel = clear & inset
    assert sel.any()
    assert torch.equal(top1.long()[sel], ref1[sel])
