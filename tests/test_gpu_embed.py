"""Embedding gather from the packed blob (lmhead_embed) against the oracle:
bit-exact rows for every layout, scale type and output type; repeated and
out-of-range ids; strided output rows; full-size heads on sampled ids."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, OD, TD, gpu, need_gpu, to_dev

pytestmark = gpu


def _table(V, K, bits, G, sdt, seed):
    rng = np.random.default_rng(seed)
    lo, hi = (-8, 7) if bits == 4 else (-128, 127)
    q = rng.integers(lo, hi + 1, size=(V, K)).astype(np.int8)
    if sdt == "f16":
        s = rng.integers(0x0001, 0x7800, size=(V, K // G)).astype(np.uint16)
    else:
        s = rng.integers(0x2000, 0x5000, size=(V, K // G)).astype(np.uint16)
    s[:, 0] = 0                                     # zero scales
    return q, s


def _blob(q, s, bits, G, sdt):
    sd = torch.from_numpy(s.view(np.int16)).view(TD[sdt]).to(DEV)
    return lmh.pack(torch.from_numpy(q).to(DEV), sd, bits, G)


def _host(t):
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("bits,K,G", [(4, 128, 32), (4, 256, 64), (4, 384, 128), (4, 512, 256),
                                      (8, 64, 32), (8, 192, 64), (8, 256, 128), (8, 512, 512)])
@pytest.mark.parametrize("sdt", ["f16", "bf16"])
@pytest.mark.parametrize("odt", ["f32", "f16", "bf16"])
def test_embed_bit_exact(bits, K, G, sdt, odt):
    need_gpu()
    V = 133
    q, s = _table(V, K, bits, G, sdt, seed=bits * 100 + G)
    blob = _blob(q, s, bits, G, sdt)
    ids = np.array([0, 1, 63, 64, 132, 5, 5, 77, -1, 133, 2**31 - 1, 100], dtype=np.int32)
    got = lmh.embed(torch.from_numpy(ids).to(DEV), blob, V, K, bits, G, TD[sdt], TD[odt])
    want = oracle.embed(q, s, OD[sdt], G, ids, OD[odt])
    g = _host(got)
    assert np.array_equal(g, want), f"first mismatch at {np.argwhere(g != want)[:4]}"


def test_embed_strided_out_and_empty():
    need_gpu()
    V, K, bits, G = 300, 256, 4, 64
    q, s = _table(V, K, bits, G, "f16", seed=9)
    blob = _blob(q, s, bits, G, "f16")
    ids = torch.arange(299, -1, -7, dtype=torch.int32, device=DEV)
    out = torch.full((ids.numel(), K + 40), 7.0, dtype=torch.float32, device=DEV)
    lmh.embed(ids, blob, V, K, bits, G, torch.float16, out=out[:, :K])
    want = oracle.embed(q, s, oracle.F16, G, ids.cpu().numpy(), oracle.F32)
    assert np.array_equal(out[:, :K].cpu().numpy(), want)
    assert (out[:, K:] == 7.0).all(), "columns past K were written"
    e = lmh.embed(torch.empty(0, dtype=torch.int32, device=DEV), blob, V, K, bits, G)
    assert e.shape == (0, K)


def test_embed_matches_logits_of_one_hot():
    """The gathered table and the logits kernel read the blob the same way: the
    logits of the one-hot inputs e_k are the embedding rows' column k."""
    need_gpu()
    V, K, bits, G = 200, 256, 4, 64
    q, s = _table(V, K, bits, G, "f16", seed=4)
    blob = _blob(q, s, bits, G, "f16")
    eye = torch.eye(K, dtype=torch.float16, device=DEV)[:48]
    y = lmh.logits(eye, blob, V, K, bits, G, torch.float16)        # [48, V]
    emb = lmh.embed(torch.arange(V, dtype=torch.int32, device=DEV), blob, V, K, bits, G,
                    torch.float16, torch.float32)
    assert torch.equal(y, emb[:, :48].t().contiguous())


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_embed_fullsize_sampled(name):
    """Full-size heads: the rows of sampled ids, each quantized by the oracle,
    gathered bit-exactly from the blob the fused quantizer writes."""
    need_gpu()
    w = synth.WORKLOADS[name]
    rng = np.random.default_rng(w.wid)
    ids = np.unique(np.concatenate([rng.integers(0, w.V, size=40), [0, w.V - 1, w.V - 64]]))
    ids = ids.astype(np.int32)
    W = synth.weight(w)
    blob = lmh.quantize_pack(to_dev(W, w.w_dtype), w.bits, w.group, TD[w.scale_dtype], w.clip)
    ratios = oracle.MSE_RATIOS if w.clip == "mse" else oracle.RTN_RATIOS
    qo, so = oracle.quantize(np.ascontiguousarray(W[ids]), w.bits, w.group, OD[w.scale_dtype],
                             ratios, w_dtype=OD[w.w_dtype])
    del W
    odt = w.x_dtype
    got = lmh.embed(torch.from_numpy(ids).to(DEV), blob, w.V, w.K, w.bits, w.group,
                    TD[w.scale_dtype], TD[odt])
    want = oracle.embed(qo, so, OD[w.scale_dtype], w.group, np.arange(len(ids)), OD[odt])
    assert np.array_equal(_host(got), want)
    del blob
    torch.cuda.empty_cache()
