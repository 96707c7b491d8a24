"""GPU quantizer and packer against the oracle: bit-exact (q, s) and byte-exact blobs."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, OD, TD, bits16, gpu, need_gpu, to_dev

pytestmark = gpu

QR = {4: (-8, 7), 8: (-128, 127)}


def _weights(V, K, wdt, seed, zero_rows=()):
    w = synth.random_weight((V, K), 0.02, seed, zero_rows)
    w[V // 3, : K // 2] *= 9.0          # outliers: the clip search moves
    w[V // 2, 32:64] = 0.0               # an all-zero group in a live row
    w[min(5, V - 1), :32] *= 1e-7         # tiny groups: the scale floor
    if wdt == "f16":
        return w.astype(np.float16)
    if wdt == "bf16":
        return synth.to_bf16_bits(w)
    return w


@pytest.mark.parametrize("wdt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits,G", [(4, 32), (4, 64), (4, 128), (8, 128), (8, 256)])
@pytest.mark.parametrize("sdt", ["f16", "bf16"])
@pytest.mark.parametrize("clip", ["rtn", "mse"])
def test_quantize_bit_exact(wdt, bits, G, sdt, clip):
    need_gpu()
    V, K = 131, 512
    w = _weights(V, K, wdt, seed=bits * 1000 + G, zero_rows=(0, V - 1))
    q, s = lmh.quantize(to_dev(w, wdt), bits, G, TD[sdt], clip)
    torch.cuda.synchronize()
    ratios = oracle.MSE_RATIOS if clip == "mse" else oracle.RTN_RATIOS
    qo, so = oracle.quantize(w, bits, G, OD[sdt], ratios, w_dtype=OD[wdt])
    qg = q.cpu().numpy()
    sg = bits16(s)
    assert np.array_equal(sg, so), f"scales differ at {np.argwhere(sg != so)[:5]}"
    assert np.array_equal(qg, qo), f"codes differ at {np.argwhere(qg != qo)[:5]}"


def test_quantize_ties_hand_case():
    """Half-way quotients round to even (same hand case as the oracle pin)."""
    need_gpu()
    u = np.float32(2.0**-6)
    w = np.zeros((2, 64), dtype=np.float32)
    w[0, :10] = np.array([7, 2.5, 3.5, -1.5, 0.5, -0.5, -2.5, 1.5, 4.5, -3.5], np.float32) * u
    for sdt in ("f16", "bf16"):
        q, s = lmh.quantize(to_dev(w, "f32"), 4, 64, TD[sdt], "rtn")
        assert list(q[0, :10].cpu().numpy()) == [7, 2, 4, -2, 0, 0, -2, 2, 4, -4]
        assert (q[1] == 0).all() and int(bits16(s)[1, 0]) == 0


@pytest.mark.parametrize("bits,K,G", [(4, 128, 32), (4, 512, 64), (4, 384, 128), (4, 256, 256),
                                      (8, 64, 32), (8, 192, 64), (8, 512, 512)])
@pytest.mark.parametrize("V", [1, 64, 65, 200])
def test_pack_byte_exact(bits, K, G, V):
    need_gpu()
    rng = np.random.default_rng(V * 7 + K + bits)
    lo, hi = QR[bits]
    q = rng.integers(lo, hi + 1, size=(V, K)).astype(np.int8)
    s = rng.integers(0, 0x7C00, size=(V, K // G)).astype(np.uint16)
    blob = lmh.pack(torch.from_numpy(q).to(DEV),
                    torch.from_numpy(s.view(np.int16)).view(torch.float16).to(DEV), bits, G)
    got = blob.cpu().numpy()
    want = oracle.pack(q, s, bits, G)
    assert got.size == want.size
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"first differing bytes at {bad[:8]}"
    q2, s2 = oracle.unpack(got, V, K, bits, G)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_pack_twice_same_bytes():
    need_gpu()
    w = _weights(100, 256, "f32", 3)
    q, s = lmh.quantize(to_dev(w, "f32"), 4, 64, torch.float16, "rtn")
    a = lmh.pack(q, s, 4, 64)
    b = lmh.pack(q, s, 4, 64)
    assert torch.equal(a, b)


# ---- fused quantize + pack (lmhead_quantize_pack) -------------------------------------------

def _oracle_blob(w, wdt, bits, G, sdt, clip):
    ratios = oracle.MSE_RATIOS if clip == "mse" else oracle.RTN_RATIOS
    qo, so = oracle.quantize(w, bits, G, OD[sdt], ratios, w_dtype=OD[wdt])
    return oracle.pack(qo, so, bits, G)


def _first_diff(got, want):
    bad = np.nonzero(got != want)[0]
    return bad[:8]


@pytest.mark.parametrize("wdt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits,G", [(4, 32), (4, 64), (4, 128), (4, 256), (8, 32), (8, 64),
                                    (8, 128), (8, 256), (8, 512)])
@pytest.mark.parametrize("sdt", ["f16", "bf16"])
@pytest.mark.parametrize("clip", ["rtn", "mse"])
def test_quantize_pack_byte_exact(wdt, bits, G, sdt, clip):
    """The fused kernel writes the oracle's pack(quantize(w)) byte for byte."""
    need_gpu()
    V, K = 131, 512
    w = _weights(V, K, wdt, seed=bits * 77 + G, zero_rows=(0, V - 1))
    got = lmh.quantize_pack(to_dev(w, wdt), bits, G, TD[sdt], clip).cpu().numpy()
    want = _oracle_blob(w, wdt, bits, G, sdt, clip)
    assert got.size == want.size
    assert np.array_equal(got, want), f"first differing bytes at {_first_diff(got, want)}"


@pytest.mark.parametrize("bits,G,wdt,clip", [(4, 128, "bf16", "mse"), (8, 64, "f32", "rtn"),
                                             (8, 256, "f16", "mse"), (4, 32, "f16", "rtn"),
                                             (4, 512, "f32", "rtn"), (8, 256, "bf16", "rtn")])
def test_quantize_pack_chunked(bits, G, wdt, clip):
    """Chunks of whole 64-row blocks, in any order and from a strided source,
    write the same bytes as one call over the head; the last chunk may be ragged."""
    need_gpu()
    V, K = 333, 512
    w = _weights(V, K, wdt, seed=G + bits, zero_rows=(7,))
    wd = to_dev(w, wdt)
    whole = lmh.quantize_pack(wd, bits, G, torch.float16, clip)
    wide = torch.zeros((V, K + 64), dtype=wd.dtype, device=DEV)
    wide[:, 16:16 + K] = wd            # rows strided by K + 64, start 32/64 bytes in
    for chunk in (64, 128, 192):
        out = torch.full_like(whole, 0xA5)
        starts = list(range(0, V, chunk))[::-1]          # last chunk first
        for r0 in starts:
            n = min(chunk, V - r0)
            src = wide[r0:r0 + n, 16:16 + K]
            lmh.quantize_pack(src, bits, G, torch.float16, clip, V=V, row0=r0, out=out)
        assert torch.equal(out, whole), f"chunk {chunk}: differs from the whole-head call"
    want = _oracle_blob(w, wdt, bits, G, "f16", clip)
    assert np.array_equal(whole.cpu().numpy(), want)


def test_quantize_pack_host_streamed():
    need_gpu()
    V, K = 300, 256
    w = _weights(V, K, "bf16", seed=5)
    wh = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
    got = lmh.quantize_pack_host(wh, 4, 128, torch.bfloat16, "mse", chunk_rows=128, device=DEV)
    want = _oracle_blob(w, "bf16", 4, 128, "bf16", "mse")
    assert np.array_equal(got.cpu().numpy(), want)


def _near_half_weights(bits, sdt, V=64, K=256, G=64, seed=0):
    """Groups whose quotients w/s sit within a few ulps of half-integers, where a
    quotient from the reciprocal can round differently from the IEEE quotient."""
    rng = np.random.default_rng(seed)
    qmax = 7 if bits == 4 else 127
    w = np.zeros((V, K), dtype=np.float32)
    for v in range(V):
        for g in range(K // G):
            s32 = np.float32(rng.uniform(0.5, 2.0) * 2.0 ** rng.integers(-12, 4))
            # the scale the quantizer derives from amax = qmax * s32 at ratio 1.0
            amax = np.float32(qmax) * s32
            s = oracle.widen16(oracle.encode16(np.array([amax * np.float32(1.0 / qmax)],
                                                        np.float32), OD[sdt]), OD[sdt])[0]
            s = np.float32(s)
            h = rng.integers(-qmax, qmax, size=G) + 0.5
            ulp = rng.integers(-4, 5, size=G).astype(np.float64)
            vals = (h * (1.0 + ulp * 2.0 ** -24) * float(s)).astype(np.float32)
            vals[0] = amax
            w[v, g * G:(g + 1) * G] = vals
    return w


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sdt", ["f16", "bf16"])
@pytest.mark.parametrize("clip", ["rtn", "mse"])
def test_near_half_quotients(bits, sdt, clip):
    """Both GPU quantizers agree with the oracle where the rounding of w/s to an
    integer depends on the last bit of the fp32 quotient."""
    need_gpu()
    w = _near_half_weights(bits, sdt, seed=bits)
    ratios = oracle.MSE_RATIOS if clip == "mse" else oracle.RTN_RATIOS
    qo, so = oracle.quantize(w, bits, 64, OD[sdt], ratios, w_dtype=oracle.F32)
    wd = to_dev(w, "f32")
    q, s = lmh.quantize(wd, bits, 64, TD[sdt], clip)
    assert np.array_equal(bits16(s), so)
    assert np.array_equal(q.cpu().numpy(), qo), f"codes differ at {np.argwhere(q.cpu().numpy() != qo)[:5]}"
    got = lmh.quantize_pack(wd, bits, 64, TD[sdt], clip).cpu().numpy()
    assert np.array_equal(got, oracle.pack(qo, so, bits, 64))
