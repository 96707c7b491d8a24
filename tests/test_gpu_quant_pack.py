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
