"""Pins for the oracle's packed-blob writer and reader.

The blob layout is this library's own (defined byte by byte in include/lmhead.h).
It is pinned by bytes worked out by hand from that definition
(tests/golden/pack_examples.json), by the round-trip identity on ragged shapes,
by the padding rule, and by the size formula.
"""
import json
import os

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_examples.json")))


@pytest.mark.parametrize("kind", ["int4", "int8"])
def test_hand_derived_bytes(orc, kind):
    ex = GOLD[kind]
    V, K, bits, G = ex["V"], ex["K"], ex["bits"], ex["group"]
    k = np.arange(K)
    q = ((k % 16) - 8 if kind == "int4" else k - 32).astype(np.int8)[None, :]
    s = np.array([[int(h, 16) for h in ex["scales_hex"]]], dtype=np.uint16)
    blob = orc.pack(q, s, bits, G)
    assert blob.size == ex["total_bytes"]
    for e in ex["expect"]:
        want = bytes.fromhex(e["hex"])
        got = blob[e["offset"]:e["offset"] + len(want)].tobytes()
        assert got == want, (e["offset"], e["why"], got.hex())


@pytest.mark.parametrize("bits,K,G", [(4, 128, 32), (4, 512, 64), (4, 384, 128), (4, 256, 256),
                                      (8, 64, 32), (8, 192, 64), (8, 512, 512)])
@pytest.mark.parametrize("V", [1, 63, 64, 65, 200])
def test_roundtrip_ragged(orc, bits, K, G, V):
    rng = np.random.default_rng(V * 1000 + K + bits)
    lo, hi = (-8, 7) if bits == 4 else (-128, 127)
    q = rng.integers(lo, hi + 1, size=(V, K)).astype(np.int8)
    s = rng.integers(0, 0x7C00, size=(V, K // G)).astype(np.uint16)
    blob = orc.pack(q, s, bits, G)
    vpad = (V + 63) // 64 * 64
    assert blob.size == vpad * K * bits // 8 + vpad * (K // G) * 2
    q2, s2 = orc.unpack(blob, V, K, bits, G)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


@pytest.mark.parametrize("bits", [4, 8])
def test_padding_rows_are_zero_weights_and_zero_scales(orc, bits):
    V, K, G = 70, 128, 64
    q = np.full((V, K), 3, dtype=np.int8)
    s = np.full((V, K // G), 0x3C00, dtype=np.uint16)
    blob = orc.pack(q, s, bits, G)
    q2, s2 = orc.unpack(blob, 128, K, bits, G)  # read the padded rows as if they were real
    assert (q2[:V] == 3).all() and (q2[V:] == 0).all()
    assert (s2[:V] == 0x3C00).all() and (s2[V:] == 0).all()


@pytest.mark.parametrize("bits,K,G", [(4, 100, 50), (4, 192, 64), (8, 96, 32), (4, 128, 48)])
def test_unsupported_shapes_rejected(orc, bits, K, G):
    q = np.zeros((4, K), dtype=np.int8)
    s = np.zeros((4, max(1, K // G)), dtype=np.uint16)
    with pytest.raises(ValueError):
        orc.pack(q, s, bits, G)


def test_every_element_has_its_own_position(orc):
    """Packing a one-hot q (one element at level 1, the rest 0) changes exactly one
    nibble/byte of the blob, and a different one for every element."""
    for bits, K in [(4, 256), (8, 128)]:
        V, G = 3, 64
        base = orc.pack(np.zeros((V, K), np.int8), np.zeros((V, K // G), np.uint16), bits, G)
        seen = set()
        for v in range(V):
            for k in range(K):
                q = np.zeros((V, K), np.int8)
                q[v, k] = 1
                d = np.nonzero(orc.pack(q, np.zeros((V, K // G), np.uint16), bits, G) != base)[0]
                assert d.size == 1
                key = (int(d[0]), int(orc.pack(q, np.zeros((V, K // G), np.uint16), bits, G)[d[0]]
                                      ^ base[d[0]]))
                assert key not in seen
                seen.add(key)
