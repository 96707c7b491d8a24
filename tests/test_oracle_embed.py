"""Pins for the oracle's embedding gather (oracle.embed), each against something
other than its own formula:
  * the logits oracle on one-hot inputs: x = e_k gives y[v] = q[v,k] s[v,k/G]
    exactly, so the identity matrix as x yields the whole dequantized table
    (the logits oracle is itself pinned by exact rational brute force);
  * 16-bit outputs against numpy's float16 and torch's bfloat16 conversions
    (independent round-to-nearest-even implementations);
  * ids outside the table give zero rows; an empty id list gives no rows."""
import numpy as np
import pytest
import torch

import oracle


def _table(V, K, G, sdt, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-128, 128, size=(V, K)).astype(np.int8)
    if sdt == oracle.F16:
        s = rng.integers(0x0001, 0x7800, size=(V, K // G)).astype(np.uint16)
    else:
        s = rng.integers(0x2000, 0x5000, size=(V, K // G)).astype(np.uint16)
    return q, s


@pytest.mark.parametrize("sdt", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("G", [8, 32, 64])
def test_embed_equals_one_hot_logits(sdt, G):
    V, K = 37, 64
    q, s = _table(V, K, G, sdt, seed=G)
    eye = np.eye(K, dtype=np.float16)
    table = oracle.logits(eye, q, s, sdt, G).T          # [V, K]: y(e_k)[v] = q[v,k] s[v,k/G]
    ids = np.arange(V)
    got = oracle.embed(q, s, sdt, G, ids, oracle.F32)
    assert np.array_equal(got.astype(np.float64), table)
    perm = np.random.default_rng(1).permutation(V)[:11]
    assert np.array_equal(oracle.embed(q, s, sdt, G, perm, oracle.F32).astype(np.float64),
                          table[perm])


@pytest.mark.parametrize("sdt", [oracle.F16, oracle.BF16])
def test_embed_16bit_outputs_round_to_nearest_even(sdt):
    V, K, G = 29, 128, 32
    q, s = _table(V, K, G, sdt, seed=7)
    ids = np.arange(V)[::-1].copy()
    exact = oracle.embed(q, s, sdt, G, ids, oracle.F32)
    h = oracle.embed(q, s, sdt, G, ids, oracle.F16)
    with np.errstate(over="ignore"):          # large products overflow to inf in fp16
        ref16 = exact.astype(np.float16)
    assert np.isinf(ref16).any() or sdt == oracle.BF16
    assert np.array_equal(h, ref16.view(np.uint16))
    b = oracle.embed(q, s, sdt, G, ids, oracle.BF16)
    tb = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, tb)


def test_embed_out_of_range_ids_and_empty():
    q, s = _table(10, 64, 32, oracle.F16, seed=3)
    out = oracle.embed(q, s, oracle.F16, 32, [-1, 10, 2**31 - 1, 3], oracle.F32)
    assert (out[:3] == 0).all() and np.array_equal(out[3], oracle.embed(q, s, oracle.F16, 32, [3])[0])
    assert oracle.embed(q, s, oracle.F16, 32, [], oracle.F16).shape == (0, 64)
