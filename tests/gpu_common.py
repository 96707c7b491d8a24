"""Helpers for the GPU parity tests (imported by tests/test_gpu_*.py).

Acceptance for logits (fp32 output vs the fp64 oracle):
  * whole call:  max |y - y_or| <= 1e-3 * max |y_or|
  * per row m:   max_v |y - y_or| <= 5e-4 * max_v |y_or[m, :]|   (the pages' per-row relative difference, normalised by that row's largest oracle logit)
  * argmax identical on rows whose oracle top1 - top2 margin exceeds 1e-3
  * per element: |y - y_or| <= gamma * sum_k |x q s| with
      gamma = (K + K/G + 16) * 2^-24,
    the standard bound for fp32 sums of exact products; every lossy step
    (e.g. a 16-bit dequantized weight, 2^-9 relative) would exceed it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth

gpu = pytest.mark.gpu
DEV = "cuda:0"

TD = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
OD = {"f16": oracle.F16, "bf16": oracle.BF16, "f32": oracle.F32}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def to_dev(a: np.ndarray, dt: str) -> torch.Tensor:
    """numpy array (float32 / float16 / uint16 bf16 bits) -> device tensor of dtype dt."""
    if dt == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dt == "f16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(DEV)


def bits16(t: torch.Tensor) -> np.ndarray:
    """16-bit device tensor -> uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def abs_terms(x: np.ndarray, xdt: str, q: np.ndarray, s: np.ndarray, sdt: int, G: int, rows=None):
    """sum_k |x q s| per (m, row) via the oracle on |x| and |q|."""
    if xdt == "bf16":
        xa = x & np.uint16(0x7FFF)
    else:
        xa = np.abs(x)
    return oracle.logits(xa, np.abs(q.astype(np.int16)).astype(np.int8), s, sdt, G, rows=rows,
                         x_dtype=OD[xdt])


def check_logits(y: np.ndarray, y_or: np.ndarray, y_abs: np.ndarray, K: int, G: int,
                 what: str = "", bias: np.ndarray | None = None) -> float:
    """Assert the acceptance bars; return the observed max per-row relative error."""
    y = y.astype(np.float64)
    d = np.abs(y - y_or)
    gmax = np.abs(y_or).max()
    assert d.max() <= 1e-3 * gmax + 1e-30, f"{what}: whole-call error {d.max()} vs max|y| {gmax}"
    rmax = np.abs(y_or).max(axis=1)
    live = rmax > 0
    rel = np.zeros(len(rmax))
    rel[live] = d[live].max(axis=1) / rmax[live]
    assert (rel <= 5e-4).all(), f"{what}: per-row error {rel.max()}"
    dead = ~live
    if dead.any():
        assert (d[dead] == 0).all(), f"{what}: an all-zero row gave non-zero logits"
    gamma = (K + K // G + 16) * 2.0**-24
    slack = gamma * y_abs + (np.abs(bias)[None, :] * 2.0**-23 if bias is not None else 0.0)
    bad = d > slack + 1e-30
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements exceed the fp32 summation bound; "
                           f"worst ratio {float((d / (slack + 1e-300)).max()):.3g}")
    # argmax gate
    if y_or.shape[1] > 1:
        srt = np.sort(y_or, axis=1)
        margin = srt[:, -1] - srt[:, -2]
        clear = margin > 1e-3
        assert (np.argmax(y, axis=1)[clear] == np.argmax(y_or, axis=1)[clear]).all(), \
            f"{what}: argmax differs on a row with a clear margin"
    return float(rel.max())
