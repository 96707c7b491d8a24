"""Seeded synthetic inputs for the LM-head workloads.

This module only draws random numbers and stores them in the input dtypes; it
holds none of the quantized-logits arithmetic.  Both the oracle-side tests and
the GPU-side tests/benchmark take their inputs from here, so the two sides see
the same bytes.

Every array is drawn from numpy ``Generator(PCG64(SeedSequence([wid, stream,
...])))`` where ``wid`` identifies the workload and ``stream`` the purpose
(0 weight normals, 1 outlier mask, 2 outlier values, 3 activations, 4 decode
states).  Weights are drawn in row chunks of 8192, so any row range can be
regenerated without drawing the rest.

The workloads follow the shapes the pages measure (vLLM PR #48870 perf table:
151936x1024 W4-g64 and W8-g128, 50304x512 W4-g64; its review comment: the
151936x2048 tied head with an int8 per-row weight; page "radiance_lmhead_int4.py":
a 248064x5120 head in int4 g128 with bf16 scales and the MSE clip search).  The
value distributions are synthetic stand-ins: no trained weights or captured
decode states exist here.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

CHUNK_ROWS = 8192

S_W, S_MASK, S_OUTLIER, S_X, S_STATE = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed id
    V: int
    K: int
    bits: int
    group: int
    scale_dtype: str         # "f16" | "bf16"
    clip: str                # "rtn" | "mse"
    x_dtype: str             # "f16" | "bf16"
    w_dtype: str             # storage type of the unquantized weight: "f32" | "f16" | "bf16"
    w_std: float
    zero_tail_rows: int      # all-zero padding rows at the end of the vocab
    outlier: str = "none"    # "none" | "x8" | "t3"
    outlier_p: float = 0.0
    Ms: Tuple[int, ...] = (1,)
    note: str = ""


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_w4g64_50304x512", 11, 50304, 512, 4, 64, "f16", "rtn", "f16", "f32",
                 0.02, 64, Ms=(1,),
                 note="tiny head, CPU-seconds scale; last 64 rows zero (vocab padding)"),
        Workload("w4g64_151936x1024", 12, 151936, 1024, 4, 64, "f16", "rtn", "f16", "f32",
                 0.02, 0, "x8", 0.01, Ms=(1, 32, 256),
                 note="int4 g64 RTN; 1% of entries are x8 outliers"),
        Workload("w8g128_151936x1024", 13, 151936, 1024, 8, 128, "f16", "rtn", "f16", "f32",
                 0.02, 64, Ms=(1, 32, 256),
                 note="int8 g128 RTN; tiny-head distribution (last 64 rows zero); fp16 GEMV control"),
        Workload("w8row_151936x2048", 14, 151936, 2048, 8, 2048, "f16", "rtn", "f16", "f16",
                 0.015, 0, Ms=(1,),
                 note="int8 per-row scale quantized from the fp16 weight; fp16 GEMV control; "
                      "decode-state agreement"),
        Workload("w4g128mse_248064x5120", 15, 248064, 5120, 4, 128, "bf16", "mse", "bf16", "bf16",
                 0.01, 256, "t3", 0.005, Ms=(1, 2, 5, 16),
                 note="int4 g128 bf16 scales by MSE clip search; 0.5% heavy-tailed entries; "
                      "last 256 rows zero"),
    ]
}

HEADLINE = "w4g64_151936x1024"


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16) via torch's CPU conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact: the pattern is the top half of the float)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _master_chunk(w: Workload, c: int) -> np.ndarray:
    """float32 master values of rows [c*CHUNK_ROWS, ...) before any 16-bit storage rounding."""
    r0 = c * CHUNK_ROWS
    rows = min(CHUNK_ROWS, w.V - r0)
    a = _rng(w.wid, S_W, c).standard_normal((rows, w.K), dtype=np.float32)
    a *= np.float32(w.w_std)
    live = rows
    tail0 = w.V - w.zero_tail_rows
    if r0 + rows > tail0:
        live = max(0, tail0 - r0)
    if w.outlier != "none" and live > 0:
        mask = _rng(w.wid, S_MASK, c).random((live, w.K), dtype=np.float32) < np.float32(w.outlier_p)
        if w.outlier == "x8":
            a[:live][mask] *= np.float32(8.0)
        elif w.outlier == "t3":
            n = int(mask.sum())
            a[:live][mask] = (np.float32(w.w_std) *
                              _rng(w.wid, S_OUTLIER, c).standard_t(3, size=n).astype(np.float32))
    a[live:] = 0.0
    return a


def weight(w: Workload, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    """Rows [r0, r1) of the unquantized weight in its storage dtype.

    f32 -> float32 array; f16 -> float16 array; bf16 -> uint16 bit patterns."""
    r1 = w.V if r1 is None else r1
    out = None
    parts = []
    for c in range(r0 // CHUNK_ROWS, (r1 - 1) // CHUNK_ROWS + 1):
        a = _master_chunk(w, c)
        lo = max(r0, c * CHUNK_ROWS) - c * CHUNK_ROWS
        hi = min(r1, c * CHUNK_ROWS + a.shape[0]) - c * CHUNK_ROWS
        a = a[lo:hi]
        if w.w_dtype == "f16":
            a = a.astype(np.float16)
        elif w.w_dtype == "bf16":
            a = to_bf16_bits(a)
        parts.append(a)
    out = np.concatenate(parts, axis=0) if len(parts) > 1 else parts[0]
    return np.ascontiguousarray(out)


def weight_rows(w: Workload, rows) -> np.ndarray:
    """Arbitrary (sorted or not) row indices of the weight, in its storage dtype."""
    rows = np.asarray(rows, dtype=np.int64)
    out = None
    for c in np.unique(rows // CHUNK_ROWS):
        blk = weight(w, int(c) * CHUNK_ROWS, min(w.V, (int(c) + 1) * CHUNK_ROWS))
        sel = np.nonzero(rows // CHUNK_ROWS == c)[0]
        if out is None:
            out = np.empty((len(rows), w.K), dtype=blk.dtype)
        out[sel] = blk[rows[sel] - int(c) * CHUNK_ROWS]
    return out


def activations(w: Workload, M: int, seed: int = 0) -> np.ndarray:
    """x [M, K] ~ N(0, 1) in the activation dtype (float16 array or bf16 bit patterns)."""
    a = _rng(w.wid, S_X, M, seed).standard_normal((M, w.K), dtype=np.float32)
    if w.x_dtype == "f16":
        return a.astype(np.float16)
    return to_bf16_bits(a)


def decode_states(w: Workload, start: int, count: int) -> np.ndarray:
    """Decode states i = start .. start+count-1, each x_i ~ N(0, 1) drawn from its own
    seed, so any batch of them can be regenerated on its own."""
    a = np.stack([_rng(w.wid, S_STATE, i).standard_normal(w.K, dtype=np.float32)
                  for i in range(start, start + count)])
    if w.x_dtype == "f16":
        return a.astype(np.float16)
    return to_bf16_bits(a)


def random_weight(shape, std: float, seed: int, zero_rows=(), dtype=np.float32) -> np.ndarray:
    """Small ad-hoc weights for edge-case tests (ragged shapes, extreme values)."""
    a = _rng(99, seed, *shape).standard_normal(shape, dtype=np.float32) * np.float32(std)
    for r in zero_rows:
        a[r] = 0.0
    return a.astype(dtype)


def random_x(M: int, K: int, seed: int, dtype: str = "f16", std: float = 1.0) -> np.ndarray:
    a = _rng(98, seed, M, K).standard_normal((M, K), dtype=np.float32) * np.float32(std)
    return a.astype(np.float16) if dtype == "f16" else to_bf16_bits(a)
