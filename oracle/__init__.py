"""Oracle for the weight-only-quantized LM-head path: a plain, slow, fp64 CPU
implementation written from the pages, used to check the GPU library.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the ``weight_only_quantized_lmhead_amd`` package and its HIP library) never
imports, links or calls anything here, and this package imports nothing from it.

The arithmetic lives in ``lmh_oracle.c`` (plain C, built with
``-O2 -ffp-contract=off``); this module only builds it, loads it with ctypes and
marshals numpy arrays.  Every function states which passage it follows:

* quantize   -- page "radiance_lmhead_int4.py", docstring "How" paragraph
                (one bf16 scale per group; codes -8..7; the clip ratio that
                gives the smallest squared error among five, from 1.0 down to
                0.8; the scale is rounded to bf16 before the codes are
                picked), module constants (CLIP_RATIOS, QMAX, ZP_BIAS) and
                ``quantize_int4_rows``;  int8 per the W8-g128 rows of the table
                on vLLM PR #48870 and the int8 per-row head of its review comment.
* logits     -- vLLM PR #48870, Purpose: a fused dequant-GEMM gives the logits of
                dequantize-then-F.linear without forming the dense weight.
* dense      -- vLLM PR #48870, review comment point 1 (the fp16 logits GEMV).
* topk_rescore -- vLLM PR #48870, review comment point 2 (the K largest
                quantized logits of a row are replaced by exact dot products
                with the unquantized weight rows they index).

Parity pins for each function are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lmh_oracle.c")
_LIB = os.path.join(_HERE, "liblmh_oracle.so")

F32, F16, BF16 = 0, 1, 2
RTN_RATIOS = (1.0,)
MSE_RATIOS = (1.0, 0.95, 0.9, 0.85, 0.8)

_lib: Optional[ctypes.CDLL] = None


def build(force: bool = True) -> str:
    """Compile lmh_oracle.c into liblmh_oracle.so (gcc, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.orc_f32_to_f16.restype = ctypes.c_uint16
        lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
        lib.orc_f32_to_bf16.restype = ctypes.c_uint16
        lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.orc_f16_to_f32.restype = ctypes.c_float
        lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f32.restype = ctypes.c_float
        lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        for name in ("orc_f32_to_f16_array", "orc_f32_to_bf16_array",
                     "orc_f16_to_f32_array", "orc_bf16_to_f32_array"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [vp, i64, vp]
        lib.orc_quantize.restype = i32
        lib.orc_quantize.argtypes = [vp, i32, i64, i64, i32, i64, i32, vp, i32, vp, vp, vp]
        lib.orc_packed_bytes.restype = i64
        lib.orc_packed_bytes.argtypes = [i64, i64, i32, i64]
        lib.orc_pack.restype = i32
        lib.orc_pack.argtypes = [vp, vp, i64, i64, i32, i64, vp]
        lib.orc_unpack.restype = i32
        lib.orc_unpack.argtypes = [vp, i64, i64, i32, i64, vp, vp]
        lib.orc_logits.restype = i32
        lib.orc_logits.argtypes = [vp, i32, i64, vp, vp, i32, i64, i64, i64, vp, vp, i64, vp]
        lib.orc_embed.restype = i32
        lib.orc_embed.argtypes = [vp, vp, i32, i64, i64, i64, vp, i64, i32, vp]
        lib.orc_dense_logits.restype = i32
        lib.orc_dense_logits.argtypes = [vp, i32, i64, vp, i32, i64, i64, vp, i64, vp]
        lib.orc_topk.restype = i32
        lib.orc_topk.argtypes = [vp, i64, i32, vp]
        lib.orc_topk_rescore.restype = i32
        lib.orc_topk_rescore.argtypes = [vp, i64, i64, i64, i32, vp, i32, vp, i32, i64, vp, vp, vp]
        lib.orc_quantize_asym.restype = i32
        lib.orc_quantize_asym.argtypes = [vp, i32, i64, i64, i32, i64, i32, vp, vp, vp]
        lib.orc_packed_bytes_zp.restype = i64
        lib.orc_packed_bytes_zp.argtypes = [i64, i64, i32, i64]
        lib.orc_pack_zp.restype = i32
        lib.orc_pack_zp.argtypes = [vp, vp, vp, i64, i64, i32, i64, vp]
        lib.orc_unpack_zp.restype = i32
        lib.orc_unpack_zp.argtypes = [vp, i64, i64, i32, i64, vp, vp, vp]
        lib.orc_logits_zp.restype = i32
        lib.orc_logits_zp.argtypes = [vp, i32, i64, vp, vp, vp, i32, i64, i64, i64, vp, vp, i64, vp]
        lib.orc_embed_zp.restype = i32
        lib.orc_embed_zp.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp, i64, i32, vp]
        lib.orc_algorithmic_bytes.restype = i64
        lib.orc_algorithmic_bytes.argtypes = [i64, i64, i64, i32, i64]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _dtype_code(a: np.ndarray, declared: Optional[int]) -> int:
    if declared is not None:
        return declared
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    raise ValueError("uint16 arrays are ambiguous: pass dtype=F16 or BF16 explicitly")


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments (rc={rc})")


# ---- 16-bit codecs (IEEE-754 binary16 / bfloat16, nearest-even) -------------

def f32_to_f16_bits(x: float) -> int:
    return int(_load().orc_f32_to_f16(float(np.float32(x))))


def f32_to_bf16_bits(x: float) -> int:
    return int(_load().orc_f32_to_bf16(float(np.float32(x))))


def f16_bits_to_f32(h: int) -> float:
    return float(_load().orc_f16_to_f32(int(h)))


def bf16_bits_to_f32(h: int) -> float:
    return float(_load().orc_bf16_to_f32(int(h)))


def encode16(a: np.ndarray, dtype: int) -> np.ndarray:
    """float32 array -> 16-bit patterns (F16 or BF16) via the oracle's encoder."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    fn = _load().orc_f32_to_f16_array if dtype == F16 else _load().orc_f32_to_bf16_array
    fn(_ptr(a), a.size, _ptr(out))
    return out


def widen16(bits: np.ndarray, dtype: int) -> np.ndarray:
    """16-bit patterns -> float32 values via the oracle's decoder (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    fn = _load().orc_f16_to_f32_array if dtype == F16 else _load().orc_bf16_to_f32_array
    fn(_ptr(b), b.size, _ptr(out))
    return out


# ---- quantizer ----------------------------------------------------------------

def default_threads() -> int:
    """Host threads the oracle's row-parallel calls use: the cores this process
    may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _row_ranges(n: int, threads: Optional[int]):
    """Contiguous row ranges for the worker threads (none shorter than 64 rows)."""
    t = default_threads() if threads is None else max(1, int(threads))
    t = max(1, min(t, n // 64 if n >= 64 else 1))
    edges = [n * i // t for i in range(t + 1)]
    return [(edges[i], edges[i + 1]) for i in range(t) if edges[i + 1] > edges[i]]


def _parallel(fn, ranges):
    """Run fn(lo, hi) for every range on its own thread.  The C calls release
    the GIL (ctypes), so the ranges run side by side; every row's arithmetic is
    the same as in one call over all rows."""
    if len(ranges) <= 1:
        return [fn(lo, hi) for lo, hi in ranges]
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(max_workers=len(ranges)) as ex:
        return list(ex.map(lambda r: fn(*r), ranges))


def quantize(w: np.ndarray, bits: int, group: int, scale_dtype: int,
             ratios: Sequence[float] = RTN_RATIOS, w_dtype: Optional[int] = None,
             return_pick: bool = False, threads: Optional[int] = None):
    """(q int8 [V,K], s uint16 [V,K/G]) per the page's quantize_int4_rows, generalised
    to int8 (qmax 127, qmin -128) and fp16/bf16 scales; readings R1-R4 and R7 of the list at the top of lmh_oracle.c.
    Rows are quantized independently, so `threads` (default: the host's cores,
    at most 16) only splits the rows into ranges run side by side."""
    w = np.ascontiguousarray(w)
    V, K = w.shape
    wd = _dtype_code(w, w_dtype)
    if group <= 0 or K % group != 0:
        raise ValueError("oracle quantize: bad arguments (K not a multiple of G)")
    NG = K // group
    q = np.empty((V, K), dtype=np.int8)
    s = np.empty((V, NG), dtype=np.uint16)
    pick = np.empty((V, NG), dtype=np.int8)
    r = np.ascontiguousarray(np.array(ratios, dtype=np.float64))
    isz = w.itemsize

    def run(lo, hi):
        return _load().orc_quantize(_ptr(w) + lo * K * isz, wd, hi - lo, K, bits, group,
                                    scale_dtype, _ptr(r), len(r), _ptr(q) + lo * K,
                                    _ptr(s) + lo * NG * 2, _ptr(pick) + lo * NG)

    rcs = _parallel(run, _row_ranges(V, threads)) if V else [
        _load().orc_quantize(_ptr(w), wd, 0, K, bits, group, scale_dtype, _ptr(r), len(r),
                             _ptr(q), _ptr(s), _ptr(pick))]
    for rc in rcs:
        _check(rc, "quantize")
    return (q, s, pick) if return_pick else (q, s)


# ---- packed blob ---------------------------------------------------------------

def packed_bytes(V: int, K: int, bits: int, group: int) -> int:
    n = int(_load().orc_packed_bytes(V, K, bits, group))
    if n < 0:
        raise ValueError("unsupported packed shape")
    return n


def pack(q: np.ndarray, s: np.ndarray, bits: int, group: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    V, K = q.shape
    out = np.empty(packed_bytes(V, K, bits, group), dtype=np.uint8)
    _check(_load().orc_pack(_ptr(q), _ptr(s), V, K, bits, group, _ptr(out)), "pack")
    return out


def unpack(blob: np.ndarray, V: int, K: int, bits: int, group: int):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    q = np.empty((V, K), dtype=np.int8)
    s = np.empty((V, K // group), dtype=np.uint16)
    _check(_load().orc_unpack(_ptr(blob), V, K, bits, group, _ptr(q), _ptr(s)), "unpack")
    return q, s


# ---- logits --------------------------------------------------------------------

def _rows_arg(rows, V):
    if rows is None:
        return None, V, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, len(r), _ptr(r)


def logits(x: np.ndarray, q: np.ndarray, s: np.ndarray, scale_dtype: int, group: int,
           bias: Optional[np.ndarray] = None, rows=None, x_dtype: Optional[int] = None,
           threads: Optional[int] = None) -> np.ndarray:
    """fp64 y[M, rows] = x * dequant(q, s)^T (+ bias), exact products, fp64 sums.
    Each output element is one sequential sum over k; `threads` (default: the
    host's cores, at most 16) only splits the rows into ranges run side by side."""
    x = np.ascontiguousarray(x)
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    M, K = x.shape
    V = q.shape[0]
    r, n, rp = _rows_arg(rows, V)
    bp = 0
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        bp = _ptr(bias)
    xd = _dtype_code(x, x_dtype)
    if r is None:
        r = np.arange(V, dtype=np.int64)

    def run(lo, hi):
        rr = np.ascontiguousarray(r[lo:hi])
        y = np.empty((M, hi - lo), dtype=np.float64)
        rc = _load().orc_logits(_ptr(x), xd, M, _ptr(q), _ptr(s), scale_dtype, V, K, group,
                                bp or None, _ptr(rr) if hi > lo else None, hi - lo, _ptr(y))
        _check(rc, "logits")
        return y

    parts = _parallel(run, _row_ranges(n, threads)) if n else []
    if not parts:
        return np.empty((M, 0), dtype=np.float64)
    return parts[0] if len(parts) == 1 else np.concatenate(parts, axis=1)


def embed(q: np.ndarray, s: np.ndarray, scale_dtype: int, group: int, ids,
          out_dtype: int = F32) -> np.ndarray:
    """Embedding rows out[t, k] = q[id,k] * s[id, k/G] rounded once to out_dtype
    (float32 array, or uint16 bit patterns for F16/BF16); ids outside [0, V)
    give zero rows."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).ravel())
    V, K = q.shape
    out = np.empty((len(ids), K), dtype=np.float32 if out_dtype == F32 else np.uint16)
    rc = _load().orc_embed(_ptr(q), _ptr(s), scale_dtype, V, K, group, _ptr(ids) if len(ids) else None,
                           len(ids), out_dtype, _ptr(out) if out.size else None)
    if len(ids):
        _check(rc, "embed")
    return out


def dense_logits(x: np.ndarray, w: np.ndarray, rows=None, x_dtype: Optional[int] = None,
                 w_dtype: Optional[int] = None) -> np.ndarray:
    """fp64 y[M, rows] = x * W^T with x, W widened exactly."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    M, K = x.shape
    V = w.shape[0]
    r, n, rp = _rows_arg(rows, V)
    y = np.empty((M, n), dtype=np.float64)
    rc = _load().orc_dense_logits(_ptr(x), _dtype_code(x, x_dtype), M, _ptr(w),
                                  _dtype_code(w, w_dtype), V, K, rp or None, n, _ptr(y))
    _check(rc, "dense_logits")
    return y


# ---- asymmetric (zero-point) form ---------------------------------------------

def quantize_asym(w: np.ndarray, bits: int, group: int, scale_dtype: int,
                  w_dtype: Optional[int] = None):
    """(n uint8 [V,K], s uint16 [V,K/G], z uint8 [V,K/G]) with w ~ (n - z) * s:
    per-group min/max round to nearest with zero exactly representable (reading R21 of lmh_oracle.c)."""
    w = np.ascontiguousarray(w)
    V, K = w.shape
    n = np.empty((V, K), dtype=np.uint8)
    s = np.empty((V, K // group), dtype=np.uint16)
    z = np.empty((V, K // group), dtype=np.uint8)
    rc = _load().orc_quantize_asym(_ptr(w), _dtype_code(w, w_dtype), V, K, bits, group,
                                   scale_dtype, _ptr(n), _ptr(s), _ptr(z))
    _check(rc, "quantize_asym")
    return n, s, z


def packed_bytes_zp(V: int, K: int, bits: int, group: int) -> int:
    n = int(_load().orc_packed_bytes_zp(V, K, bits, group))
    if n < 0:
        raise ValueError("unsupported packed shape")
    return n


def pack_zp(n: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int, group: int) -> np.ndarray:
    n = np.ascontiguousarray(n, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    z = np.ascontiguousarray(z, dtype=np.uint8)
    V, K = n.shape
    out = np.empty(packed_bytes_zp(V, K, bits, group), dtype=np.uint8)
    _check(_load().orc_pack_zp(_ptr(n), _ptr(s), _ptr(z), V, K, bits, group, _ptr(out)), "pack_zp")
    return out


def unpack_zp(blob: np.ndarray, V: int, K: int, bits: int, group: int):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    n = np.empty((V, K), dtype=np.uint8)
    s = np.empty((V, K // group), dtype=np.uint16)
    z = np.empty((V, K // group), dtype=np.uint8)
    _check(_load().orc_unpack_zp(_ptr(blob), V, K, bits, group, _ptr(n), _ptr(s), _ptr(z)),
           "unpack_zp")
    return n, s, z


def logits_zp(x: np.ndarray, n: np.ndarray, s: np.ndarray, z: np.ndarray, scale_dtype: int,
              group: int, bias: Optional[np.ndarray] = None, rows=None,
              x_dtype: Optional[int] = None) -> np.ndarray:
    """fp64 y[M, rows] = x * ((n - z) * s)^T (+ bias), exact products, fp64 sums."""
    x = np.ascontiguousarray(x)
    n = np.ascontiguousarray(n, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    z = np.ascontiguousarray(z, dtype=np.uint8)
    M, K = x.shape
    V = n.shape[0]
    r, nr, rp = _rows_arg(rows, V)
    y = np.empty((M, nr), dtype=np.float64)
    bp = 0
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        bp = _ptr(bias)
    rc = _load().orc_logits_zp(_ptr(x), _dtype_code(x, x_dtype), M, _ptr(n), _ptr(s), _ptr(z),
                               scale_dtype, V, K, group, bp or None, rp or None, nr, _ptr(y))
    _check(rc, "logits_zp")
    return y


def embed_zp(n: np.ndarray, s: np.ndarray, z: np.ndarray, scale_dtype: int, group: int, ids,
             out_dtype: int = F32) -> np.ndarray:
    """Embedding rows (n[id,k] - z[id,g]) * s[id,g] rounded once to out_dtype;
    ids outside [0, V) give zero rows."""
    n = np.ascontiguousarray(n, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    z = np.ascontiguousarray(z, dtype=np.uint8)
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).ravel())
    V, K = n.shape
    out = np.empty((len(ids), K), dtype=np.float32 if out_dtype == F32 else np.uint16)
    if len(ids):
        rc = _load().orc_embed_zp(_ptr(n), _ptr(s), _ptr(z), scale_dtype, V, K, group, _ptr(ids),
                                  len(ids), out_dtype, _ptr(out))
        _check(rc, "embed_zp")
    return out


# ---- top-K and rescoring -------------------------------------------------------

def topk(y: np.ndarray, k: int) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    idx = np.empty(k, dtype=np.int64)
    _check(_load().orc_topk(_ptr(y), len(y), k, _ptr(idx)), "topk")
    return idx


def topk_rescore(y: np.ndarray, k: int, x: np.ndarray, w: np.ndarray,
                 x_dtype: Optional[int] = None, w_dtype: Optional[int] = None):
    """(idx [M,k], exact values [M,k] fp64, top1 [M]) from logits y [M, V] (fp32)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    M, V = y.shape
    K = x.shape[1]
    idx = np.empty((M, k), dtype=np.int64)
    val = np.empty((M, k), dtype=np.float64)
    top1 = np.empty(M, dtype=np.int64)
    rc = _load().orc_topk_rescore(_ptr(y), V, M, V, k, _ptr(x), _dtype_code(x, x_dtype), _ptr(w),
                                  _dtype_code(w, w_dtype), K, _ptr(idx), _ptr(val), _ptr(top1))
    _check(rc, "topk_rescore")
    return idx, val, top1


def algorithmic_bytes(M: int, V: int, K: int, bits: int, group: int) -> int:
    """Bytes one logits call must move: packed weight + scales + x (16-bit) + fp32 y."""
    return int(_load().orc_algorithmic_bytes(M, V, K, bits, group))
