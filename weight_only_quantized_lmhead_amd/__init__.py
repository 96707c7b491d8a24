"""Weight-only-quantized LM-head logits for AMD MI355X (gfx950).

A thin ctypes binding over ``liblmhead.so`` (C ABI in ``include/lmhead.h``):
argument marshalling only.  Every step of the path -- quantize, pack, logits,
top-K rescoring -- runs in the library's HIP kernels; torch supplies device
memory and the current stream.  There is no CPU fallback: if the library is
missing or fails to load, importing the binding's functions raises.

    import weight_only_quantized_lmhead_amd as lmh
    packed = lmh.quantize_pack(w, bits=4, group=64, scale_dtype=torch.float16, clip="rtn")
    y = lmh.logits(x, packed, V, K, bits=4, group=64, scale_dtype=torch.float16)
    idx, val, top1 = lmh.topk_rescore(x, w_ref, y, topk=8)

Zero-point (asymmetric) heads: pass ``bits | lmh.ZP`` wherever a ``bits``
argument is taken (quantize_pack, embed, logits, logits_topk, packed_bytes);
``quantize_zp`` / ``pack_zp`` are the codes-mode quantizer and packer.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblmhead.so")

LMH_OK = 0
_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_CLIP = {"rtn": 0, "mse": 1}
PATH_AUTO, PATH_GEMV, PATH_MFMA, PATH_MFMA_LDS, PATH_MFMA_XRES, PATH_MFMA_SPLITK = 0, 1, 2, 3, 4, 5
ZP = 0x10  # LMH_ZP: OR'd into `bits`, selects the zero-point form

_lib: Optional[ctypes.CDLL] = None


class LmheadError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib().lmhead_status_string(status).decode()}")


def lib() -> ctypes.CDLL:
    """Load liblmhead.so (built in-tree by ``python -m weight_only_quantized_lmhead_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m weight_only_quantized_lmhead_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        sig = {
            "lmhead_status_string": (ctypes.c_char_p, [i32]),
            "lmhead_abi_version": (i32, []),
            "lmhead_packed_bytes": (sz, [i64, i64, i32, i64]),
            "lmhead_quantize": (i32, [vp, i32, i64, i64, i32, i64, i32, i32, vp, vp, vp]),
            "lmhead_pack": (i32, [vp, vp, i64, i64, i32, i64, vp, vp]),
            "lmhead_quantize_zp": (i32, [vp, i32, i64, i64, i32, i64, i32, vp, vp, vp, vp]),
            "lmhead_pack_zp": (i32, [vp, vp, vp, i64, i64, i32, i64, vp, vp]),
            "lmhead_quantize_pack": (i32, [vp, i32, i64, i64, i64, i32, i64, i32, i32, i64, i64,
                                           vp, vp]),
            "lmhead_embed": (i32, [vp, i64, vp, i64, i64, i32, i64, i32, vp, i32, i64, vp]),
            "lmhead_logits_workspace_bytes": (sz, [i64, i64, i32]),
            "lmhead_logits": (i32, [vp, i32, i64, vp, i64, i64, i32, i64, i32, vp, vp, i64, vp,
                                    sz, vp]),
            "lmhead_logits_path": (i32, [vp, i32, i64, vp, i64, i64, i32, i64, i32, vp, vp, i64,
                                         vp, sz, i32, vp]),
            "lmhead_logits_typed": (i32, [vp, i32, i64, vp, i64, i64, i32, i64, i32, vp, vp, i32, i64,
                                          vp, sz, i32, vp]),
            "lmhead_logits_auto_path": (i32, [i64, i64, i32, i64, vp]),
            "lmhead_logits_auto_path_x": (i32, [i64, i64, i32, i64, i32, vp]),
            "lmhead_dense_logits": (i32, [vp, i32, i64, vp, i32, i64, i64, vp, i64, vp]),
            "lmhead_topk_workspace_bytes": (sz, [i64, i64, i32]),
            "lmhead_topk_rescore": (i32, [vp, i32, i64, vp, i32, i64, i64, vp, i64, i32, vp, vp,
                                          vp, vp, sz, vp]),
            "lmhead_logits_topk_workspace_bytes": (sz, [i64, i64, i64, i32, i32]),
            "lmhead_logits_topk": (i32, [vp, i32, i64, vp, i64, i64, i32, i64, i32, vp, vp, i32, i32,
                                         vp, i64, vp, vp, vp, vp, sz, vp]),
            "lmhead_stream_read": (i32, [vp, sz, vp, vp]),
            "lmhead_stream_mix": (i32, [vp, sz, vp, sz, vp]),
            "lmhead_mfma_ceiling": (i32, [i64, i32, vp, vp]),
            "lmhead_mfma_ceiling_mfmas": (i64, [i64]),
            "lmhead_logits_topk_noalloc": (i32, [vp, i32, i64, vp, i64, i64, i32, i64, i32, vp, vp,
                                                 i32, i32, vp, i64, vp, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != LMH_OK:
        raise LmheadError(fn, rc)


def _need_cuda(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("lmhead tensors must live on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("lmhead tensors must be contiguous")


def packed_bytes(V: int, K: int, bits: int, group: int) -> int:
    n = lib().lmhead_packed_bytes(V, K, bits, group)
    if n == 0:
        raise ValueError(f"unsupported packed shape V={V} K={K} bits={bits} G={group}")
    return int(n)


def quantize(w: torch.Tensor, bits: int, group: int, scale_dtype: torch.dtype = torch.float16,
             clip: str = "rtn") -> Tuple[torch.Tensor, torch.Tensor]:
    """(q int8 [V,K], s [V,K/G] in scale_dtype) -- lmhead_quantize."""
    _need_cuda(w)
    V, K = w.shape
    q = torch.empty((V, K), dtype=torch.int8, device=w.device)
    s = torch.empty((V, K // group), dtype=scale_dtype, device=w.device)
    _check("lmhead_quantize", lib().lmhead_quantize(
        _ptr(w), _DT[w.dtype], V, K, bits, group, _DT[scale_dtype], _CLIP[clip], _ptr(q), _ptr(s),
        _stream(w)))
    return q, s


def pack(q: torch.Tensor, s: torch.Tensor, bits: int, group: int) -> torch.Tensor:
    """Packed blob (uint8) -- lmhead_pack."""
    _need_cuda(q, s)
    V, K = q.shape
    out = torch.empty(packed_bytes(V, K, bits, group), dtype=torch.uint8, device=q.device)
    _check("lmhead_pack", lib().lmhead_pack(_ptr(q), _ptr(s), V, K, bits, group, _ptr(out),
                                            _stream(q)))
    return out


def quantize_zp(w: torch.Tensor, bits: int, group: int,
                scale_dtype: torch.dtype = torch.float16
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(n uint8 [V,K], s [V,K/G] in scale_dtype, z uint8 [V,K/G]) -- lmhead_quantize_zp."""
    _need_cuda(w)
    V, K = w.shape
    n = torch.empty((V, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((V, K // group), dtype=scale_dtype, device=w.device)
    z = torch.empty((V, K // group), dtype=torch.uint8, device=w.device)
    _check("lmhead_quantize_zp", lib().lmhead_quantize_zp(
        _ptr(w), _DT[w.dtype], V, K, bits, group, _DT[scale_dtype], _ptr(n), _ptr(s), _ptr(z),
        _stream(w)))
    return n, s, z


def pack_zp(n: torch.Tensor, s: torch.Tensor, z: torch.Tensor, bits: int, group: int) -> torch.Tensor:
    """Zero-point packed blob (uint8) -- lmhead_pack_zp."""
    _need_cuda(n, s, z)
    V, K = n.shape
    out = torch.empty(packed_bytes(V, K, bits | ZP, group), dtype=torch.uint8, device=n.device)
    _check("lmhead_pack_zp", lib().lmhead_pack_zp(_ptr(n), _ptr(s), _ptr(z), V, K, bits, group,
                                                  _ptr(out), _stream(n)))
    return out


def quantize_pack(w: torch.Tensor, bits: int, group: int,
                  scale_dtype: torch.dtype = torch.float16, clip: str = "rtn", *,
                  V: Optional[int] = None, row0: int = 0,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed blob straight from the unquantized weight -- lmhead_quantize_pack.

    ``w`` holds rows ``[row0, row0 + w.shape[0])`` of a ``V``-row head (``V``
    defaults to ``row0 + w.shape[0]``); its rows may be strided (unit column
    stride).  ``out`` is the whole head's blob, allocated when None; only this
    chunk's 64-row blocks are written."""
    if not w.is_cuda or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D GPU tensor with unit column stride")
    rows, K = w.shape
    V = row0 + rows if V is None else V
    n = packed_bytes(V, K, bits, group)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w.device)
    elif not out.is_cuda or not out.is_contiguous() or out.numel() * out.element_size() < n:
        raise ValueError(f"out must be a contiguous GPU buffer of at least {n} bytes")
    _check("lmhead_quantize_pack", lib().lmhead_quantize_pack(
        _ptr(w), _DT[w.dtype], w.stride(0), V, K, bits, group, _DT[scale_dtype], _CLIP[clip], row0,
        rows, _ptr(out), _stream(w)))
    return out


def quantize_pack_host(w: torch.Tensor, bits: int, group: int,
                       scale_dtype: torch.dtype = torch.float16, clip: str = "rtn", *,
                       chunk_rows: int = 8192, device="cuda") -> torch.Tensor:
    """Quantize a head held in host memory chunk by chunk into a device blob.

    Each chunk of ``chunk_rows`` rows (a multiple of 64) is copied into one
    device staging buffer and handed to lmhead_quantize_pack, so the device
    holds the blob plus one chunk, never the whole unquantized head."""
    if w.is_cuda or w.dim() != 2:
        raise ValueError("w must be a 2-D host tensor")
    if chunk_rows <= 0 or chunk_rows % 64 != 0:
        raise ValueError("chunk_rows must be a positive multiple of 64")
    V, K = w.shape
    out = torch.empty(packed_bytes(V, K, bits, group), dtype=torch.uint8, device=device)
    stage = torch.empty((min(chunk_rows, max(V, 1)), K), dtype=w.dtype, device=device)
    for r0 in range(0, V, chunk_rows):
        n = min(chunk_rows, V - r0)
        stage[:n].copy_(w[r0:r0 + n])  # same stream as the kernel: ordered
        quantize_pack(stage[:n], bits, group, scale_dtype, clip, V=V, row0=r0, out=out)
    return out


def embed(ids: torch.Tensor, packed: torch.Tensor, V: int, K: int, bits: int, group: int,
          scale_dtype: torch.dtype = torch.float16, out_dtype: torch.dtype = torch.float16,
          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dequantized embedding rows [T, K] for int32 token ids -- lmhead_embed.
    Ids outside [0, V) give zero rows."""
    _need_cuda(ids, packed)
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    ids = ids.reshape(-1)
    T = ids.numel()
    if out is None:
        out = torch.empty((T, K), dtype=out_dtype, device=packed.device)
    elif not out.is_cuda or out.dim() != 2 or out.shape[0] != T or out.stride(1) != 1:
        raise ValueError("out must be a [T, >=K] GPU tensor with unit column stride")
    _check("lmhead_embed", lib().lmhead_embed(
        _ptr(ids), T, _ptr(packed), V, K, bits, group, _DT[scale_dtype], _ptr(out), _DT[out.dtype],
        out.stride(0), _stream(packed)))
    return out


def auto_path(M: int, K: int, bits: int, group: int, x_dtype: torch.dtype = torch.float16) -> int:
    """The kernel lmhead_logits runs for this shape and activation type
    (PATH_GEMV .. PATH_MFMA_SPLITK); host only."""
    out = ctypes.c_int(0)
    _check("lmhead_logits_auto_path_x",
           lib().lmhead_logits_auto_path_x(M, K, bits, group, _DT[x_dtype], ctypes.byref(out)))
    return out.value


def logits_workspace(M: int, K: int, x_dtype: torch.dtype, device) -> Optional[torch.Tensor]:
    n = int(lib().lmhead_logits_workspace_bytes(M, K, _DT[x_dtype]))
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def logits(x: torch.Tensor, packed: torch.Tensor, V: int, K: int, bits: int, group: int,
           scale_dtype: torch.dtype, bias: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           path: int = PATH_AUTO, out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Logits [M, V] (or into ``out`` [M, ldy]) in ``out_dtype`` (fp32, or fp16 / bf16
    rounded once from the fp32 result) -- lmhead_logits_typed."""
    _need_cuda(x, packed, bias)
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, V), dtype=out_dtype, device=x.device)
    elif out.stride(-1) != 1:
        raise ValueError("out must have unit column stride")
    ldy = out.stride(0) if out.dim() == 2 else V
    if workspace is None:
        workspace = logits_workspace(M, K, x.dtype, x.device)
    ws_n = 0 if workspace is None else workspace.numel()
    _check("lmhead_logits", lib().lmhead_logits_typed(
        _ptr(x), _DT[x.dtype], M, _ptr(packed), V, K, bits, group, _DT[scale_dtype], _ptr(bias),
        _ptr(out), _DT[out.dtype], ldy, _ptr(workspace), ws_n, path, _stream(x)))
    return out


def dense_logits(x: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 logits of an unquantized 16-bit weight -- lmhead_dense_logits (the control)."""
    _need_cuda(x, w)
    M, K = x.shape
    V = w.shape[0]
    if out is None:
        out = torch.empty((M, V), dtype=torch.float32, device=x.device)
    _check("lmhead_dense_logits", lib().lmhead_dense_logits(
        _ptr(x), _DT[x.dtype], M, _ptr(w), _DT[w.dtype], V, K, _ptr(out), out.stride(0),
        _stream(x)))
    return out


def topk_workspace(M: int, V: int, topk: int, device) -> torch.Tensor:
    n = int(lib().lmhead_topk_workspace_bytes(M, V, topk))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def topk_rescore(x: torch.Tensor, w_ref: torch.Tensor, y: torch.Tensor, topk: int,
                 workspace: Optional[torch.Tensor] = None):
    """In place on y; returns (idx int32 [M,topk], val fp32 [M,topk], top1 int32 [M])."""
    _need_cuda(x, w_ref, y)
    M, K = x.shape
    V = w_ref.shape[0]
    idx = torch.empty((M, topk), dtype=torch.int32, device=x.device)
    val = torch.empty((M, topk), dtype=torch.float32, device=x.device)
    top1 = torch.empty((M,), dtype=torch.int32, device=x.device)
    if workspace is None:
        workspace = topk_workspace(M, V, topk, x.device)
    _check("lmhead_topk_rescore", lib().lmhead_topk_rescore(
        _ptr(x), _DT[x.dtype], M, _ptr(w_ref), _DT[w_ref.dtype], V, K, _ptr(y), y.stride(0), topk,
        _ptr(idx), _ptr(val), _ptr(top1), _ptr(workspace), workspace.numel(), _stream(x)))
    return idx, val, top1


def logits_topk_workspace(M: int, V: int, K: int, x_dtype: torch.dtype, topk: int,
                          device) -> torch.Tensor:
    n = lib().lmhead_logits_topk_workspace_bytes(M, V, K, _DT[x_dtype], topk)
    if n == 0:
        raise ValueError("invalid arguments for lmhead_logits_topk_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def logits_topk(x: torch.Tensor, packed: torch.Tensor, V: int, K: int, bits: int, group: int,
                scale_dtype: torch.dtype, w_ref: torch.Tensor, topk: int,
                bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                val: Optional[torch.Tensor] = None, top1: Optional[torch.Tensor] = None):
    """Logits + exact top-K rescoring in one call -- lmhead_logits_topk.  ``out``
    (fp32 [M, >= V]) receives the logits with the rescored values scattered in;
    when None they are not stored.  Returns (idx, val, top1)."""
    _need_cuda(x, packed, w_ref, bias)
    M = x.shape[0]
    if idx is None:
        idx = torch.empty((M, topk), dtype=torch.int32, device=x.device)
    if val is None:
        val = torch.empty((M, topk), dtype=torch.float32, device=x.device)
    if top1 is None:
        top1 = torch.empty((M,), dtype=torch.int32, device=x.device)
    if workspace is None:
        workspace = logits_topk_workspace(M, V, K, x.dtype, topk, x.device)
    ldy = out.stride(0) if out is not None else 0
    _check("lmhead_logits_topk", lib().lmhead_logits_topk(
        _ptr(x), _DT[x.dtype], M, _ptr(packed), V, K, bits, group, _DT[scale_dtype], _ptr(bias),
        _ptr(w_ref), _DT[w_ref.dtype], topk, _ptr(out), ldy, _ptr(idx), _ptr(val), _ptr(top1),
        _ptr(workspace), workspace.numel(), _stream(x)))
    return idx, val, top1


# ---- prepared calls: arguments converted once, for tight decode loops ----------

_raw_lib: Optional[ctypes.CDLL] = None


def _raw() -> ctypes.CDLL:
    """A second handle on the library whose functions carry no argtypes, so a
    prepared call passes its ready-made ctypes values without conversion."""
    global _raw_lib
    if _raw_lib is None:
        lib()  # raises if the library is missing
        _raw_lib = ctypes.CDLL(LIB_PATH)
        for name in ("lmhead_logits_typed", "lmhead_logits_topk", "lmhead_topk_rescore",
                     "lmhead_embed", "lmhead_dense_logits", "lmhead_stream_read",
                     "lmhead_stream_mix", "lmhead_mfma_ceiling"):
            getattr(_raw_lib, name).restype = ctypes.c_int
    return _raw_lib


def _cargs(sig, vals):
    """Python values -> ctypes values of the declared argument types."""
    return tuple(None if v is None and t is ctypes.c_void_p else t(v) for t, v in zip(sig, vals))


class PreparedCall:
    """One library call whose arguments were checked and converted once.
    Calling it enqueues the same work again on the stream that was current when
    it was prepared (no Python-side checks, no allocation); the tensors it
    refers to are kept alive by the object and must not be resized or freed."""

    def __init__(self, name: str, args: tuple, keep: tuple):
        self._fn = getattr(_raw(), name)
        self._name = name
        self._args = _cargs(getattr(lib(), name).argtypes, args)
        self._keep = keep

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != LMH_OK:
            raise LmheadError(self._name, rc)


def prepare_logits(x: torch.Tensor, packed: torch.Tensor, V: int, K: int, bits: int, group: int,
                   scale_dtype: torch.dtype, out: torch.Tensor, bias: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, path: int = PATH_AUTO) -> PreparedCall:
    """lmhead_logits_typed on fixed tensors, as a PreparedCall (see logits)."""
    _need_cuda(x, packed, bias)
    if out.stride(-1) != 1:
        raise ValueError("out must have unit column stride")
    M = x.shape[0]
    if workspace is None:
        workspace = logits_workspace(M, K, x.dtype, x.device)
    ws_n = 0 if workspace is None else workspace.numel()
    args = (_ptr(x), _DT[x.dtype], M, _ptr(packed), V, K, bits, group, _DT[scale_dtype], _ptr(bias),
            _ptr(out), _DT[out.dtype], out.stride(0), _ptr(workspace), ws_n, path, _stream(x))
    return PreparedCall("lmhead_logits_typed", args, (x, packed, bias, out, workspace))


def prepare_logits_topk(x: torch.Tensor, packed: torch.Tensor, V: int, K: int, bits: int,
                        group: int, scale_dtype: torch.dtype, w_ref: torch.Tensor, topk: int,
                        idx: torch.Tensor, val: torch.Tensor, top1: torch.Tensor,
                        bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> PreparedCall:
    """lmhead_logits_topk on fixed tensors, as a PreparedCall (see logits_topk)."""
    _need_cuda(x, packed, w_ref, bias)
    M = x.shape[0]
    if workspace is None:
        workspace = logits_topk_workspace(M, V, K, x.dtype, topk, x.device)
    ldy = out.stride(0) if out is not None else 0
    args = (_ptr(x), _DT[x.dtype], M, _ptr(packed), V, K, bits, group, _DT[scale_dtype], _ptr(bias),
            _ptr(w_ref), _DT[w_ref.dtype], topk, _ptr(out), ldy, _ptr(idx), _ptr(val), _ptr(top1),
            _ptr(workspace), workspace.numel(), _stream(x))
    return PreparedCall("lmhead_logits_topk", args,
                        (x, packed, w_ref, idx, val, top1, bias, out, workspace))


def stream_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """One read-only pass over src's bytes (lmhead_stream_read; a measurement aid)."""
    _need_cuda(src, sink)
    nb = src.numel() * src.element_size()
    _check("lmhead_stream_read", lib().lmhead_stream_read(_ptr(src), nb, _ptr(sink), _stream(src)))


def prepare_stream_read(src: torch.Tensor, sink: torch.Tensor) -> PreparedCall:
    _need_cuda(src, sink)
    nb = src.numel() * src.element_size()
    return PreparedCall("lmhead_stream_read", (_ptr(src), nb, _ptr(sink), _stream(src)), (src, sink))


def stream_mix(src: torch.Tensor, dst: torch.Tensor) -> None:
    """One pass reading src's bytes and writing dst's (lmhead_stream_mix; a measurement aid)."""
    _need_cuda(src, dst)
    _check("lmhead_stream_mix", lib().lmhead_stream_mix(
        _ptr(src), src.numel() * src.element_size(), _ptr(dst), dst.numel() * dst.element_size(),
        _stream(src)))


def prepare_stream_mix(src: torch.Tensor, dst: torch.Tensor) -> PreparedCall:
    _need_cuda(src, dst)
    return PreparedCall("lmhead_stream_mix",
                        (_ptr(src), src.numel() * src.element_size(), _ptr(dst),
                         dst.numel() * dst.element_size(), _stream(src)), (src, dst))


MFMA_CEILING_SINK = 256 * 1024  # floats lmhead_mfma_ceiling's sink receives


def prepare_mfma_ceiling(rounds: int, valu_per_mfma: int, sink: torch.Tensor) -> PreparedCall:
    """lmhead_mfma_ceiling (a measurement aid) on a fixed sink, as a PreparedCall."""
    _need_cuda(sink)
    if sink.dtype != torch.float32 or sink.numel() < MFMA_CEILING_SINK:
        raise ValueError(f"sink must be a float32 GPU tensor of at least {MFMA_CEILING_SINK} elements")
    return PreparedCall("lmhead_mfma_ceiling", (int(rounds), int(valu_per_mfma), _ptr(sink), _stream(sink)),
                        (sink,))


def mfma_ceiling_flops(rounds: int) -> int:
    """Flops of one lmhead_mfma_ceiling call with `rounds` rounds."""
    return int(lib().lmhead_mfma_ceiling_mfmas(int(rounds))) * 16 * 16 * 32 * 2


def prepare_dense_logits(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor) -> PreparedCall:
    """lmhead_dense_logits on fixed tensors, as a PreparedCall."""
    _need_cuda(x, w)
    M, K = x.shape
    args = (_ptr(x), _DT[x.dtype], M, _ptr(w), _DT[w.dtype], w.shape[0], K, _ptr(out),
            out.stride(0), _stream(x))
    return PreparedCall("lmhead_dense_logits", args, (x, w, out))


def prepare_topk_rescore(x: torch.Tensor, w_ref: torch.Tensor, y: torch.Tensor, topk: int,
                         idx: torch.Tensor, val: torch.Tensor, top1: torch.Tensor,
                         workspace: torch.Tensor) -> PreparedCall:
    """lmhead_topk_rescore on fixed tensors, as a PreparedCall."""
    _need_cuda(x, w_ref, y)
    M, K = x.shape
    args = (_ptr(x), _DT[x.dtype], M, _ptr(w_ref), _DT[w_ref.dtype], w_ref.shape[0], K, _ptr(y),
            y.stride(0), topk, _ptr(idx), _ptr(val), _ptr(top1), _ptr(workspace),
            workspace.numel(), _stream(x))
    return PreparedCall("lmhead_topk_rescore", args, (x, w_ref, y, idx, val, top1, workspace))


def prepare_embed(ids: torch.Tensor, packed: torch.Tensor, V: int, K: int, bits: int, group: int,
                  scale_dtype: torch.dtype, out: torch.Tensor) -> PreparedCall:
    """lmhead_embed on fixed tensors, as a PreparedCall."""
    _need_cuda(ids, packed)
    args = (_ptr(ids), ids.numel(), _ptr(packed), V, K, bits, group, _DT[scale_dtype], _ptr(out),
            _DT[out.dtype], out.stride(0), _stream(ids))
    return PreparedCall("lmhead_embed", args, (ids, packed, out))


def logits_topk_noalloc(x: torch.Tensor, packed: torch.Tensor, V: int, K: int, bits: int,
                        group: int, scale_dtype: torch.dtype, w_ref: torch.Tensor, topk: int,
                        idx: torch.Tensor, val: torch.Tensor, top1: torch.Tensor,
                        bias: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None) -> None:
    """logits_topk without a workspace -- lmhead_logits_topk_noalloc (the
    library's own scratch; nothing is allocated, the outputs are given)."""
    _need_cuda(x, packed, w_ref, bias)
    M = x.shape[0]
    ldy = out.stride(0) if out is not None else 0
    _check("lmhead_logits_topk_noalloc", lib().lmhead_logits_topk_noalloc(
        _ptr(x), _DT[x.dtype], M, _ptr(packed), V, K, bits, group, _DT[scale_dtype], _ptr(bias),
        _ptr(w_ref), _DT[w_ref.dtype], topk, _ptr(out), ldy, _ptr(idx), _ptr(val), _ptr(top1),
        _stream(x)))


class QuantizedHead:
    """A packed LM head resident on the GPU: quantize + pack once, then logits per call."""

    def __init__(self, w: torch.Tensor, bits: int, group: int,
                 scale_dtype: torch.dtype = torch.float16, clip: str = "rtn", zp: bool = False):
        self.V, self.K = w.shape
        # zero-point heads carry the LMH_ZP flag in `bits` for every call
        self.bits = bits | ZP if zp else bits
        self.group, self.scale_dtype = group, scale_dtype
        self.packed = quantize_pack(w, self.bits, group, scale_dtype, clip)

    def embed(self, ids: torch.Tensor, out_dtype: torch.dtype = torch.float16) -> torch.Tensor:
        """Input-embedding rows of the same packed table (tied head)."""
        return embed(ids, self.packed, self.V, self.K, self.bits, self.group, self.scale_dtype,
                     out_dtype)

    def __call__(self, x: torch.Tensor, bias: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
        return logits(x, self.packed, self.V, self.K, self.bits, self.group, self.scale_dtype,
                      bias=bias, out=out)
