"""Host-side checks of the C ABI (no GPU needed, nothing launched).

  * liblmhead.so loads and exports every function include/lmhead.h declares;
  * the size helpers agree with the layout definition (and with the oracle);
  * every validation error path returns its status before any HIP call.
Calls here only pass arguments the library must reject, or empty (M == 0 / V == 0)
requests, so no kernel is ever launched.
"""
import ctypes
import os
import re

import pytest
import torch

import oracle
import weight_only_quantized_lmhead_amd as lmh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmhead.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_UNSUP, E_WS, E_HIP, E_SCRATCH = range(9)
F32, F16, BF16 = 0, 1, 2
P = 0x10000  # a fake, 16-byte-aligned non-null address: never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lmhead_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = lmh.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} declared in lmhead.h but not exported"
    assert L.lmhead_abi_version() == 2


def test_status_strings():
    L = lmh.lib()
    for s in range(9):
        assert L.lmhead_status_string(s).startswith(b"LMH_")
    assert b"unknown" in L.lmhead_status_string(99)


@pytest.mark.parametrize("V,K,bits,G", [(151936, 1024, 4, 64), (151936, 1024, 8, 128),
                                        (151936, 2048, 8, 2048), (248064, 5120, 4, 128),
                                        (50304, 512, 4, 64), (1, 128, 4, 32), (65, 64, 8, 32),
                                        (100, 256, 4, 256), (7, 384, 4, 128)])
def test_packed_bytes_matches_layout(V, K, bits, G):
    assert lmh.packed_bytes(V, K, bits, G) == oracle.packed_bytes(V, K, bits, G)


@pytest.mark.parametrize("V,K,bits,G", [(10, 100, 4, 50), (10, 192, 4, 64), (10, 96, 8, 32),
                                        (10, 384, 4, 96), (10, 128, 3, 32), (10, 128, 4, 16),
                                        (10, 256, 8, 96)])
def test_packed_bytes_rejects(V, K, bits, G):
    assert lmh.lib().lmhead_packed_bytes(V, K, bits, G) == 0


def _logits(**kw):
    a = dict(x=P, xd=F16, M=1, packed=P, V=128, K=128, bits=4, G=64, sd=F16, bias=None, y=P,
             ldy=128, ws=None, wsn=0, path=0, st=None)
    a.update(kw)
    return lmh.lib().lmhead_logits_path(a["x"], a["xd"], a["M"], a["packed"], a["V"], a["K"],
                                        a["bits"], a["G"], a["sd"], a["bias"], a["y"], a["ldy"],
                                        a["ws"], a["wsn"], a["path"], a["st"])


def test_logits_validation():
    assert _logits(bits=3) == E_UNSUP
    assert _logits(K=100) == E_SHAPE
    assert _logits(K=192) == E_SHAPE          # int4 needs K % 128 == 0
    assert _logits(G=48) == E_SHAPE
    assert _logits(K=384, G=96) == E_UNSUP    # a 96-column group straddles 128-column superchunks
    assert _logits(xd=F32) == E_DTYPE
    assert _logits(sd=F32) == E_DTYPE
    assert _logits(M=-1) == E_SHAPE
    assert _logits(M=70000) == E_SHAPE
    assert _logits(ldy=100) == E_SHAPE
    assert _logits(x=None) == E_NULL
    assert _logits(packed=None) == E_NULL
    assert _logits(y=None) == E_NULL
    assert _logits(x=P + 8) == E_ALIGN
    assert _logits(packed=P + 4) == E_ALIGN
    assert _logits(y=P + 2) == E_ALIGN
    # bf16 x: the MFMA kernels take it converted in the workspace (the GEMV,
    # M <= 2 by default, converts it itself and needs none)
    assert _logits(xd=BF16, M=3) == E_WS
    assert _logits(xd=BF16, path=2) == E_WS
    assert _logits(xd=BF16, path=3, ws=P, wsn=16) == E_WS
    assert _logits(path=1, M=5) == E_UNSUP   # the GEMV serves M <= 4
    assert _logits(path=6) == E_UNSUP
    assert _logits(path=5, M=17) == E_UNSUP  # the split-K kernel serves M <= 16
    # empty requests are valid and launch nothing
    assert _logits(M=0) == OK
    assert _logits(V=0) == OK


def test_workspace_sizes():
    L = lmh.lib()
    assert L.lmhead_logits_workspace_bytes(4, 1024, F16) == 0
    n = L.lmhead_logits_workspace_bytes(3, 5120, BF16)
    assert n >= 3 * 5120 * 2 + 3 * 4 and n % 256 == 0
    assert L.lmhead_topk_workspace_bytes(1, 151936, 8) >= 1 * 38 * 9 * 8
    assert L.lmhead_topk_workspace_bytes(1, 151936, 65) == 0


def test_quantize_pack_validation():
    L = lmh.lib()
    q = L.lmhead_quantize
    assert q(P, F32, 4, 128, 5, 64, F16, 0, P, P, None) == E_UNSUP
    assert q(P, 7, 4, 128, 4, 64, F16, 0, P, P, None) == E_DTYPE
    assert q(P, F32, 4, 128, 4, 64, F32, 0, P, P, None) == E_DTYPE
    assert q(P, F32, 4, 128, 4, 64, F16, 2, P, P, None) == E_UNSUP
    assert q(P, F32, 4, 100, 4, 64, F16, 0, P, P, None) == E_SHAPE
    assert q(P, F32, 4, 128, 4, 16, F16, 0, P, P, None) == E_SHAPE
    assert q(None, F32, 4, 128, 4, 64, F16, 0, P, P, None) == E_NULL
    assert q(P + 4, F32, 4, 128, 4, 64, F16, 0, P, P, None) == E_ALIGN
    assert q(P, F32, 0, 128, 4, 64, F16, 0, P, P, None) == OK
    # one wavefront per 64 rows and group, at most 2^26 - 32 of them (the
    # grid's work-item count fits 32 bits); None pointers: nothing launches
    assert q(None, F32, 64 * (2**21 - 1), 1024, 4, 32, F16, 0, P, P, None) == E_NULL
    assert q(None, F32, 64 * 2**21, 1024, 4, 32, F16, 0, P, P, None) == E_UNSUP
    pk = L.lmhead_pack
    assert pk(P, P, 4, 100, 4, 64, P, None) == E_SHAPE
    assert pk(None, P, 4, 128, 4, 64, P, None) == E_NULL
    assert pk(P, P, 4, 128, 4, 64, P + 1, None) == E_ALIGN
    assert pk(P, P, 0, 128, 4, 64, P, None) == OK


def test_fused_quantize_pack_validation():
    L = lmh.lib()

    def qp(w=P, wdt=F32, ldw=128, V=200, K=128, bits=4, G=64, sdt=F16, clip=0, row0=0, rows=200,
           out=P):
        return L.lmhead_quantize_pack(w, wdt, ldw, V, K, bits, G, sdt, clip, row0, rows, out, None)

    assert qp(bits=5) == E_UNSUP
    assert qp(K=100) == E_SHAPE
    assert qp(G=48) == E_SHAPE
    assert qp(wdt=7) == E_DTYPE
    assert qp(sdt=F32) == E_DTYPE
    assert qp(clip=2) == E_UNSUP
    assert qp(row0=32, rows=64) == E_SHAPE            # chunks start on a 64-row block
    assert qp(row0=64, rows=100) == E_SHAPE           # a chunk that is not last: whole blocks
    assert qp(row0=128, rows=100) == E_SHAPE          # past V
    assert qp(row0=-64, rows=64) == E_SHAPE
    assert qp(rows=-1) == E_SHAPE
    assert qp(ldw=120) == E_SHAPE                     # ldw < K
    assert qp(ldw=132) == E_SHAPE                     # rows must stay 16-byte aligned
    assert qp(w=None) == E_NULL
    assert qp(out=None) == E_NULL
    assert qp(w=P + 8) == E_ALIGN
    assert qp(out=P + 4) == E_ALIGN
    assert qp(w=None, rows=0, row0=64) == OK          # empty chunk: nothing launched
    assert qp(V=0, rows=0) == OK
    # at most 2^26 - 32 wavefronts (64 rows x one 128-column superchunk each)
    big = 64 * (2**23 - 4)
    assert qp(w=None, V=big, rows=big, K=1024, ldw=1024) == E_NULL
    assert qp(w=None, V=64 * 2**23, rows=64 * 2**23, K=1024, ldw=1024) == E_UNSUP


def test_dense_and_topk_validation():
    L = lmh.lib()
    d = L.lmhead_dense_logits
    assert d(P, F16, 1, P, BF16, 10, 64, P, 10, None) == E_DTYPE
    assert d(P, F32, 1, P, F32, 10, 64, P, 10, None) == E_DTYPE
    assert d(P, F16, 5, P, F16, 10, 64, P, 10, None) == E_SHAPE
    assert d(P, F16, 1, P, F16, 10, 60, P, 10, None) == E_SHAPE
    assert d(P, F16, 1, P, F16, 10, 64, P, 9, None) == E_SHAPE
    assert d(None, F16, 1, P, F16, 10, 64, P, 10, None) == E_NULL
    assert d(P, F16, 0, P, F16, 10, 64, P, 10, None) == OK
    t = L.lmhead_topk_rescore
    args = lambda **k: [k.get("x", P), k.get("xd", F16), k.get("M", 1), k.get("w", P),
                        k.get("wd", F16), k.get("V", 100), k.get("K", 64), k.get("y", P),
                        k.get("ldy", 100), k.get("topk", 8), None, None, None, k.get("ws", P),
                        k.get("wsn", 1 << 20), None]
    assert t(*args(topk=0)) == E_SHAPE
    assert t(*args(topk=65)) == E_SHAPE
    assert t(*args(topk=101)) == E_SHAPE
    assert t(*args(xd=F32)) == E_DTYPE
    assert t(*args(wd=5)) == E_DTYPE
    assert t(*args(ws=None)) == E_WS
    assert t(*args(wsn=8)) == E_WS
    assert t(*args(y=None)) == E_NULL
    assert t(*args(M=0)) == OK


def _logits_topk(**kw):
    a = dict(x=P, xd=F16, M=1, packed=P, V=128, K=128, bits=4, G=64, sd=F16, bias=None, w=P,
             wd=F16, topk=8, y=P, ldy=128, idx=P, val=P, top1=P, ws=P, wsn=1 << 30, st=None)
    a.update(kw)
    return lmh.lib().lmhead_logits_topk(a["x"], a["xd"], a["M"], a["packed"], a["V"], a["K"],
                                        a["bits"], a["G"], a["sd"], a["bias"], a["w"], a["wd"],
                                        a["topk"], a["y"], a["ldy"], a["idx"], a["val"],
                                        a["top1"], a["ws"], a["wsn"], a["st"])


def test_logits_topk_validation():
    """Every error path of the fused entry returns before any HIP call."""
    assert _logits_topk(bits=3) == E_UNSUP
    assert _logits_topk(K=100) == E_SHAPE
    assert _logits_topk(xd=F32) == E_DTYPE
    assert _logits_topk(sd=F32) == E_DTYPE
    assert _logits_topk(wd=7) == E_DTYPE
    assert _logits_topk(topk=0) == E_SHAPE
    assert _logits_topk(topk=65) == E_SHAPE
    assert _logits_topk(topk=129, V=128) == E_SHAPE
    assert _logits_topk(M=70000) == E_SHAPE
    assert _logits_topk(ldy=100) == E_SHAPE
    assert _logits_topk(V=(1 << 21) + 64, ldy=(1 << 21) + 64) == E_UNSUP
    assert _logits_topk(x=None) == E_NULL
    assert _logits_topk(w=None) == E_NULL
    assert _logits_topk(x=P + 8) == E_ALIGN
    assert _logits_topk(w=P + 2) == E_ALIGN
    assert _logits_topk(y=P + 2) == E_ALIGN
    assert _logits_topk(ws=None) == E_WS
    assert _logits_topk(wsn=16) == E_WS
    assert _logits_topk(ws=P + 8) == E_ALIGN
    assert _logits_topk(M=0) == OK
    assert _logits_topk(V=0) == OK
    L = lmh.lib()
    n1 = L.lmhead_logits_topk_workspace_bytes(1, 151936, 1024, F16, 8)
    # the top-K lists (75 blocks of 2048 entries x 9 codes) and an fp32 logits scratch
    assert n1 >= 75 * 9 * 8 + 151936 * 4 and n1 % 256 == 0
    assert L.lmhead_logits_topk_workspace_bytes(1, 151936, 1024, F16, 65) == 0
    assert L.lmhead_logits_topk_workspace_bytes(1, 151936, 1024, F32, 8) == 0


def test_embed_validation():
    L = lmh.lib()

    def em(ids=P, T=4, packed=P, V=200, K=128, bits=4, G=64, sdt=F16, out=P, odt=F16, ldo=128):
        return L.lmhead_embed(ids, T, packed, V, K, bits, G, sdt, out, odt, ldo, None)

    assert em(bits=5) == E_UNSUP
    assert em(K=100) == E_SHAPE
    assert em(sdt=F32) == E_DTYPE
    assert em(odt=7) == E_DTYPE
    assert em(T=-1) == E_SHAPE
    assert em(ldo=120) == E_SHAPE
    assert em(ids=None) == E_NULL
    assert em(out=None) == E_NULL
    assert em(ids=P + 2) == E_ALIGN
    assert em(out=P + 8) == E_ALIGN
    assert em(ldo=132) == E_ALIGN                 # 16-bit rows must stay 16-byte aligned
    assert em(T=0, ids=None, out=None) == OK


def test_logits_typed_validation():
    L = lmh.lib()

    def lt(ydt=F16, y=P, path=0, **kw):
        a = dict(x=P, xdt=F16, M=2, packed=P, V=200, K=128, bits=4, G=64, sdt=F16, bias=None,
                 ldy=200, ws=None, wsn=0)
        a.update(kw)
        return L.lmhead_logits_typed(a["x"], a["xdt"], a["M"], a["packed"], a["V"], a["K"], a["bits"],
                                     a["G"], a["sdt"], a["bias"], y, ydt, a["ldy"], a["ws"], a["wsn"],
                                     path, None)

    assert lt(ydt=7) == E_DTYPE
    assert lt(ydt=F16, y=P + 1) == E_ALIGN
    assert lt(ydt=F32, y=P + 2) == E_ALIGN
    assert lt(ydt=BF16, ldy=100) == E_SHAPE
    assert lt(ydt=F16, M=0) == OK


ZP = 0x10


@pytest.mark.parametrize("V,K,bits,G", [(151936, 1024, 4, 64), (151936, 1024, 8, 128),
                                        (1, 128, 4, 32), (65, 64, 8, 32), (100, 256, 4, 256)])
def test_zero_point_packed_bytes_matches_layout(V, K, bits, G):
    assert lmh.packed_bytes(V, K, bits | ZP, G) == oracle.packed_bytes_zp(V, K, bits, G)
    assert lmh.lib().lmhead_packed_bytes(10, 128, 3 | ZP, 32) == 0


def test_zero_point_validation():
    L = lmh.lib()
    qz = L.lmhead_quantize_zp
    assert qz(P, F32, 4, 128, 5, 64, F16, P, P, P, None) == E_UNSUP
    assert qz(P, 7, 4, 128, 4, 64, F16, P, P, P, None) == E_DTYPE
    assert qz(P, F32, 4, 128, 4, 64, F32, P, P, P, None) == E_DTYPE
    assert qz(P, F32, 4, 100, 4, 64, F16, P, P, P, None) == E_SHAPE
    assert qz(P, F32, 4, 128, 4, 64, F16, P, P, None, None) == E_NULL   # z_out is required
    assert qz(P, F32, 4, 128, 4, 64, F16, P + 8, P, P, None) == E_ALIGN
    assert qz(P, F32, 0, 128, 4 | ZP, 64, F16, P, P, P, None) == OK
    # the symmetric entry points do not take the flag
    assert L.lmhead_quantize(P, F32, 4, 128, 4 | ZP, 64, F16, 0, P, P, None) == E_UNSUP
    assert L.lmhead_pack(P, P, 4, 128, 4 | ZP, 64, P, None) == E_UNSUP
    pz = L.lmhead_pack_zp
    assert pz(P, P, P, 4, 100, 4, 64, P, None) == E_SHAPE
    assert pz(P, P, None, 4, 128, 4, 64, P, None) == E_NULL
    assert pz(P, P, P, 4, 128, 4, 64, P + 1, None) == E_ALIGN
    assert pz(P, P, P, 0, 128, 8, 64, P, None) == OK
    # fused quantize + pack: round to nearest only
    qp = L.lmhead_quantize_pack
    assert qp(P, F32, 128, 200, 128, 4 | ZP, 64, F16, 1, 0, 200, P, None) == E_UNSUP
    assert qp(P, F32, 128, 200, 128, 4 | ZP, 64, F16, 0, 0, 0, P, None) == OK
    # logits and embedding accept the flag (empty requests launch nothing)
    assert _logits(bits=4 | ZP, M=0) == OK
    assert _logits(bits=8 | ZP, G=64, V=0) == OK
    assert _logits(bits=3 | ZP) == E_UNSUP
    assert _logits(bits=4 | ZP, path=6) == E_UNSUP
    assert L.lmhead_embed(P, 0, P, 128, 128, 4 | ZP, 64, F16, P, F16, 128, None) == OK


def _auto(M, K=1024, bits=4, G=64):
    out = ctypes.c_int(-1)
    rc = lmh.lib().lmhead_logits_auto_path(M, K, bits, G, ctypes.byref(out))
    return rc, out.value


def test_auto_path_choice():
    # the automatic kernel choice, host only: the GEMV for one row (and two bf16
    # rows, or two rows of K > 2048), the split-K kernel for two fp16 rows and
    # for 3..16 rows when K <= 2048, the activation-resident
    # kernel when the tile fits (K <= 1024, G >= 64) beyond 32 rows, and from
    # 17 rows on for int4 heads; the LDS-staged kernel for int8 heads of
    # 17..32 rows
    GEMV, MFMA, LDS, XRES, SPLITK = (lmh.PATH_GEMV, lmh.PATH_MFMA, lmh.PATH_MFMA_LDS,
                                     lmh.PATH_MFMA_XRES, lmh.PATH_MFMA_SPLITK)
    for M, want in [(1, GEMV), (2, SPLITK), (3, SPLITK), (16, SPLITK), (17, XRES), (32, XRES),
                    (33, XRES), (64, XRES), (256, XRES), (65535, XRES)]:
        assert _auto(M) == (OK, want), M
    assert _auto(24, G=32) == (OK, LDS)               # 32-column groups: no resident tile
    for M, want in [(1, GEMV), (2, SPLITK), (3, SPLITK), (16, SPLITK), (17, LDS), (32, LDS),
                    (33, XRES), (256, XRES)]:
        assert _auto(M, bits=8, G=128) == (OK, want), M
    # the activation type matters at two rows only: bf16 rows stay on the GEMV
    # (no workspace); lmhead_logits_auto_path is the fp16 case
    for M, want in [(1, GEMV), (2, GEMV), (3, SPLITK), (40, XRES)]:
        assert lmh.auto_path(M, 1024, 4, 64, torch.bfloat16) == want, M
    for M in (1, 2, 3, 16, 40):
        assert lmh.auto_path(M, 1024, 4, 64, torch.float16) == _auto(M)[1]
    assert _auto(2, K=4096, G=128) == (OK, GEMV)       # K > 2048: two rows stay on the GEMV
    assert _auto(8, K=2048, bits=8, G=2048) == (OK, SPLITK)
    assert _auto(256, G=32) == (OK, LDS)              # 32-column groups: no resident tile
    assert _auto(256, K=2048) == (OK, LDS)            # the 64-row tile of K > 1024 exceeds LDS
    for M, want in [(2, GEMV), (3, LDS), (24, LDS), (25, MFMA), (32, MFMA), (33, LDS)]:
        assert _auto(M, K=5120, G=128) == (OK, want), M
    assert _auto(2, K=32768, G=128) == (OK, LDS)       # 2 x 32768 halves exceed the GEMV's LDS
    assert _auto(1, bits=4 | lmh.ZP) == (OK, GEMV)     # zero-point heads choose alike
    assert _auto(64, bits=8 | lmh.ZP, G=128) == (OK, XRES)
    assert lmh.auto_path(256, 1024, 4, 64) == XRES


def test_auto_path_validation():
    assert _auto(0) == (E_SHAPE, -1)
    assert _auto(65536) == (E_SHAPE, -1)
    assert _auto(1, bits=3) == (E_UNSUP, -1)
    assert _auto(1, K=192) == (E_SHAPE, -1)
    assert _auto(1, K=384, G=96) == (E_UNSUP, -1)
    assert lmh.lib().lmhead_logits_auto_path(1, 1024, 4, 64, None) == E_NULL
    out = ctypes.c_int(-1)
    assert lmh.lib().lmhead_logits_auto_path_x(1, 1024, 4, 64, F32, ctypes.byref(out)) == E_DTYPE
    assert lmh.lib().lmhead_logits_auto_path_x(2, 1024, 4, 64, BF16, None) == E_NULL
    assert out.value == -1


def test_logits_topk_noalloc_validation():
    """The allocation-free decode entry validates like lmhead_logits_topk and
    refuses, before any HIP call, a working set beyond its 16 MiB scratch."""
    L = lmh.lib()

    def call(**kw):
        a = dict(x=P, xd=F16, M=1, packed=P, V=151936, K=1024, bits=4, G=64, sd=F16, bias=None,
                 w=P, wd=F16, topk=8, y=P, ldy=151936)
        a.update(kw)
        return L.lmhead_logits_topk_noalloc(a["x"], a["xd"], a["M"], a["packed"], a["V"], a["K"],
                                            a["bits"], a["G"], a["sd"], a["bias"], a["w"], a["wd"],
                                            a["topk"], a["y"], a["ldy"], P, P, P, None)
    assert call(bits=3) == E_UNSUP
    assert call(topk=0) == E_SHAPE
    assert call(topk=65) == E_SHAPE
    assert call(xd=F32) == E_DTYPE
    assert call(wd=7) == E_DTYPE
    assert call(x=None) == E_NULL
    assert call(packed=P + 4) == E_ALIGN
    assert call(M=0) == OK
    # 64 rows of 200000 logits kept in the scratch (no y): 51 MB > 16 MiB
    assert call(M=64, V=200000, K=128, y=None, ldy=0) == E_SCRATCH
    assert L.lmhead_status_string(E_SCRATCH).decode().startswith("LMH_E_SCRATCH")


def test_measurement_aids_validation():
    """The ceiling kernels' entry points reject bad arguments before any HIP
    call, and report the MFMA count of a ceiling call."""
    L = lmh.lib()
    E_SHAPE, E_UNSUP, E_NULL = 2, 5, 1
    assert L.lmhead_stream_read(None, 17, None, None) == E_SHAPE
    assert L.lmhead_stream_read(None, 0, None, None) == OK
    assert L.lmhead_stream_read(None, 16, None, None) == E_NULL
    mix = L.lmhead_stream_mix
    assert mix(None, 17, None, 0, None) == E_SHAPE
    assert mix(None, 16, None, 24, None) == E_SHAPE
    assert mix(None, 0, None, 0, None) == OK
    assert mix(None, 16, P, 16, None) == E_NULL             # reads from nowhere
    assert mix(P, 16, None, 16, None) == E_NULL             # writes to nowhere
    assert mix(P + 8, 16, P, 16, None) == E_ALIGN
    assert mix(None, 1 << 38, None, 0, None) == E_UNSUP     # 2^24 workgroups: 2^32 work-items
    assert mix(None, 1 << 46, None, 0, None) == E_SHAPE
    assert L.lmhead_mfma_ceiling(0, 0, None, None) == E_SHAPE
    assert L.lmhead_mfma_ceiling(1 << 31, 0, None, None) == E_SHAPE
    assert L.lmhead_mfma_ceiling(10, 3, None, None) == E_UNSUP
    assert L.lmhead_mfma_ceiling(10, 2, None, None) == E_NULL
    # 256 workgroups x 16 waves x 8 MFMAs per round
    assert L.lmhead_mfma_ceiling_mfmas(10) == 10 * 8 * 16 * 256
    assert L.lmhead_mfma_ceiling_mfmas(0) == 0
    assert lmh.mfma_ceiling_flops(3) == 3 * 8 * 16 * 256 * 16 * 16 * 32 * 2
