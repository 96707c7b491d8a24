"""lmhead_logits_topk_noalloc (the library's own scratch, no workspace) against
lmhead_logits_topk (caller's workspace), through the C ABI: identical outputs,
bit for bit, on two calls in a row, the second with a smaller input (the
scratch then holds the first call's bytes), on the unfused path (several
activation rows, bf16 x through the MFMA kernel's conversion, logits kept in
the scratch) and on the fused one-row decode path; and a call whose working
set exceeds the scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, gpu, need_gpu, to_dev

pytestmark = gpu

E_SCRATCH = 8


def _case(V, K, bits, G, M, xdt, topk, with_y, seed):
    sdt = torch.bfloat16 if xdt == "bf16" else torch.float16
    w = synth.random_weight((V, K), 0.02, seed, (V - 1,))
    wd = torch.from_numpy(w).to(DEV)
    blob = lmh.quantize_pack(wd, bits, G, sdt, "rtn")
    w_ref = wd.to(sdt)
    x = to_dev(synth.random_x(M, K, seed=seed + 1, dtype=xdt), xdt)
    return dict(V=V, K=K, bits=bits, G=G, M=M, sdt=sdt, topk=topk, with_y=with_y, blob=blob,
                w_ref=w_ref, x=x)


def _outputs(c):
    M, V, topk = c["M"], c["V"], c["topk"]
    y = torch.full((M, V + 3), float("nan"), dtype=torch.float32, device=DEV) if c["with_y"] else None
    idx = torch.full((M, topk), -7, dtype=torch.int32, device=DEV)
    val = torch.full((M, topk), float("nan"), dtype=torch.float32, device=DEV)
    top1 = torch.full((M,), -7, dtype=torch.int32, device=DEV)
    return y, idx, val, top1


def _run_pair(c):
    # the existing entry point, with a workspace the binding allocates
    y0, i0, v0, t0 = _outputs(c)
    a, b, d = lmh.logits_topk(c["x"], c["blob"], c["V"], c["K"], c["bits"], c["G"], c["sdt"],
                              c["w_ref"], c["topk"], out=y0, idx=i0, val=v0, top1=t0)
    # the allocation-free entry point
    y1, i1, v1, t1 = _outputs(c)
    lmh.logits_topk_noalloc(c["x"], c["blob"], c["V"], c["K"], c["bits"], c["G"], c["sdt"],
                            c["w_ref"], c["topk"], i1, v1, t1, out=y1)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1), "top-K indices differ"
    assert torch.equal(v0.view(torch.int32), v1.view(torch.int32)), "rescored values differ"
    assert torch.equal(t0, t1), "top-1 differs"
    if c["with_y"]:
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), "logits differ"
    assert (i1 >= 0).all() and (i1 < c["V"]).all()


def test_noalloc_equals_workspace_entry_two_calls():
    need_gpu()
    # first call: 4 activation rows (unfused path), bf16 x (converted for the
    # MFMA kernel in the scratch), logits kept in the scratch (y not given)
    big = _case(V=30000, K=2048, bits=4, G=128, M=4, xdt="bf16", topk=16, with_y=False, seed=3)
    _run_pair(big)
    # second call, smaller: one row through the fused decode path, y stored
    small = _case(V=5000, K=512, bits=4, G=64, M=1, xdt="f16", topk=8, with_y=True, seed=5)
    _run_pair(small)
    # and a smaller unfused one with y given (int8 head)
    mid = _case(V=3000, K=256, bits=8, G=128, M=2, xdt="f16", topk=4, with_y=True, seed=7)
    _run_pair(mid)


def test_noalloc_rejects_requests_beyond_the_scratch():
    need_gpu()
    # 64 rows x 100000 logits kept in the scratch: 25.6 MB > 16 MiB
    M, V, K = 64, 100000, 128
    x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    blob = torch.zeros(lmh.packed_bytes(V, K, 4, 64), dtype=torch.uint8, device=DEV)
    w_ref = torch.zeros((V, K), dtype=torch.float16, device=DEV)
    idx = torch.zeros((M, 8), dtype=torch.int32, device=DEV)
    val = torch.zeros((M, 8), dtype=torch.float32, device=DEV)
    top1 = torch.zeros((M,), dtype=torch.int32, device=DEV)
    with pytest.raises(lmh.LmheadError) as e:
        lmh.logits_topk_noalloc(x, blob, V, K, 4, 64, torch.float16, w_ref, 8, idx, val, top1)
    assert e.value.status == E_SCRATCH
    assert (idx == 0).all() and (val == 0).all() and (top1 == 0).all()
