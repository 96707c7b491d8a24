"""Library calls captured in a HIP graph (the use the allocation-free decode
entry exists for): the M = 1 GEMV, the split-K MFMA kernel at M = 8, the
activation-resident MFMA kernel at M = 40 and the
allocation-free logits + top-K call are captured once on a side stream, then
the graph is replayed three times with new inputs written by ordinary eager
work between the replays; every replay's outputs must equal, bit for bit,
the same calls made eagerly on the same inputs (the library records no
memset and allocates nothing, so replays read and write only the captured
buffers)."""
import numpy as np
import pytest
import torch

import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, gpu, need_gpu

pytestmark = gpu


def test_graph_replays_match_eager_calls():
    need_gpu()
    V, K, bits, G, topk = 64 * 41 + 19, 1024, 4, 64, 8
    w = synth.random_weight((V, K), 0.02, 77, (V - 1,))
    wd = torch.from_numpy(w).to(DEV)
    blob = lmh.quantize_pack(wd, bits, G, torch.float16, "rtn")
    w_ref = wd.to(torch.float16)
    x1 = torch.empty((1, K), dtype=torch.float16, device=DEV)
    x8 = torch.empty((8, K), dtype=torch.float16, device=DEV)
    x40 = torch.empty((40, K), dtype=torch.float16, device=DEV)
    y1 = torch.empty((1, V), dtype=torch.float32, device=DEV)
    y8 = torch.empty((8, V), dtype=torch.float32, device=DEV)
    y40 = torch.empty((40, V), dtype=torch.float32, device=DEV)
    yk = torch.empty((1, V), dtype=torch.float32, device=DEV)
    idx = torch.empty((1, topk), dtype=torch.int32, device=DEV)
    val = torch.empty((1, topk), dtype=torch.float32, device=DEV)
    top1 = torch.empty((1,), dtype=torch.int32, device=DEV)
    outs = (y1, y8, y40, yk, idx, val, top1)

    def fill(seed):
        x1.copy_(torch.from_numpy(synth.random_x(1, K, seed=seed)).to(DEV))
        x8.copy_(torch.from_numpy(synth.random_x(8, K, seed=seed + 2)).to(DEV))
        x40.copy_(torch.from_numpy(synth.random_x(40, K, seed=seed + 1)).to(DEV))

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c1 = lmh.prepare_logits(x1, blob, V, K, bits, G, torch.float16, y1)
        c8 = lmh.prepare_logits(x8, blob, V, K, bits, G, torch.float16, y8)
        c40 = lmh.prepare_logits(x40, blob, V, K, bits, G, torch.float16, y40)

        def decode():
            lmh.logits_topk_noalloc(x1, blob, V, K, bits, G, torch.float16, w_ref, topk, idx, val,
                                    top1, out=yk)

        fill(1)
        c1()
        c8()
        c40()
        decode()  # first call on the device also looks up the scratch address
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        c1()
        c8()
        c40()
        decode()
    for r in range(3):
        for o in outs:
            o.fill_(-1)  # eager work between the replays
        fill(10 + r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        for o in outs:
            o.fill_(-2)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            c1()
            c8()
            c40()
            decode()
        s.synchronize()
        for a, b, name in zip(got, outs, ("y M=1", "y M=8", "y M=40", "decode y", "idx", "val", "top1")):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), (r, name)
        assert lmh.auto_path(8, K, bits, G) == lmh.PATH_MFMA_SPLITK
        assert lmh.auto_path(40, K, bits, G) == lmh.PATH_MFMA_XRES
        # the replay really used the new inputs: the logits differ between replays
        if r > 0:
            assert not torch.equal(got[0], prev0)
        prev0 = got[0]
