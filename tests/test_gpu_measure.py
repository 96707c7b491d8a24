"""The measurement aids bench.py times beside the logits kernels: the
read-only stream and the MFMA ceiling run, write what they promise, and the
MFMA ceiling's accumulators grow linearly with its round count (integer
operands, exact in fp32)."""
import pytest
import torch

import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, gpu, need_gpu

pytestmark = gpu


def test_stream_read_runs():
    need_gpu()
    src = torch.arange(1 << 20, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1024, dtype=torch.uint8, device=DEV)
    lmh.stream_read(src, sink)
    lmh.stream_read(src[:4], sink)  # a partial run of one workgroup
    torch.cuda.synchronize()


@pytest.mark.parametrize("nv", [0, 2, 4])
def test_mfma_ceiling_linear_in_rounds(nv):
    need_gpu()
    outs = []
    for rounds in (1, 2, 3):
        sink = torch.full((lmh.MFMA_CEILING_SINK,), float("nan"), dtype=torch.float32, device=DEV)
        lmh.prepare_mfma_ceiling(rounds, nv, sink)()
        torch.cuda.synchronize()
        assert torch.isfinite(sink).all(), rounds
        outs.append(sink.double())
    if nv == 0:  # the VALU values stay fixed: sum(acc) grows by the same amount per round
        assert torch.equal(outs[2] - outs[1], outs[1] - outs[0])
        assert (outs[1] - outs[0]).abs().max() > 0
