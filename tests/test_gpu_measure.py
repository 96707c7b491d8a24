"""The measurement aids bench.py times beside the logits kernels: the
read-only stream, the read+write stream and the MFMA ceiling run and write
what they promise, and the MFMA ceiling's accumulators grow linearly with its
round count (integer operands, exact in fp32)."""
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


def _mix_expected(src_words: torch.Tensor, n_dst: int) -> torch.Tensor:
    """What lmhead_stream_mix writes (its header): thread t of workgroup b
    XORs the words b*1024 + 256 j + t (j < 4) it reads and writes that, plus i
    in the first 32-bit lane, to words b*W*256 + 256 i + t (i < W)."""
    n_src = src_words.shape[0]
    grid = max(1, -(-n_src // 1024))
    W = -(-n_dst // (grid * 256))
    pad = torch.zeros((grid * 1024, 4), dtype=torch.int32)
    pad[:n_src] = src_words
    a = pad.view(grid, 4, 256, 4)
    x = a[:, 0] ^ a[:, 1] ^ a[:, 2] ^ a[:, 3]                 # [grid, 256, 4]
    out = x[:, None].repeat(1, W, 1, 1)                       # [grid, W, 256, 4]
    out[..., 0] += torch.arange(W, dtype=torch.int32)[None, :, None]
    return out.reshape(-1, 4)[:n_dst]


@pytest.mark.parametrize("n_src,n_dst", [(4096, 1024), (5000, 1187), (1000, 7000), (0, 300),
                                         (3000, 0), (1 << 16, 1 << 17)])
def test_stream_mix_writes_its_function(n_src, n_dst):
    """The read+write stream reads each source word once and writes every
    destination word once, with the values its header states (so that no
    write is dead and none lands outside dst)."""
    need_gpu()
    gen = torch.Generator().manual_seed(n_src + n_dst)
    src = torch.randint(-2**31, 2**31 - 1, (max(n_src, 1), 4), dtype=torch.int32, generator=gen)
    dst = torch.full((n_dst + 64, 4), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    src_d = src.to(DEV)
    lmh.lib().lmhead_stream_mix(src_d.data_ptr(), n_src * 16, dst.data_ptr(), n_dst * 16, None)
    torch.cuda.synchronize()
    got = dst.cpu()
    assert torch.equal(got[:n_dst], _mix_expected(src[:n_src], n_dst))
    assert (got[n_dst:] == 0x5A5A5A5A).all(), "words past write_bytes were written"


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
