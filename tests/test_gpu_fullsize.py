"""Full-size workloads (the shapes the pages measure) on the GPU, checked against
the oracle on sampled rows: quantizer bit-exact on those rows, their packed row
blocks byte-exact, and their logits within the acceptance bars, in the same
launch configuration the benchmark times.  For M = 1 the oracle computes the
whole row of every head (its calls run row ranges on all host cores), so the
argmax gate covers every vocabulary row."""
import time

import numpy as np
import pytest
import torch

import oracle
import synth
import weight_only_quantized_lmhead_amd as lmh
from gpu_common import DEV, OD, TD, abs_terms, bits16, check_logits, gpu, need_gpu, to_dev

pytestmark = gpu


def _sample_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    V = w.V
    pick = set(rng.choice(V, size=n, replace=False).tolist())
    pick |= {0, 1, 63, 64, V - 1, V - 2, V - 64, V - 65}
    if w.zero_tail_rows:
        pick |= {V - w.zero_tail_rows, V - w.zero_tail_rows - 1}
    return np.array(sorted(pick), dtype=np.int64)


def _blocks_of(rows):
    return np.unique(rows // 64)


@pytest.fixture(scope="module", params=list(synth.WORKLOADS))
def built(request):
    need_gpu()
    w = synth.WORKLOADS[request.param]
    t0 = time.time()
    W = synth.weight(w)
    Wd = to_dev(W, w.w_dtype)
    q, s = lmh.quantize(Wd, w.bits, w.group, TD[w.scale_dtype], w.clip)
    blob = lmh.pack(q, s, w.bits, w.group)
    torch.cuda.synchronize()
    print(f"{w.name}: generated + quantized + packed in {time.time() - t0:.1f}s")
    yield w, W, Wd, q, s, blob
    del Wd, q, s, blob
    torch.cuda.empty_cache()


def test_fullsize_quantize_and_pack_sampled(built):
    w, W, Wd, q, s, blob = built
    rows = _sample_rows(w, 192, seed=w.wid)
    blocks = _blocks_of(rows)
    brows = (blocks[:, None] * 64 + np.arange(64)[None, :]).ravel()
    brows = brows[brows < w.V]
    ratios = oracle.MSE_RATIOS if w.clip == "mse" else oracle.RTN_RATIOS
    qo, so = oracle.quantize(np.ascontiguousarray(W[brows]), w.bits, w.group, OD[w.scale_dtype],
                             ratios, w_dtype=OD[w.w_dtype])
    qg = q[torch.from_numpy(brows).to(DEV)].cpu().numpy()
    sg = bits16(s[torch.from_numpy(brows).to(DEV)])
    assert np.array_equal(sg, so), "scales differ"
    assert np.array_equal(qg, qo), "codes differ"
    # packed bytes of the sampled row blocks
    NC = w.K // (128 if w.bits == 4 else 64)
    NG = w.K // w.group
    NB = (w.V + 63) // 64
    wreg = NB * 64 * w.K * w.bits // 8
    bl = blob.cpu().numpy()
    for b in blocks[:12]:
        r0, r1 = b * 64, min(w.V, b * 64 + 64)
        sel = (brows >= r0) & (brows < r1)
        ob = oracle.pack(qo[sel], so[sel], w.bits, w.group)
        owreg = 64 * w.K * w.bits // 8
        assert np.array_equal(bl[b * NC * 4096:(b + 1) * NC * 4096], ob[:owreg]), f"block {b} codes"
        sc = bl[wreg + b * NG * 128: wreg + (b + 1) * NG * 128]
        assert np.array_equal(sc, ob[owreg:]), f"block {b} scales"


def test_fullsize_fused_quantize_pack(built):
    """The fused quantize + pack kernel writes exactly the two-step blob at full
    size, in one call and in 8192-row chunks (the blob the sampled rows above
    pin to the oracle)."""
    w, W, Wd, q, s, blob = built
    fused = lmh.quantize_pack(Wd, w.bits, w.group, TD[w.scale_dtype], w.clip)
    assert torch.equal(fused, blob), "fused blob differs from pack(quantize(w))"
    fused.fill_(0x5A)
    for r0 in range(0, w.V, 8192):
        lmh.quantize_pack(Wd[r0:r0 + 8192], w.bits, w.group, TD[w.scale_dtype], w.clip, V=w.V,
                          row0=r0, out=fused)
    assert torch.equal(fused, blob), "chunked fused blob differs"
    del fused


def test_fullsize_logits_sampled(built):
    w, W, Wd, q, s, blob = built
    rows = _sample_rows(w, 256, seed=w.wid + 1)
    ratios = oracle.MSE_RATIOS if w.clip == "mse" else oracle.RTN_RATIOS
    qo, so = oracle.quantize(np.ascontiguousarray(W[rows]), w.bits, w.group, OD[w.scale_dtype],
                             ratios, w_dtype=OD[w.w_dtype])
    for M in w.Ms:
        x = synth.activations(w, M)
        y = lmh.logits(to_dev(x, w.x_dtype), blob, w.V, w.K, w.bits, w.group, TD[w.scale_dtype])
        torch.cuda.synchronize()
        ys = y[:, torch.from_numpy(rows).to(DEV)].cpu().numpy()
        y_or = oracle.logits(x, qo, so, OD[w.scale_dtype], w.group, x_dtype=OD[w.x_dtype])
        y_abs = abs_terms(x, w.x_dtype, qo, so, OD[w.scale_dtype], w.group)
        rel = check_logits(ys, y_or, y_abs, w.K, w.group, what=f"{w.name} M={M}")
        print(f"{w.name} M={M}: max row rel err on {len(rows)} sampled rows {rel:.2e}")
        # every padding row is exactly zero
        if w.zero_tail_rows:
            assert (y[:, w.V - w.zero_tail_rows:] == 0).all()


SWEEP_MS = (2, 3, 8, 16, 17, 24, 25, 32, 33)


def test_fullsize_kernel_choice_sweep_sampled(built):
    """Every kernel the automatic choice takes between 2 and 33 activation
    rows, at the workload's full size (split-K, the activation-resident tiles,
    the LDS-staged and register-fed kernels, the GEMV for two bf16 rows),
    checked on sampled rows against the oracle."""
    w, W, Wd, q, s, blob = built
    rows = _sample_rows(w, 128, seed=w.wid + 2)
    ratios = oracle.MSE_RATIOS if w.clip == "mse" else oracle.RTN_RATIOS
    qo, so = oracle.quantize(np.ascontiguousarray(W[rows]), w.bits, w.group, OD[w.scale_dtype],
                             ratios, w_dtype=OD[w.w_dtype])
    rows_d = torch.from_numpy(rows).to(DEV)
    used = {}
    for M in SWEEP_MS:
        x = synth.activations(w, M)
        y = lmh.logits(to_dev(x, w.x_dtype), blob, w.V, w.K, w.bits, w.group, TD[w.scale_dtype])
        torch.cuda.synchronize()
        ys = y[:, rows_d].cpu().numpy()
        y_or = oracle.logits(x, qo, so, OD[w.scale_dtype], w.group, x_dtype=OD[w.x_dtype])
        y_abs = abs_terms(x, w.x_dtype, qo, so, OD[w.scale_dtype], w.group)
        check_logits(ys, y_or, y_abs, w.K, w.group, what=f"{w.name} M={M}")
        used[M] = lmh.auto_path(M, w.K, w.bits, w.group, TD[w.x_dtype])
        del y
    print(f"{w.name}: kernel per M {used}")
    assert len(set(used.values())) >= 2


def test_fullsize_whole_row_argmax_m1(built):
    w, W, Wd, q, s, blob = built
    ratios = oracle.MSE_RATIOS if w.clip == "mse" else oracle.RTN_RATIOS
    t0 = time.time()
    qo, so = oracle.quantize(W, w.bits, w.group, OD[w.scale_dtype], ratios, w_dtype=OD[w.w_dtype])
    # the GPU quantizer is bit-exact on every row of the head
    assert np.array_equal(bits16(s), so), "scales differ"
    assert np.array_equal(q.cpu().numpy(), qo), "codes differ"
    x = synth.activations(w, 1)
    y = lmh.logits(to_dev(x, w.x_dtype), blob, w.V, w.K, w.bits, w.group, TD[w.scale_dtype])
    y = y.cpu().numpy()
    y_or = oracle.logits(x, qo, so, OD[w.scale_dtype], w.group, x_dtype=OD[w.x_dtype])
    y_abs = abs_terms(x, w.x_dtype, qo, so, OD[w.scale_dtype], w.group)
    rel = check_logits(y, y_or, y_abs, w.K, w.group, what=f"{w.name} whole row")
    print(f"{w.name} M=1 whole row: max rel err {rel:.2e}, argmax {int(np.argmax(y))} "
          f"(oracle {int(np.argmax(y_or))}), oracle took {time.time() - t0:.1f}s")
