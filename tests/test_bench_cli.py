"""bench.py's host side, without a GPU: the one-GPU contract (asking for more
than one GPU exits with a message before anything touches a device), the
options it documents, and the writers of the profiles/ summaries on small
hand-made rocprofv3 CSV files -- kernel-name shortening, the FETCH_SIZE /
WRITE_SIZE calibration against the read-only stream and the head clones, the
sources hash that gates `traffic`, and the SQ counters' derived columns --
and the size sweep's fit of a fixed cost plus a steady rate."""
import argparse
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")

import bench  # noqa: E402  (the repository root is on sys.path, see conftest)


def _run(*argv, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, BENCH, *argv], capture_output=True, text=True, env=e,
                          timeout=120)


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = _run(*argv, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_names_the_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--ms", "--path", "--size-sweep",
                "--agreement", "--summarize", "--summarize-sq", "--record"):
        assert opt in r.stdout, opt


def test_short_kernel_names():
    mangled = ("_ZN3lmh12_GLOBAL__N_111gemv_kernelILi4ELi1ELi2ELi1ELi0ELb0ELb1ELi0EEEvPK15HIP_vector_"
               "typeIjLj4EEPKtPKhS8_PKfPvliiiiiiiiiPyi")
    assert bench._short_kernel(mangled) == "gemv_kernel<4,1,2,1,0,false,true,0>"
    demangled = ("void lmh::(anonymous namespace)::mfma_xres_kernel<4, 2, 2, false, 0, false, 2, 0, 4>"
                 "(HIP_vector_type<unsigned int, 4u> const*, float*)")
    assert bench._short_kernel(demangled) == "mfma_xres_kernel<4,2,2,false,0,false,2,0,4>"
    assert bench._short_kernel("void lmh::(anonymous namespace)::stream_read_kernel(uint4 const*)") \
        == "stream_read_kernel"
    assert bench._short_kernel("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)
    return str(path)


STREAM = "void lmh::(anonymous namespace)::stream_read_kernel(uint4 const*, long, unsigned int*)"
GEMV = ("void lmh::(anonymous namespace)::gemv_kernel<4, 1, 2, 1, 0, false, false, 0>"
        "(HIP_vector_type<unsigned int, 4u> const*)")


def _traffic_files(tmp_path, head, zp_blob):
    stats = _write_csv(tmp_path / "stats.csv",
                       ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
                       [[GEMV, 10, 50000, 5000, 60.0, 4800, 5300],
                        [STREAM, 10, 40000, 4000, 40.0, 3900, 4100]])
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    # the stream reads the head once: FETCH_SIZE half its KiB -> factor 2
    fetch = _write_csv(tmp_path / "fetch.csv", hdr,
                       [[STREAM, 4096, "FETCH_SIZE", head / 1024 / 2]] * 2 +
                       [[GEMV, 8192, "FETCH_SIZE", 1000.0], [GEMV, 8192, "FETCH_SIZE", 1200.0]])
    # the clones of the zero-point head write its bytes exactly -> factor 1;
    # a small unrelated copy is left out of the calibration
    write = _write_csv(tmp_path / "write.csv", hdr,
                       [["__amd_rocclr_copyBuffer", 1, "WRITE_SIZE", zp_blob / 1024],
                        ["__amd_rocclr_copyBuffer", 1, "WRITE_SIZE", 3.0],
                        [GEMV, 8192, "WRITE_SIZE", 10.0], [STREAM, 4096, "WRITE_SIZE", 0.0]])
    return stats, fetch, write


def test_summarize_traffic_calibration(tmp_path, monkeypatch):
    import weight_only_quantized_lmhead_amd as lmh

    wl = "tiny_w4g64_50304x512"
    head = lmh.packed_bytes(50304, 512, 4, 64)
    zp_blob = lmh.packed_bytes(50304, 512, 4 | lmh.ZP, 64)
    stats, fetch, write = _traffic_files(tmp_path, head, zp_blob)
    out = tmp_path / "summary.md"
    args = argparse.Namespace(workload=wl, cmd=["rocprofv3 ... (test)"], stats=stats, fetch=fetch,
                              write=write, out=str(out))
    assert bench.summarize(args) == 0
    text = out.read_text()
    assert "| `gemv_kernel<4,1,2,1,0,false,false,0>` | 10 | 5.00 | 4.80 | 5.30 | 60.0% |" in text
    rec = json.loads(text.split("<!-- traffic ", 1)[1].rsplit("-->", 1)[0])
    assert rec["workload"] == wl and rec["sources_sha"] == bench.sources_sha()
    k = {r["kernel"]: r for r in rec["kernels"]}
    g = k["gemv_kernel<4,1,2,1,0,false,false,0> grid 8192"]
    assert g["read_bytes"] == round(1100.0 * 2 * 1024) and g["write_bytes"] == 10 * 1024
    assert g["dispatches"] == 2
    s = k["stream_read_kernel grid 4096"]
    assert s["read_bytes"] == head and s["write_bytes"] == 0
    # bench reports the recorded bytes only while the kernel sources match
    monkeypatch.setattr(bench, "traffic_file", lambda w: str(out))
    got = bench.recorded_traffic(wl, "gemv_kernel<", ",false,false,0>")
    assert got is not None and got["bytes"] == g["bytes"]
    assert bench.recorded_traffic(wl, "gemv_kernel<", ",false,true,0>") is None
    monkeypatch.setattr(bench, "sources_sha", lambda: "0" * 16)
    assert bench.recorded_traffic(wl, "gemv_kernel<", ",false,false,0>") is None


def test_summarize_sq_derived_columns(tmp_path):
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    K = "void lmh::(anonymous namespace)::mfma_xres_kernel<4, 2, 2, false, 0, false, 2, 0, 4>(float*)"
    cyc = 1000.0  # GPU cycles of the dispatch; the counter sums the 8 XCDs
    p1 = _write_csv(tmp_path / "sq1.csv", hdr, [
        [K, 262144, "GRBM_GUI_ACTIVE", 8 * cyc],
        [K, 262144, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * 1024],
        [K, 262144, "SQ_WAVE_CYCLES", 4000.0], [K, 262144, "SQ_ACTIVE_INST_LDS", 1000.0],
        [K, 262144, "SQ_ACTIVE_INST_VMEM", 400.0], [K, 262144, "SQ_WAIT_INST_ANY", 2000.0],
        ["__amd_rocclr_copyBuffer", 1, "SQ_WAVES", 5.0]])
    p2 = _write_csv(tmp_path / "sq2.csv", hdr, [
        [K, 262144, "SQ_INSTS_MFMA", 100.0], [K, 262144, "SQ_INSTS_VALU", 100.0 + 64000.0],
        [K, 262144, "SQ_INSTS_LDS", 50.0], [K, 262144, "SQ_LDS_BANK_CONFLICT", 25.0],
        [K, 262144, "SQ_WAVES", 4096.0]])
    out = tmp_path / "sq.md"
    args = argparse.Namespace(workload="w4g64_151936x1024", cmd=["(test)"], sq=[p1, p2], out=str(out))
    assert bench.summarize_sq(args) == 0
    row = [l for l in out.read_text().splitlines()
           if l.startswith("| `mfma_xres_kernel<4,2,2,false,0,false,2,0,4> grid 262144` | 50.0%")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    # MFMA busy, VALU busy = 4 x 64000 / (1000 x 1024), LDS / VMEM active and
    # wait over wave cycles, VALU per MFMA, LDS per MFMA, conflicts per LDS
    # instruction, waves
    assert cells[1:] == ["50.0%", "25.0%", "25.0%", "10.0%", "50.0%", "640.00", "0.50", "0.50", "4096"]
    assert "copyBuffer" not in out.read_text()


def test_size_sweep_fit():
    """time = fixed + bytes / rate, recovered from points on an exact line
    (6000 GB/s and 2 us: a call of B bytes takes 2 + B / 6000 * 1e-3 us) and
    from the same points with symmetric noise."""
    nb = [82653184 * m for m in (1, 2, 4, 8)]
    us = [2.0 + b / 6000.0 * 1e-3 for b in nb]
    f = bench.fit_fixed_rate(nb, us)
    assert f == {"GB/s": 6000.0, "frac_of_hbm_peak": 0.75, "fixed_us": 2.0}
    noisy = [t + d for t, d in zip(us, (0.05, -0.05, -0.05, 0.05))]
    g = bench.fit_fixed_rate(nb, noisy)
    assert abs(g["GB/s"] - 6000.0) < 10 and abs(g["fixed_us"] - 2.0) < 0.1
