"""The C ABI called from plain C (tests/c_abi/*.c): each program is compiled
by gcc as C11 with every warning an error against include/lmhead.h, linked to
liblmhead.so, and run as a child process.  The host program needs no GPU; the
GPU program quantizes, packs and runs every logits path on a small head."""
import os
import subprocess

from gpu_common import gpu, need_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "weight_only_quantized_lmhead_amd")


def _build(name: str, hip: bool) -> str:
    src = os.path.join(ROOT, "tests", "c_abi", name + ".c")
    out_dir = os.path.join(ROOT, "_build", "c_abi")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, name)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include")]
    if hip:
        cmd += ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]
    cmd += [src, "-L", LIB_DIR, "-llmhead", f"-Wl,-rpath,{LIB_DIR}"]
    if hip:
        cmd += ["-L", "/opt/rocm/lib", "-lamdhip64"]
    cmd += ["-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_program_host_calls():
    exe = _build("abi_host", hip=False)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c host abi ok" in r.stdout, r.stdout + r.stderr


@gpu
def test_c_program_gpu_round_trip():
    need_gpu()
    exe = _build("abi_gpu", hip=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c gpu abi ok" in r.stdout, r.stdout + r.stderr
