"""Build the gfx950 HIP library (libssd_mi355x.so) in-tree with hipcc.

Each source compiles to an object in parallel; the objects link into one shared library
under ``state_space_sequence_chunk_amd/_lib``. All device code is built with packed-fp32
instructions disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_lib")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(OUT, "libssd_mi355x.so")
SOURCES = ["ssd_api.cpp", "k_cumsum.hip", "k_chunk_state.hip", "k_chunk_state_mh_bf16.hip",
           "k_chunk_state_mh_f32.hip", "k_state_carry.hip", "k_state_scan.cpp",
           "k_state_scan_bf16.hip", "k_state_scan_bf16_f32.hip", "k_state_seg_bf16.hip", "k_decode.hip",
           "k_backward.hip", "k_backward_bf16.hip", "k_backward_f32.hip", "k_backward_mfma.hip",
           "k_chunk_out.cpp", "k_chunk_out_bf16.hip", "k_chunk_out_bf16_f32.hip", "k_chunk_out_bf16_ybf16.hip",
           "k_chunk_out_f32.hip", "k_chunk_out_bf16_seg.hip", "k_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str, extra) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc()] + common_flags() + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if src.endswith(".hip"):
        # the gfx950 assembly of the same source, for the instruction-level checks of the
        # test suite (tests/test_kernel_asm.py)
        asm = os.path.join(OBJ, os.path.basename(src) + ".s")
        cmd_s = [hipcc()] + common_flags() + list(extra) + lang + [
            "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm]
        rs = subprocess.run(cmd_s, capture_output=True, text=True)
        if rs.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src}:\n{rs.stdout}\n{rs.stderr}")
    if r.stderr.strip():
        # keep the compiler's warnings visible, minus hipcc's note that the host pass does
        # not know the device-only feature flag
        lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if any(ln.strip() for ln in lines):
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(extra_flags=(), jobs: int | None = None) -> str:
    os.makedirs(OUT, exist_ok=True)
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
