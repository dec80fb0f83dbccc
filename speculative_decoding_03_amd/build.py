"""Builds libspecdec.so (HIP kernels + C ABI) for gfx950 in-tree with hipcc.

Usage: python -m speculative_decoding_03_amd.build  (or __graft_entry__.build()).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of every kernel (the compiler may otherwise form
# them from scalar float code).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function"]

# the GEMM's (storage type, M-tile count) instantiations compile in translation units of their own
SOURCES = ["gemm.hip", *[f"gemm_{t}_m{m}.hip" for t in ("bf16", "f32", "q4") for m in (1, 2, 4)],
           "gemm_mm.hip", "attention.hip", "misc.hip", "specdec.cpp", "policy.cpp"]
LIB = os.path.join(HERE, "libspecdec.so")
# The 4-bit weight kernels read every MFMA result with VALU instructions (the per-block step):
# results in architectural VGPRs save a copy out of the accumulation registers per element
# (the calls of at most 16 rows; the compiler fails on the wider instantiations with this form).
FILE_FLAGS = {"gemm_q4_m1.hip": ("-mllvm", "-amdgpu-mfma-vgpr-form")}


def _compile(src: str, obj: str, extra=()) -> None:
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *lang, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build_specdec(verbose: bool = True) -> str:
    bdir = os.path.join(ROOT, "_build", "specdec")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(os.cpu_count() or 4, 16, len(SOURCES))) as ex:
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(bdir, s + ".o")
            objs.append(obj)
            jobs.append(ex.submit(_compile, src, obj, FILE_FLAGS.get(s, ())))
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_specdec()
