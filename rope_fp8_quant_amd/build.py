"""Build libdsaidx.so in-tree with hipcc for gfx950.

    python -m rope_fp8_quant_amd.build

Device code is compiled without floating-point contraction (the arithmetic is
defined op by op) and without packed-fp32 instructions.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libdsaidx.so")
ARCH = "gfx950"

SOURCES = ["dsaidx_kernels.hip", "dsaidx_topk.hip", "dsaidx_logits.hip", "dsaidx_hbm_ref.hip",
           "dsaidx_proj.hip", "dsaidx_api.cpp"]
HEADERS = [os.path.join(INCLUDE, "dsaidx.h"), os.path.join(CSRC, "dsaidx_internal.h"),
           os.path.join(CSRC, "dsaidx_prep_device.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdsaidx)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
            "-ffp-contract=off", "-I" + INCLUDE, "-I" + CSRC]


def device_flags():
    return ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source device flags.  The logits kernel takes its MFMA results in
# ordinary VGPRs (it reads every element back for the epilogue, so results in
# AGPRs would cost a copy per element).
SOURCE_FLAGS = {"dsaidx_logits.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False, extra_defines=(), out_path: str = LIB_PATH,
          build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link libdsaidx.so; returns the library path.
    extra_defines / out_path / build_dir serve tuning builds of variants."""
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(build_dir, src + ".o")
        cmd = [cc] + common_flags() + ["-D" + d for d in extra_defines]
        if src.endswith(".hip"):
            cmd += device_flags() + SOURCE_FLAGS.get(src, []) + ["-x", "hip"]
        cmd += ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
