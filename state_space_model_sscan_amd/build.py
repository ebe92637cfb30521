"""Build libsscan.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsscan.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = ["api.cpp", "tokenloop.hip", "m1_fast.hip", "tl_m1_f32.hip", "tl_m1_bf16.hip", "tl_ssd_f32.hip",
           "tl_ssd_bf16.hip", "m1f_f32_16.hip", "m1f_f32_32.hip", "m1f_f32_64.hip", "m1f_bf16_16.hip",
           "m1f_bf16_32.hip", "m1f_bf16_64.hip", "m1r_f32_16.hip", "m1r_f32_32.hip", "m1r_f32_64.hip",
           "m1r_bf16_16.hip", "m1r_bf16_32.hip", "m1r_bf16_64.hip", "ssd_chunk.hip", "mixer_ops.hip", "ssd_attention.hip",
           "scratch.hip", "m1q_f32_16.hip", "m1q_f32_32.hip", "m1q_f32_64.hip", "m1q_bf16_16.hip", "m1q_bf16_32.hip",
           "m1q_bf16_64.hip"]
ARCH = os.environ.get("SSCAN_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU instructions are switched off for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source flags. The SSD chunk kernel runs one workgroup per compute unit, so
# the compiler may also use the accumulation registers; kept in the vector form,
# its MFMA results need no copies between the two register files.
SOURCE_FLAGS = {"ssd_chunk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), "-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
           "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(extra: list[str] | None = None, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libsscan.so. Always recompiles."""
    os.makedirs(OBJDIR, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
