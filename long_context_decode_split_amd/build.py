"""Build libkvd.so for gfx950 with hipcc (in-tree, no JIT cache).

Every source under csrc/ is compiled to an object in _build/ (in parallel) and
linked into long_context_decode_split_amd/libkvd.so.  Packed-fp32 instruction
selection is disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "kvd")
LIB = os.path.join(PKG, "libkvd.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "lse_merge.hip", "partial_valu.hip", "partial_gqa_mfma.hip",
           "partial_gqa_mfma_tokens.hip", "partial_gqa_tokens32.hip", "partial_mla_mfma.hip", "append_kv.hip"]

# Per-source extra flags.  The GQA kernels keep their MFMA accumulators in
# ordinary VGPRs (they have room, and the occasional vector-ALU rescale of
# the accumulator would otherwise make the compiler shuttle them between
# AGPRs and VGPRs every tile; the four-token kernel holds its query operands
# in AGPRs instead); the two-token one-wave instances
# (partial_gqa_mfma_tokens.hip) and the latent kernel need the AGPRs for their
# accumulators and keep the default.
SOURCE_FLAGS = {"partial_gqa_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "partial_gqa_tokens32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + SOURCE_FLAGS.get(src, []) + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line
                    and "not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    return obj


EXAMPLE_SRC = os.path.join(PKG, "examples", "decode_from_c.c")
EXAMPLE = os.path.join(PKG, "examples", "decode_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_example(verbose: bool = False) -> str:
    """Compile the plain-C caller of the ABI (gcc, host code only) against
    libkvd.so and the HIP runtime; returns its path."""
    tmp = EXAMPLE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", os.path.join(ROCM, "include"), EXAMPLE_SRC, "-L", PKG, "-lkvd", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/..:" + os.path.join(ROCM, "lib"), "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, EXAMPLE)
    if verbose:
        print("built", EXAMPLE)
    return EXAMPLE


def build(extra=(), jobs: int = 8, verbose: bool = False) -> str:
    """Compile all sources and link libkvd.so, then the C example; returns the
    library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_example(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
