"""Compile the HIP sources into kv_cache_attention_amd/libkvattn.so for gfx950.

Each translation unit is compiled by hipcc in parallel, then linked into one
shared library whose exported symbols are the extern "C" entry points of
include/kvattn.h.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kvattn.cpp", "decode_valu.hip", "valu_f16.hip", "valu_bf16.hip", "valu_f32.hip",
           "valu_f16_fp8.hip", "valu_bf16_fp8.hip", "decode_mfma.hip", "decode_mfma_fp8.hip", "debug_gather.hip",
           "append.hip", "prefill_mfma.hip", "validate.hip",
           "stream_read.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-Wall",
    # an oversized shift is undefined and lets the compiler drop the code after it
    "-Werror=shift-count-overflow", "-Werror=shift-count-negative",
    # no packed fp32 arithmetic on the device (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leave branches on wave-uniform conditions unstructured: the decode tile loops
    # branch only on scalars, and structuring them added paths on which the
    # compiler's load-wait counts fell to zero at the loop head
    "-mllvm", "-structurizecfg-skip-uniform-regions=true",
    # keep all-lane LDS atomics as written (the atomic optimizer turns them into a
    # single-lane atomic behind a lane-divergent branch, which brings structuring back)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I", os.path.join(os.path.dirname(HERE), "include"),
]

# Per-source additions.  The split-KV matrix-core kernels keep their output accumulators
# in ordinary vector registers (the matrix instructions read and write them there):
# with the accumulators in the accumulation registers, the rare rescale of the online
# softmax, which needs vector arithmetic on them, led the register allocator to copy
# all of them on every tile.
MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCE_FLAGS = {
    "decode_mfma.hip": MFMA_VGPR,
    "decode_mfma_fp8.hip": MFMA_VGPR,
}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *lang, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops" not in line)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
