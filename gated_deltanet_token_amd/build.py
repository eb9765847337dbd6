"""Build libgdn.so in-tree for gfx950 with hipcc.

Usage: python gated_deltanet_token_amd/build.py   (or __graft_entry__.build());
this script never imports the package, which binds the library on import.

Every .hip source under csrc/ is compiled to an object in _build/ and linked
into gated_deltanet_token_amd/libgdn.so; ceiling/ceiling.hip (the benchmark's
reference copy kernels, not part of the library) into
gated_deltanet_token_amd/ceiling/libgdn_ceiling.so.  Packed-FP32 instruction selection
is disabled for all device code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
CEILING_SRC = os.path.join(PKG, "ceiling", "ceiling.hip")
CEILING_LIB = os.path.join(PKG, "ceiling", "libgdn_ceiling.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-result",
    # no packed-FP32 (v_pk_*_f32) instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: the chunkwise scan's accumulators
    # feed vector arithmetic directly, with no accumulator-register copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # the first 14 dwords of a kernel's arguments arrive in SGPRs at wave
    # launch (kernarg preloading), so a kernel's first dependent fetch (a slot
    # index, a descriptor) need not wait for its arguments' load; kernels put
    # the arguments of that chain first.  (A kernel entry also carries the
    # loads, skipped by firmware that preloads.)
    "-mllvm", "-amdgpu-kernarg-preload-count=14",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device-only feature flag; drop that note
    out = "\n".join(ln for ln in r.stdout.splitlines()
                    if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def hip_runtime_dir() -> str:
    """Directory of the HIP runtime the process will use.

    PyTorch ships its own libamdhip64.so and loads it under that name.  A
    second HIP runtime in the same process (e.g. /opt/rocm's
    libamdhip64.so.7) does not see the device, so libgdn links against
    exactly the library torch loads and records it by that name; the
    dynamic loader then resolves both to one runtime.
    """
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        raise RuntimeError("PyTorch (ROCm build) is required: it provides the HIP runtime")
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError("no libamdhip64.so in %s" % d)
    return d


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    rt = hip_runtime_dir()
    subprocess.check_call(["g++", "-shared", "-fPIC", "-o", tmp] + objs +
                          ["-L" + rt, "-lamdhip64", "-Wl,-rpath," + rt, "-Wl,--no-undefined"])
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(min(8, len(srcs) + 1)) as ex:
        objs = list(ex.map(_compile, srcs + [CEILING_SRC]))
    _link(objs[:-1], LIB)
    # the benchmark's reference copy / read-modify-write kernels, a library of
    # their own (not part of libgdn)
    _link(objs[-1:], CEILING_LIB)
    if verbose:
        print("built", LIB, "and", CEILING_LIB)
    return LIB


if __name__ == "__main__":
    build()
