"""Build libgqe.so (HIP, gfx950) in-tree with hipcc.

    python -m sparse_query_gqa_amd.build

Every source in csrc/ is compiled to an object in parallel, then linked into
sparse_query_gqa_amd/libgqe.so. The packed-fp32 target feature is switched
off for every device compile.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqe.so")
ARCH = os.environ.get("GQE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["gqe_api.hip", "route.hip", "prefill.hip", "decode.hip", "out_proj.hip", "qkv_proj.hip", "prefill_bwd.hip",
           "layer_bwd.hip"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    # device code only: no NaN canonicalisation around min/max (infinities are
    # still honoured); the host code keeps IEEE NaN semantics for its argument checks
    "-Xarch_device", "-fno-honor-nans",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source flags. The attention backward keeps its MFMA accumulators in
# VGPRs: its exponentials read the score accumulators, and with the AGPR form
# the d = 128 dK/dV kernel copied them out of AGPRs on every tile.
EXTRA = {"prefill_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the GQE library needs ROCm's hipcc to build")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only target feature; drop that note
    err = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


# Host-code sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) for a
# CPU-only check of the C ABI's argument handling; the device code is built
# as usual (no GPU sanitizer). Each -fsanitize= goes to the host pass only.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN_BUILD = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_BUILD, "libgqe_san.so")


def _compile_and_link(build_dir: str, lib: str, extra: list, link_extra: list, verbose: bool) -> str:
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        jobs.append([hipcc, *FLAGS, *extra, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out, file=sys.stderr)
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs])
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libgqe.so; returns the library path."""
    return _compile_and_link(BUILD, LIB, [], [], verbose)


def build_sanitized(verbose: bool = False) -> str:
    """libgqe_san.so: the same library with host-code ASan + UBSan (for CPU tests
    of the C ABI; load it with the sanitizer runtime preloaded)."""
    return _compile_and_link(SAN_BUILD, SAN_LIB, SANITIZE,
                             ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                              "-shared-libsan"], verbose)


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
