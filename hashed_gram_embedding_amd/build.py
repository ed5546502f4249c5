"""Build libengram.so (HIP, gfx950) in-tree.

    python -m hashed_gram_embedding_amd.build

Compiles every source under csrc/ with hipcc for gfx950 only and links them
into hashed_gram_embedding_amd/libengram.so, and a second time with
ENGRAM_DEBUG_CHECKS defined into libengram_debug.so (the kernels check the
device-resident preconditions into the caller's error word; see
engram_debug_checks in include/engram.h).  Packed-FP32 instructions are
disabled in device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libengram.so")
LIB_DEBUG = os.path.join(PKG, "libengram_debug.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libengram.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function"]


# Per-source flags.  ahead.hip: the compiler's wave-level atomic combining
# would read the arrival count's return value at once (to spread it over the
# lanes), so the count's round trip to memory would stall the wavefront
# instead of overlapping the loads that follow it; its one atomic comes from
# a single lane anyway.
FILE_FLAGS = {"ahead.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + FILE_FLAGS.get(os.path.basename(src), []) + list(extra) + \
        ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    lines = [l for l in out.splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(lines))
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Builds libengram.so and libengram_debug.so; returns the release path."""
    debug_dir = os.path.join(BUILD, "debug")
    os.makedirs(debug_dir, exist_ok=True)
    srcs = sources()
    jobs = [(src, BUILD, ()) for src in srcs] + [(src, debug_dir, ("-DENGRAM_DEBUG_CHECKS",)) for src in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], LIB_DEBUG)
    if verbose:
        print(f"built {LIB} and {LIB_DEBUG}")
    return LIB


if __name__ == "__main__":
    build()
