"""Build libgdn.so (the HIP library behind include/gdn.h) for gfx950.

    python -m speculative_verify_gdn_amd.build [--timeline | --debug]

--timeline builds libgdn_timeline.so instead: the same library with the
wall-clock marks of csrc/gdn_timeline.h compiled into the fused verify step
(-DGDN_TIMELINE, objects in _build_timeline/), read back by
speculative_verify_gdn_amd/timeline.py.  The product library never has them.
--debug builds libgdn_debug.so (-DGDN_DEBUG, objects in _build_debug/): the
same library with the count of clamped accept lengths of csrc/gdn_debug.h,
read by gdn_debug_clamped_accepts.

Each .hip file under csrc/ is compiled to an object in _build/ (in parallel),
then linked into speculative_verify_gdn_amd/libgdn.so.  Flags:
  --offload-arch=gfx950          MI355X only
  -ffp-contract=off              every fused multiply-add is written out
  -fhip-fp32-correctly-rounded-divide-sqrt, -fno-gpu-flush-denormals-to-zero
                                 IEEE float division and denormals (the conv
                                 step is bit-exact by construction)
  -target-feature -packed-fp32-ops   no packed fp32 VALU instructions
  -mllvm -amdgpu-mfma-padding-ratio=100
                                 s_nops cover the latency between neighbouring
                                 MFMAs (only MFMA code changes).  Without them the
                                 chunked prefill gave wrong outputs in two elements
                                 of one accumulator tile, depending on timing: an
                                 MFMA that takes its accumulator from the MFMA
                                 just before it (into another register) read it
                                 after a later LDS load had refilled the register
                                 the compiler had freed.  With the same
                                 instructions and registers and the latency padded
                                 the outputs are right; the padding costs nothing
                                 measurable on the MFMA kernels here.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
ROOT = os.path.dirname(PKG)

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-padding-ratio=100",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I" + os.path.join(ROOT, "include"),
]
SOURCE_FLAGS: dict = {}


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), ()), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, timeline: bool = False, debug: bool = False) -> str:
    """Compile every HIP source and link libgdn.so (with timeline libgdn_timeline.so, with debug
    libgdn_debug.so); returns its path."""
    assert not (timeline and debug), "one variant at a time"
    variant = "_timeline" if timeline else ("_debug" if debug else "")
    build_dir = os.path.join(PKG, "_build" + variant)
    lib = os.path.join(PKG, "libgdn%s.so" % variant)
    extra = ("-DGDN_TIMELINE",) if timeline else (("-DGDN_DEBUG",) if debug else ())
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")), key=lambda f: -os.path.getsize(f))  # largest first
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, timeline="--timeline" in sys.argv[1:], debug="--debug" in sys.argv[1:])
    sys.exit(0)
