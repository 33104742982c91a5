"""Build the HIP library ``libdwps.so`` for gfx950 with hipcc (in-tree).

Usage: ``python -m device_wide_prefix_chained_amd.build`` (or ``build()``).
Every ``csrc/*.hip`` file is compiled to an object in ``_build/`` in parallel,
then linked into ``device_wide_prefix_chained_amd/libdwps.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libdwps.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are switched off for every HIP source.
COMMON_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep single-lane atomics as written: the wave-wide rewrite consumes the
    # returned ticket at once, which serialises it with the look-back polls
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-command-line-argument",
]


# Extra hipcc flags (e.g. -D overrides of the tile shape or look-back width
# for tuning builds); empty for the library as shipped.
EXTRA_FLAGS = os.environ.get("DWPS_HIPCC_FLAGS", "").split()


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *EXTRA_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libdwps.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources under " + CSRC)
    jobs = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIBRARY)
    if verbose:
        print("built", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
