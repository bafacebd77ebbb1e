"""Build libqmm.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Every source is compiled to an object in parallel (one hipcc per source),
then the objects are linked into the shared library."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqmm.so")
# The timing build: the same library with the streaming and resident kernels
# compiled with per-wave timestamps (QMM_WAVE_STAMPS); loaded only by
# `bench.py --wave-timeline`.
STAMPS_LIB = os.path.join(PKG, "libqmm_stamps.so")
STAMPED = ("qmm_stream.hip", "qmm_resident.hip", "qmm_slab.hip")
SOURCES = ["qmm_layout.hip", "qmm_mfma.hip", "qmm_stream.hip", "qmm_resident.hip",
           "qmm_slab.hip", "qmm_wide.hip", "qmm_norm.hip", "qmm_attention.hip",
           "qmm_generic.hip", "qmm_fmt.hip", "qmm_noalloc.hip", "qmm_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, obj: str, verbose: bool, extra=()):
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def _link(objs, lib, verbose):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking " + os.path.basename(lib))
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int = 0, stamps: bool = True) -> str:
    """Build libqmm.so and, unless stamps=False, the timing build
    libqmm_stamps.so; returns the path of libqmm.so."""
    tmpdir = tempfile.mkdtemp(prefix="qmm_build_")
    try:
        units = [(s, os.path.join(tmpdir, s + ".o"), ()) for s in SOURCES]
        if stamps:
            units += [(s, os.path.join(tmpdir, s + ".stamps.o"), ("-DQMM_WAVE_STAMPS",))
                      for s in STAMPED]
        jobs = jobs or min(len(units), os.cpu_count() or 4, 16)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda u: _compile(u[0], u[1], verbose, u[2]), units))
        bad = [(u[0], r) for u, r in zip(units, results) if r.returncode != 0]
        for s, r in bad:
            sys.stderr.write("--- %s\n%s%s" % (s, r.stdout, r.stderr))
        if bad:
            raise RuntimeError("hipcc failed on " + ", ".join(s for s, _ in bad))
        _link([u[1] for u in units[:len(SOURCES)]], LIB, verbose)
        if stamps:
            stamped = {u[0]: u[1] for u in units[len(SOURCES):]}
            _link([stamped.get(s, os.path.join(tmpdir, s + ".o")) for s in SOURCES], STAMPS_LIB,
                  verbose)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
