"""Build libmla_decode.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 and linked into one shared
library next to this file. Run as a module or call build()."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmla_decode.so")
# the device peak microbenchmarks (HBM, matrix cores, LDS), a separate program
PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS_BIN = os.path.join(PKG, "peaks", "mla_peaks")
ARCH = "gfx950"

# Per-source extra hipcc flags, by file name (none needed at present).
EXTRA_FLAGS = {}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    common = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
              "-mcode-object-version=5",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
              "-Wno-unused-command-line-argument"]
    objs, procs = [], []
    for src in sources():
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc(), "-c", src, "-o", obj] + common + EXTRA_FLAGS.get(os.path.basename(src), [])
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs)
    # the peak microbenchmark program, built alongside
    cmd = [hipcc(), PEAKS_SRC, "-o", PEAKS_BIN + ".tmp"] + [a for a in common if a != "-fPIC"]
    procs.append((PEAKS_SRC, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    _drain(procs)
    os.replace(PEAKS_BIN + ".tmp", PEAKS_BIN)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}", "-fPIC"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    return LIB


def _drain(procs):
    errs = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            errs.append(f"{src}:\n{text}")
    procs.clear()
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
