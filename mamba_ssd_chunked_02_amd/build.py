"""Build the gfx950 HIP library libssd_mi355x.so in-tree with hipcc.

    python -m mamba_ssd_chunked_02_amd.build

Every source is compiled for gfx950 only, with packed-fp32 VALU forms
disabled (-packed-fp32-ops), and linked into one shared object next to this
file; only the C ABI of include/ssd.h is exported.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libssd_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["ssd_api.cpp", "ssd_prefill.hip", "ssd_scan_walk.hip", "ssd_decode.hip", "ssd_conv.hip",
           "ssd_noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile_flags():
    return ["--offload-arch=%s" % ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source and link the library.  Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [cc] + _compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = (r.stdout + r.stderr)
        # hipcc's host pass does not know the device-only feature name
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
        if verbose and out.strip():
            print(out)
        return obj

    n = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=%s" % ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
