"""Build liblora_mi355x.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblora_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library (always rebuilds)."""
    with tempfile.TemporaryDirectory(prefix="lora_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
            if verbose and r.stderr:
                print(r.stderr)
            return obj
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            objs = list(ex.map(compile_one, sources()))
        out = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s" % r.stderr)
        os.replace(out, LIB)
    return LIB


def ensure_built() -> str:
    """Build only when no library is present (tests, smoke and bench use this)."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
