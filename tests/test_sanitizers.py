"""The CPU oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU needed).

* The oracle (oracle/lora_oracle.c) is built with gcc -fsanitize=address,
  undefined and driven on small seeded cases whose arrays have exactly the
  sizes the oracle's contract states (tests/sanitize/oracle_driver.c).
* The library's sources are built with the sanitizers on their host code only
  (each -fsanitize= behind -Xarch_host; the gfx950 code is built as usual and
  never runs here) and linked with tests/sanitize/abi_driver.cpp, which calls
  every entry point with arguments the host checks reject, plus the host-only
  calls.
Any report fails the run (-fno-sanitize-recover=all, nonzero exit).
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fopenmp", os.path.join(ROOT, "oracle", "lora_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = _run([exe], env=env, timeout=300)
    assert r.stdout.strip() == "ok"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "segmented_gather_lora_amd", "csrc")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", csrc] + SAN_HOST
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip"))) + [os.path.join(HERE, "abi_driver.cpp")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC, *flags, *lang, "-c", src, "-o", obj])
        return obj
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", *SAN_HOST, *objs, "-o", exe])
    # leak checks stay off: the HIP runtime keeps allocations of its own for the process
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env, timeout=300)
    assert r.stdout.startswith("ok ")
