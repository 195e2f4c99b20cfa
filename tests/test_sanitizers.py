"""AddressSanitizer and UndefinedBehaviorSanitizer builds, CPU only: the oracle (gcc) and the host
side of the C ABI (the library's sources with host-side instrumentation, hipcc; the device code is
not instrumented), each driven by a small C program over every path that runs without a GPU
(tests/sanitize/).  Any sanitizer report fails the run."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-o", exe, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "dpsgd_oracle.c"), "-lm"])
    r = _run([exe], env=SAN_ENV)
    assert r.stdout.strip().endswith("OK")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_abi_under_sanitizers(tmp_path):
    # each -fsanitize flag goes to the host compilation only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    srcs = sorted(glob.glob(os.path.join(ROOT, "differentially_private_amd", "csrc", "*.hip")) +
                  glob.glob(os.path.join(ROOT, "differentially_private_amd", "csrc", "*.cpp")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-x", "hip", "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "host_driver")
    _run([HIPCC, "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"), "-x", "c",
          os.path.join(ROOT, "tests", "sanitize", "host_driver.c"), "-x", "none", *objs, "-o", exe])
    r = _run([exe], env=SAN_ENV)
    assert r.stdout.strip().endswith("OK")
