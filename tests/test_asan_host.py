"""The C ABI's argument validation built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side (device code unchanged) and driven
by tests/asan/abi_driver.cpp: every entry point with invalid, extreme and
boundary arguments.  Nothing gets past validation, so this runs on the CPU."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ulysses_sequence_parallelism_share_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers on the host pass only: each -fsanitize= right after -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.timeout(900)
def test_abi_validation_under_address_and_ub_sanitizers():
    out = os.path.join(ROOT, "_build", "asan")
    os.makedirs(out, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(f):
        obj = os.path.join(out, f[:-4] + ".o")
        r = subprocess.run([HIPCC, *FLAGS, *SAN, "-c", os.path.join(CSRC, f), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = os.path.join(out, "abi_driver.o")
    r = subprocess.run([HIPCC, *FLAGS, *SAN, "-c", os.path.join(ROOT, "tests", "asan", "abi_driver.cpp"),
                        "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = os.path.join(out, "abi_driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, drv, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]
    assert "all expectations held" in r.stdout
