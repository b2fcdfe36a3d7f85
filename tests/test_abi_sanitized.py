"""The host layer of the C ABI (moe_api.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/abi_host_check.cpp drives the host-only
calls over a grid of configurations and the argument checks of the device
calls, linked against a copy of the host layer built with the sanitizers on
its host code (the device code is built as usual).  No GPU is used."""
import concurrent.futures as cf
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_39_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# sanitizers on the host code only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
BASE = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-function"]


def _compile(src, obj, extra):
    subprocess.run([HIPCC] + BASE + extra + ["-c", src, "-o", obj], check=True, capture_output=True)
    return obj


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.timeout(900)
def test_host_layer_under_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        jobs = [(os.path.join(ROOT, "tests", "abi_host_check.cpp"), os.path.join(d, "check.o"), SAN)]
        for f in sorted(os.listdir(CSRC)):
            if f.endswith((".hip", ".cpp")):
                jobs.append((os.path.join(CSRC, f), os.path.join(d, f + ".o"), SAN if f == "moe_api.cpp" else []))
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            objs = list(ex.map(lambda j: _compile(*j), jobs))
        exe = os.path.join(d, "abi_host_check")
        subprocess.run([HIPCC, "--offload-arch=gfx950"] + SAN[:4] + objs + ["-o", exe], check=True,
                       capture_output=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.startswith("OK")
