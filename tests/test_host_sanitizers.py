"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

build() also links libssc_hostsan.so: the same kernels, with the host code of
the C ABI (argument validation, workspace layout, status handling) compiled
with -fsanitize=address,undefined.  The host-side ABI and binding tests run
here again in a child process through that library, with the ASan runtime
preloaded; any sanitizer report fails the test.  No kernel is launched (every
call in those tests stops in validation), so no GPU is needed.
"""

import glob
import os
import subprocess
import sys

import pytest

import spatial_spectral_coupling_amd as ssc
from spatial_spectral_coupling_amd import build as ssc_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this ROCm install")
    if not os.path.exists(ssc_build.LIB_HOSTSAN):
        ssc_build.build()
    logs = tmp_path / "san"
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": f"detect_leaks=0:abort_on_error=1:log_path={logs}",
        "UBSAN_OPTIONS": f"print_stacktrace=1:halt_on_error=1:log_path={logs}",
        "SSC_LIBRARY": ssc_build.LIB_HOSTSAN,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py"),
                        os.path.join(ROOT, "tests", "test_binding_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = sorted(glob.glob(str(logs) + "*"))
    text = "".join(open(f).read() for f in reports)
    assert not reports, text[:4000]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout
