"""The host layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds libhstu with api.cpp's host code instrumented (hstu_jagged_pointwise_amd/asan_build.py)
and runs the host-side test files against that build, in a child process that preloads the
shared ASan runtime. Any sanitizer report aborts the child, which fails this test. No GPU
is used: every call in those files returns before its first HIP call."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_abi.py", "tests/test_sl_host.py"]


def _have_hipcc():
    from hstu_jagged_pointwise_amd import build as B
    return os.path.exists(B.HIPCC)


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")
def test_host_layer_is_clean_under_asan_and_ubsan(tmp_path):
    from hstu_jagged_pointwise_amd import asan_build as A
    lib = A.build_asan(verbose=False)
    env = dict(os.environ)
    env.update(HSTU_LIB=lib, LD_PRELOAD=A.asan_runtime(),
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:log_path={tmp_path}/asan",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={tmp_path}/ubsan")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *HOST_TESTS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    reports = "".join(open(os.path.join(tmp_path, f)).read() for f in os.listdir(tmp_path)
                      if f.startswith(("asan", "ubsan")))
    assert r.returncode == 0 and not reports, \
        f"sanitized host tests failed (rc {r.returncode}):\n{reports}\n{r.stdout[-3000:]}"
    assert " passed" in r.stdout
