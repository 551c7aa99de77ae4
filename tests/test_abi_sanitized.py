"""The CPU-only ABI tests again, against a build of the library whose host
code runs under AddressSanitizer and UndefinedBehaviorSanitizer (argument
checks, size arithmetic, status strings).  The sanitized build is made on
demand (``python -m sparse_gemm_layers_amd.build --host-sanitizers``, about a
minute) when it is missing or older than a source; the tests then run in a
child process with the sanitizer runtime preloaded, and any sanitizer report
fails them."""
import os
import subprocess
import sys

import pytest

from sparse_gemm_layers_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale() -> bool:
    if not os.path.exists(B.SAN_LIB):
        return True
    t = os.path.getmtime(B.SAN_LIB)
    deps = B.sources() + [os.path.join(ROOT, "include", "sg.h")]
    deps += [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC) if f.endswith(".h")]
    return any(os.path.getmtime(d) > t for d in deps)


@pytest.mark.timeout(600)
def test_abi_under_host_sanitizers():
    if os.environ.get("SG_LIBRARY"):
        pytest.skip("already running against another library build")
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    if _stale():
        B.build(verbose=False, sanitize=True)
    runtime = B.host_sanitizer_runtime()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, LD_PRELOAD=runtime, SG_LIBRARY=B.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-s", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=500)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "Sanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in out, out[-4000:]
