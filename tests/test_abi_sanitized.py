"""The C-ABI validation tests again, against a build of the library whose host
code is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer.

No GPU is needed: every validation error returns before any HIP call. The
sanitized build (mxfp4_block_scaled_02_amd/build.py, build_sanitized) differs
from the normal one only in its host-side flags; device code is unchanged. The
uninstrumented python interpreter gets the clang ASan runtime preloaded, and
any sanitizer report fails the run."""
import os
import subprocess
import sys

from mxfp4_block_scaled_02_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_under_asan_and_ubsan():
    lib = build.build_sanitized(verbose=False)
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in syms and "__ubsan_handle_" in syms, "the check build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(), MXFP4_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
