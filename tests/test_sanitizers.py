"""The host side under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds the oracle and the library's host code with ``-fsanitize=address,
undefined`` (any report aborts), then runs the host-side suites -- the C
ABI's validation, planning and path selection, and every pin of the oracle
-- in a child process that preloads the sanitizer runtime and loads those
builds (CONVMI_SANITIZED=1).  The kernels themselves are device code and are
built as usual; nothing here launches one.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi_host.py", "tests/test_oracle_pins.py", "tests/test_oracle_pins_next.py",
          "tests/test_oracle_norm_pins.py"]


def runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(runtime() is None, reason="clang's AddressSanitizer runtime is not installed")
def test_host_suites_are_clean_under_asan_and_ubsan():
    import oracle
    from convolution_implicit_gemm_conv2d_amd import build

    oracle.build(sanitize=True)
    build.build(sanitize=True)
    env = dict(os.environ)
    env.update({
        "CONVMI_SANITIZED": "1",
        "LD_PRELOAD": runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *SUITES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "Sanitizer" not in r.stdout + r.stderr, tail
