"""The C-ABI boundary tests (test_abi_cpu.py) once more, against the
validation layer compiled with host AddressSanitizer and
UndefinedBehaviorSanitizer: qlora_api.hip's host code is rebuilt with the
sanitizers (device code unchanged), linked with the regular objects into
_build/libqlora_san.so, and the tests run in a child process with the clang
ASan runtime preloaded.  Any invalid memory access or undefined behaviour in
the argument checks, size computations and workspace layouts those tests
exercise aborts the child, and the test fails.  No GPU is used: every call
the tests make is refused or answered on the host."""

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "qlora_build", os.path.join(ROOT, "bit_nf4_quantized_20_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.slow
def test_abi_tests_pass_under_asan_and_ubsan():
    b = _build_module()
    try:
        runtime = b.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = b.build_sanitized()
    env = dict(os.environ,
               LD_PRELOAD=runtime,
               QLORA_ABI_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the exhaustive threshold scan exercises only numpy and the oracle
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-k", "not every_fp32"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert " passed" in res.stdout
