"""The ABI tests again, against the library whose host API unit is built
under AddressSanitizer and UndefinedBehaviorSanitizer (host code only; CPU
only: no test there launches a kernel).  A sanitizer report ends the child
process with a non-zero status and fails this test."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_egm_build_sanitized", os.path.join(ROOT, "dense_gemm_epilogue_fp16_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_under_host_sanitizers():
    b = _build_module()
    try:
        b.hipcc()
        runtime = b.host_sanitizer_runtime()
    except RuntimeError as exc:
        pytest.skip(f"no sanitizer toolchain: {exc}")
    lib = b.build_host_sanitized()
    env = dict(os.environ)
    env.update(EGM_LIBRARY=lib, LD_PRELOAD=runtime,
               # the interpreter itself leaks by design; the library's own
               # errors (overflows, use after free, UB) still halt the run
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-x", "-q",
                        "-s", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    tail = "\n".join(r.stdout.splitlines()[-40:])
    assert r.returncode == 0, f"sanitized ABI run failed ({r.returncode}):\n{tail}"
    assert "passed" in tail and "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout, tail
