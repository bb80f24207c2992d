"""The C ABI tests (tests/test_abi.py) again, on a build whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer: argument validation, error reporting and the struct mirrors must run clean
(any report aborts the run). CPU only; the sanitized library is built here when missing or older than
its sources."""
import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp8_quantized_attention_amd")


def _build_module():
    spec = importlib.util.spec_from_file_location("fa4_build", os.path.join(PKG, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


@pytest.mark.timeout(900)
def test_abi_under_asan_and_ubsan():
    b = _build_module()
    if not os.path.exists(b.HIPCC):
        pytest.skip("no hipcc")
    rt = b.sanitizer_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime")
    srcs = glob.glob(os.path.join(PKG, "csrc", "*")) + [os.path.join(ROOT, "include", "fa4.h")]
    if not os.path.exists(b.SAN_LIB) or os.path.getmtime(b.SAN_LIB) < max(os.path.getmtime(s) for s in srcs):
        b.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=rt, FA4_LIBRARY=b.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True, text=True)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out, out[-4000:]
