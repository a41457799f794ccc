"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

libkvc.so is rebuilt with its host code instrumented (device code unchanged)
and every host-side ABI test -- the validation of each entry point's
arguments, the workspace and scratch queries, the status strings -- runs
against that build in a child process that preloads the ASan runtime.  Any
out-of-bounds access, use after free or undefined behaviour in the
validation aborts the child.  A planted heap overflow in a scratch program
built with the same flags shows that the instrumentation is live.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "kv_cache_attention_kvcache_amd"))
import build as kvc_build  # noqa: E402

pytestmark = pytest.mark.slow


@pytest.fixture(scope="module")
def sanitized_lib():
    return kvc_build.build_sanitized()


def _env(lib_path):
    env = dict(os.environ)
    env.update(KVC_LIB_PATH=lib_path, LD_PRELOAD=kvc_build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env


def test_host_abi_tests_pass_under_the_sanitizers(sanitized_lib):
    check = ("import kv_cache_attention_kvcache_amd as k, ctypes, os; "
             "assert k.LIB_PATH == os.environ['KVC_LIB_PATH']; "
             "assert hasattr(ctypes.CDLL(k.LIB_PATH), '__asan_init') or 'asan' in open('/proc/self/maps').read()")
    r = subprocess.run([sys.executable, "-c", check], env=_env(sanitized_lib), cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       env=_env(sanitized_lib), cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout


def test_the_instrumentation_catches_a_planted_overflow():
    src = "#include <stdlib.h>\nint main(int c, char** v) { int* p = (int*)malloc(4 * sizeof(int)); " \
          "int r = p[c + 3]; free(p); return r & 1; }\n"
    with tempfile.TemporaryDirectory() as d:
        cpp, exe = os.path.join(d, "overflow.cpp"), os.path.join(d, "overflow")
        with open(cpp, "w") as f:
            f.write(src)
        r = subprocess.run([kvc_build.hipcc(), *kvc_build.SANITIZE_FLAGS, "-x", "c++", cpp, "-o", exe],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=60,
                           env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
        assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
