"""The host-side ABI layer (validation, device check, dispatch) under AddressSanitizer and
UndefinedBehaviorSanitizer: the CPU boundary tests, run in a child process against a build of
libkaio.so whose host code is instrumented (GPU code as usual), with the sanitizer runtime
preloaded.  Any report aborts the child (halt_on_error), failing this test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def asan_runtime():
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the instrumented library")
@pytest.mark.timeout(600)
def test_boundary_tests_clean_under_asan_and_ubsan():
    runtime = asan_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    from int4_group_quantized_w4a16_amd.build_lib import build_host_sanitized
    lib = build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", KAIO_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
