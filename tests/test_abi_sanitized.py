"""The C-ABI validation layer under host sanitizers (CPU only).

tests/test_abi.py runs again, in a child process, against libra_attn_san.so: the same library with
the host code of the C-ABI layer (ra_api.hip, noalloc.hip) compiled with AddressSanitizer and
UndefinedBehaviorSanitizer, and the kernels' objects as in the ordinary build.  The child preloads
the shared ASan runtime (the Python interpreter itself is not instrumented) and stops at the first
report.  Device code is not instrumented.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

from long_context_exact_attn_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _have_toolchain():
    try:
        B.hipcc()
        B.asan_runtime()
    except RuntimeError:
        return False
    return shutil.which("nm") is not None


pytestmark = pytest.mark.skipif(not _have_toolchain(), reason="ROCm clang with its sanitizer runtimes is required")


@pytest.fixture(scope="module")
def san_lib():
    return B.build_sanitized()


def test_sanitized_library_is_instrumented(san_lib):
    # the validation layer's host code calls into both runtimes; without them the build would be a
    # plain one under another name
    undef = subprocess.run(["nm", "-D", "--undefined-only", san_lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in undef
    assert "__ubsan_handle_" in undef


def test_abi_suite_under_host_sanitizers(san_lib):
    env = dict(os.environ)
    env.update(RA_ATTN_LIB=san_lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("from long_context_exact_attn_amd import api; import os; "
             "api.load_library(); print('loaded', os.path.realpath(api.library_path()))")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert f"loaded {os.path.realpath(san_lib)}" in r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    summary = [ln for ln in out.splitlines() if ln.strip()][-1]
    assert re.search(r"\d+ passed", summary) and "skipped" not in summary, summary
