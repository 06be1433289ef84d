"""The C ABI's argument checks (tests/test_boundary.py: fake pointers, no
GPU) run against liblmhead_hostsan.so -- api.hip's host code built with
AddressSanitizer + UndefinedBehaviorSanitizer, the kernels as in the normal
build -- in a child process that preloads the ASan runtime.  An out-of-bounds
access or undefined behaviour in the host code of any entry point (a signed
overflow in its size arithmetic, for one) aborts that run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from lm_head_fp32_amd import build as hbuild  # noqa: E402

_CHILD = (
    "import sys\n"
    "sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})\n"
    "import lm_head_fp32_amd as lmh\n"
    "lmh._LIB_PATH = {lib!r}\n"
    "import pytest\n"
    "sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', {test!r}]))\n")


@pytest.fixture(scope="module")
def san():
    if not os.path.exists(hbuild.HOSTSAN_LIB):
        pytest.skip("liblmhead_hostsan.so not built (build() makes it)")
    rt = hbuild.sanitizer_runtime()
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env


def test_boundary_checks_pass_under_asan_and_ubsan(san):
    code = _CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=hbuild.HOSTSAN_LIB,
                         test=os.path.join(ROOT, "tests", "test_boundary.py"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=san, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_library_is_instrumented():
    if not os.path.exists(hbuild.HOSTSAN_LIB):
        pytest.skip("liblmhead_hostsan.so not built")
    nm = shutil.which("nm")
    if not nm:
        pytest.skip("nm not found")
    out = subprocess.run([nm, "-D", "--undefined-only", hbuild.HOSTSAN_LIB], capture_output=True,
                         text=True, check=True).stdout
    assert "__asan_" in out and "__ubsan_handle_" in out
