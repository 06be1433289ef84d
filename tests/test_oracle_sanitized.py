"""The oracle's pins run against an AddressSanitizer + UndefinedBehaviorSanitizer
build of oracle.c (host code only; gcc), in a child process that preloads the
ASan runtime.  Any out-of-bounds access, use after free or undefined
behaviour in the oracle aborts that run.  A second child makes a call with an
output buffer that is too small, to show that the sanitizer is live."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import build as obuild  # noqa: E402


@pytest.fixture(scope="module")
def san_env():
    try:
        obuild.build(sanitize=True)
        env = obuild.sanitizer_env()
    except (OSError, subprocess.CalledProcessError) as e:  # no gcc / no ASan runtime
        pytest.skip(f"sanitizer build unavailable: {e}")
    if not os.path.exists(env["LD_PRELOAD"]):
        pytest.skip("gcc's ASan runtime is not installed")
    return env


def test_pins_pass_under_asan_and_ubsan(san_env):
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests",
                                                                     "test_oracle_pins.py"),
                        "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=san_env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout


def test_sanitizer_is_live(san_env):
    code = (
        "import ctypes, numpy as np, oracle\n"
        "assert oracle._LIB_PATH.endswith('liboracle_san.so')\n"
        "lib = oracle._load()\n"
        "v = np.ones(64)\n"
        "out = np.empty(8, dtype=np.uint16)\n"     # 56 elements short
        "lib.orc_round_bf16_array(v.ctypes.data, 64, out.ctypes.data)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=san_env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr
