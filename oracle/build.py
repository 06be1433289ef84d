"""Build the FP64 CPU oracle (test infrastructure) with gcc.

Compiles ``oracle.c`` into ``liboracle.so`` beside it.  Plain C99 + POSIX
threads; no fast-math and no floating-point contraction, so every sum is the
sequential one the source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# The same source built with AddressSanitizer and UndefinedBehaviorSanitizer
# (host code only; any report aborts).  A process that loads it must preload
# gcc's ASan runtime (sanitizer_env() gives the environment).
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g", "-O1"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    cmd = (["gcc", "-std=gnu99"] + (SAN_FLAGS if sanitize else ["-O2"]) +
           ["-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-fno-fast-math", "-Wall",
            "-Wextra", SRC, "-o", out + ".tmp", "-lm"])
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def sanitizer_env() -> dict:
    """Environment for a Python process that loads the sanitized oracle:
    gcc's ASan runtime preloaded (it must come first), leak checks off (the
    interpreter's own allocations are not this library's), and the oracle
    package pointed at liboracle_san.so."""
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["LMH_ORACLE_LIB"] = SAN_LIB
    return env


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
    sys.exit(0)
