"""Build liblmhead.so in-tree with hipcc for gfx950 (MI355X) only.

Each HIP source compiles to its own object in parallel; the objects link
into ``lm_head_fp32_amd/liblmhead.so``.  Flags:

* ``--offload-arch=gfx950`` -- the one target.
* ``-mcode-object-version=5`` -- loadable by the HIP runtime torch ships.
* ``-Xclang -target-feature -Xclang -packed-fp32-ops`` -- no packed FP32
  VALU instructions in device code (the host pass warns it does not know the
  feature; that is expected).
* ``-ffp-contract=off`` -- no implicit FMA contraction; every FMA in the
  kernels is written out, so the BF16 and FP32 gradient kernels compute
  bit-identical FP32 values.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liblmhead.so")
SOURCES = ("api.hip", "gemm.hip", "xent.hip", "diag.hip")

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off",
    "-Wall",
    "-Wno-unused-function",
]


# A second library for CPU tests of the C ABI's argument checks: api.hip's
# host code built with AddressSanitizer and UndefinedBehaviorSanitizer (the
# size arithmetic of every entry point runs there), linked with the normal
# objects of the other sources.  Never loaded by GPU runs.
HOSTSAN_LIB = os.path.join(HERE, "liblmhead_hostsan.so")
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblmhead.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature name; drop that note.
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_host_sanitized(verbose: bool = False) -> str:
    """liblmhead_hostsan.so (see HOSTSAN_FLAGS); needs build()'s objects."""
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: {missing} missing")
    obj = os.path.join(BUILD_DIR, "api_hostsan.o")
    cmd = [hipcc(), *COMMON_FLAGS, *HOSTSAN_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
           os.path.join(CSRC, "api.hip"), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on api.hip (sanitized host code):\n{res.stderr}")
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
            *HOSTSAN_FLAGS[:4], obj, *objs, "-o", HOSTSAN_LIB + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed (sanitized host code):\n{res.stderr}")
    os.replace(HOSTSAN_LIB + ".tmp", HOSTSAN_LIB)
    return HOSTSAN_LIB


def sanitizer_runtime() -> str:
    """The ASan runtime (it carries the UBSan handlers) that a process loading
    liblmhead_hostsan.so must preload; '' when not found."""
    import glob

    found = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib",
                                          "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else ""


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
