"""Build the gfx950 shared library libsplitzip.so in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "splitzip_kernels.hip"), os.path.join(CSRC, "splitzip_e5m2.hip"),
           os.path.join(CSRC, "splitzip_host.hip")]
HEADERS = [os.path.join(CSRC, "splitzip_internal.h"), os.path.join(CSRC, "splitzip_device.h"),
           os.path.join(ROOT, "include", "splitzip.h")]
LIB_PATH = os.path.join(HERE, "libsplitzip.so")
# streaming read / write / copy kernels that the benchmark times as the achievable ceiling
CEILING_SOURCES = [os.path.join(CSRC, "stream_ceiling.hip")]
CEILING_PATH = os.path.join(HERE, "libszceiling.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    # never let the compiler form packed-FP32 instructions.  The clang driver cannot scope an
    # -Xclang pair to the device pass (-Xarch_device refuses options that take arguments), so
    # the host pass sees the feature too and prints a notice that it does not know it; build()
    # drops exactly that notice from the compiler output.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
_HOST_PASS_NOTICE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB_PATH, extra_flags: tuple = (), verbose: bool = False) -> str:
    """Compile every HIP source of the codec for gfx950 into one shared library, and the
    streaming-ceiling kernels into their own (when building the default library)."""
    if out == LIB_PATH:
        _compile(CEILING_PATH, CEILING_SOURCES, extra_flags, verbose)
    return _compile(out, SOURCES, extra_flags, verbose)


def _compile(out: str, sources: list, extra_flags: tuple, verbose: bool) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-o", out + ".tmp", *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    text = "".join(line for line in r.stdout.splitlines(keepends=True)
                   if line.strip() != _HOST_PASS_NOTICE)
    if text:
        print(text, end="", flush=True)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)
    os.replace(out + ".tmp", out)
    return out


def is_stale(path: str = LIB_PATH) -> bool:
    srcs = CEILING_SOURCES if path == CEILING_PATH else SOURCES
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    return any(os.path.getmtime(s) > t for s in srcs + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
