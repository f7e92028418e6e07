"""Build libtq.so (HIP kernels for gfx950 + C ABI) in place, next to this file."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtq.so")
SOURCES = ["tq_codebook.cpp", "tq_api.cpp", "tq_kernels.hip", "tq_zip.hip"]
PROBE_LIB = os.path.join(HERE, "libtqprobe.so")   # bandwidth probe used by the benchmark
PROBE_SOURCES = ["tq_probe.hip"]


def hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def _compile(sources, lib, verbose):
    srcs = [os.path.join(HERE, "csrc", s) for s in sources]
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared", "-Wall",
           # packed fp32 VALU ops are kept out of every kernel
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # the direct global->LDS copies name M0 as clobbered, which clang reports
           "-Wno-inline-asm",
           # no kernel produces or tests NaN on purpose: max/min need no NaN quieting
           "-fno-honor-nans",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
