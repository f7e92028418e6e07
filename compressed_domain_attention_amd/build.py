"""Build libtq.so (HIP kernels for gfx950 + C ABI) in place, next to this file."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtq.so")
SOURCES = ["tq_codebook.cpp", "tq_api.cpp", "tq_gtq.cpp", "tq_kernels.hip", "tq_zip.hip", "tq_gtq.hip", "tq_dense.hip"]
PROBE_LIB = os.path.join(HERE, "libtqprobe.so")   # bandwidth probe used by the benchmark
PROBE_SOURCES = ["tq_probe.hip"]


def hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


# Sources compiled on their own with extra flags, then linked in.  The codec's attention
# kernel keeps its matrix-core accumulators in ordinary vector registers: its rarely taken
# rescale branch otherwise costs a copy of every accumulator out of the accumulation
# registers on each loop iteration.
SEPARATE = {"tq_zip.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def _flags():
    return ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-Wall",
            # packed fp32 VALU ops are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # the direct global->LDS copies name M0 as clobbered, which clang reports
            "-Wno-inline-asm",
            # no kernel produces or tests NaN on purpose: max/min need no NaN quieting
            "-fno-honor-nans",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def _messages(res):
    noise = "packed-fp32-ops"
    return [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]


def _compile(sources, lib, verbose):
    """Each source to an object (in parallel), then one shared library."""
    tag = ".tmp%d" % os.getpid()
    jobs = []
    for s in sources:
        obj = os.path.join(HERE, "%s%s.o" % (s.replace(".", "_"), tag))
        cmd = [hipcc(), *_flags(), *SEPARATE.get(s, []), "-c", os.path.join(HERE, "csrc", s), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    tmp = lib + tag
    try:
        failed = []
        for obj, p in jobs:
            out, err = p.communicate()
            res = subprocess.CompletedProcess(p.args, p.returncode, out, err)
            if p.returncode != 0:
                failed += _messages(res)
            elif verbose and _messages(res):
                print("\n".join(_messages(res)), flush=True)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        cmd = [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *[o for o, _ in jobs], "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + "\n".join(_messages(res)))
    finally:
        for obj, _ in jobs:
            if os.path.exists(obj):
                os.remove(obj)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
