"""The library's host-side code built on its own with the address and undefined-behaviour
sanitizers: the codebooks, Block-GTQ allocation and encoder preparation, calibration energies
and two-stage projection (tests/native/host_check.cpp), and the C ABI's argument checks over
stub launchers (tests/native/api_check.cpp).  Host code only: no device code is built or run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["tests/native/host_check.cpp", "compressed_domain_attention_amd/csrc/tq_codebook.cpp",
           "compressed_domain_attention_amd/csrc/tq_gtq.cpp"]


def test_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(CLANG) or shutil.which(CLANG) is None:
        pytest.skip("the ROCm clang++ host compiler is not installed")
    exe = str(tmp_path / "host_check")
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include")]
    cmd += [os.path.join(ROOT, s) for s in SOURCES] + ["-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:abort_on_error=0:exitcode=3",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks passed" in r.stdout


def test_c_abi_host_code_under_sanitizers(tmp_path):
    # tq_api.cpp (argument checks, launch arguments) with the host code it calls, over stub
    # launchers (tests/native/api_stubs.cpp): tests/native/api_check.cpp calls every entry
    # point, well-formed and malformed, with extreme counts
    if not os.path.exists(CLANG):
        pytest.skip("the ROCm clang++ host compiler is not installed")
    exe = str(tmp_path / "api_check")
    srcs = ["tests/native/api_check.cpp", "tests/native/api_stubs.cpp", "compressed_domain_attention_amd/csrc/tq_api.cpp",
            "compressed_domain_attention_amd/csrc/tq_codebook.cpp", "compressed_domain_attention_amd/csrc/tq_gtq.cpp"]
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I",
           os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "compressed_domain_attention_amd", "csrc")]
    cmd += [os.path.join(ROOT, s) for s in srcs] + ["-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:abort_on_error=0:exitcode=3",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "api checks passed" in r.stdout
