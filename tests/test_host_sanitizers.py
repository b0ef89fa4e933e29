"""AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI's host code.

capi.cpp (argument checks) and plan.cpp (launch plans, workspace arithmetic)
are compiled for the CPU with g++ together with host stand-ins for the kernel
launchers (tests/asan/stub_launch.cpp), which read and write on host memory
every element the kernels would, and a driver (tests/asan/driver.cpp) that
calls every entry point with buffers of exactly the documented sizes, with
invalid arguments, and with sizes at the ends of the int32 range. A second
build plants a workspace shorter than the size the call is told, to show that
the sanitizer sees an overrun in this setup.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_cache_append_amd", "csrc")
ASAN = os.path.join(ROOT, "tests", "asan")
HIP_INCLUDE = "/opt/rocm/include"

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                                reason="needs g++ and the HIP headers (types only)")


def _build(out, *defines):
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", *defines, "-I" + HIP_INCLUDE,
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "capi.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ASAN, "stub_launch.cpp"), os.path.join(ASAN, "driver.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]


def _run(exe):
    # verify_asan_link_order=0: the sanitizer runtime need not come first among
    # preloaded libraries (the environment may preload its own)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)


def test_c_abi_host_code_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "mla_asan")
    _build(exe)
    r = _run(exe)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all entry points checked" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_planted_short_workspace_is_caught(tmp_path):
    exe = str(tmp_path / "mla_asan_plant")
    _build(exe, "-DPLANT_SHORT_WORKSPACE")
    r = _run(exe)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
