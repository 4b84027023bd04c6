"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed): csrc/api.hip is built with both sanitizers on its host side
only, linked with host-only stand-ins for the kernel launchers
(tests/host_sanitize/launch_stubs.cpp), and driven by
tests/host_sanitize/abi_driver.cpp through every entry point with ordinary
and extreme arguments (int32/int64 limits, sizes past any memory). Any
sanitizer report aborts the driver; every status must be the expected one."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm toolchain not found")

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    out = str(tmp_path)
    api_o, stubs_o, drv_o = (os.path.join(out, n) for n in ("api.o", "stubs.o", "drv.o"))
    # the device side of api.hip is built without sanitizers (each host flag
    # follows -Xarch_host)
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xarch_host", "-fsanitize=address,undefined",
         "-Xarch_host", "-fno-sanitize-recover=all",
         "-c", os.path.join(ROOT, "long_context_attention_paged_amd", "csrc", "api.hip"),
         "-o", api_o])
    run([CLANG, "-O1", "-g", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__",
         f"-I{ROCM}/include", "-c", os.path.join(ROOT, "tests", "host_sanitize", "launch_stubs.cpp"),
         "-o", stubs_o])
    run([CLANG, "-O1", "-g", "-std=c++17", *SAN, "-c",
         os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.cpp"), "-o", drv_o])
    exe = os.path.join(out, "abi_driver")
    run([CLANG, *SAN, drv_o, api_o, stubs_o, f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib",
         "-lamdhip64", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "0 failures" in r.stdout
