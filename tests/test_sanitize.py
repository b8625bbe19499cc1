"""Host-side safety tier: the C ABI layer and the launch index arithmetic under
AddressSanitizer and UndefinedBehaviorSanitizer. tests/abi_sanitize.cpp drives every
entry point (kernel launchers replaced by recorders, so no GPU is touched) and
enumerates the workgroup placement and the LDS tile swizzle; any out-of-bounds access,
overflow or undefined behaviour aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.fail("g++ and the ROCm headers are needed for the sanitizer build")
    exe = str(tmp_path / "abi_sanitize")
    # host code only: g++, no .hip source on this line
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", os.path.join(ROOT, "tests", "abi_sanitize.cpp"),
           os.path.join(ROOT, "io_aware_softmax_tiled_amd", "csrc", "fa_api.cpp"),
           "-o", exe, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ALL OK" in r.stdout, (r.stdout[-4000:], r.stderr[-4000:])
