"""The library's host code (validation, workspace arithmetic, launch plans,
error paths) built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven by tests/sanitize/abi_driver.cpp on the CPU.  The sanitizers apply to
host code only; the kernels' objects are linked as built."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "token_level_head_block_amd", "csrc")
OBJ = os.path.join(ROOT, "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not present")
def test_host_code_under_asan_and_ubsan(tmp_path):
    from token_level_head_block_amd import _build
    kernels = [os.path.splitext(f)[0] for f in _build.SOURCES if f.endswith(".hip")]
    if not all(os.path.exists(os.path.join(OBJ, k + ".o")) for k in kernels):
        _build.build()
    api = str(tmp_path / "mhla_api_san.o")
    host_san = []
    for flag in SAN:          # sanitizers for the host pass only
        host_san += ["-Xarch_host", flag]
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "mhla_api.cpp"), "-o", api] + host_san
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    drv = str(tmp_path / "abi_driver.o")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
                        "-o", drv] + SAN, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "abi_driver")
    objs = [drv, api] + [os.path.join(OBJ, k + ".o") for k in kernels]
    r = subprocess.run([CLANG, "-o", exe] + objs + SAN + ["-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("MHLA_FAIL_ALLOC", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.startswith("OK"), r.stdout
