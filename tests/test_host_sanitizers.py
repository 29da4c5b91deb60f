"""The host planner and the C ABI's validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

sp_plan.cpp and sp_api.cpp are compiled for the host only, with the sanitizers
on the host side, and linked with generated stubs for the device launchers
(every launcher returns an error; the checks never reach one) and
tests/host_check.cpp, which walks config defaults, validation of every
setting, workspace sizes over many shapes and the early rejections.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "free_block_sparse_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")
def test_host_code_under_sanitizers(tmp_path):
    decls = re.findall(r"(hipError_t\s+(?:launch_\w+|noalloc_scratch)\s*\([^;]*\));",
                       open(os.path.join(CSRC, "sp_kernels.h")).read())
    assert len(decls) >= 20
    stubs = tmp_path / "stubs.cpp"
    stubs.write_text('#include "sp_kernels.h"\nnamespace sp {\n' +
                     "\n".join(d + " { return hipErrorNotSupported; }" for d in decls) + "\n}\n")
    flags = ["-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", "-std=c++17", "-O1", "-g",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "sp_plan.cpp"), os.path.join(CSRC, "sp_api.cpp"), str(stubs),
                os.path.join(ROOT, "tests", "host_check.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        objs.append(obj)
    exe = str(tmp_path / "host_check")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failures" in r.stdout
