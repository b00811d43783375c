"""The library's host C++ under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/host_sanitize_driver.cpp links the C-ABI layer (argument validation, workspace carving, the
page-move rules), the plane packer and the width planner, built with both sanitizers on the host
side only, against recorders in place of the device launchers; it checks the packer against the
documented bit layout, the planner's invariants, the validation codes, and that the default LYNX
bin width computed in C is k/E in fp32.  Any sanitizer finding aborts the driver.  The device
code is not instrumented and no GPU is used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "any_precision_expert_router_amd", "csrc")
ROCM = "/opt/rocm"


def _tool(path):
    return path if os.path.exists(path) else None


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    hipcc = _tool(os.path.join(ROCM, "bin", "hipcc")) or shutil.which("hipcc")
    clang = _tool(os.path.join(ROCM, "llvm", "bin", "clang++"))
    if not hipcc or not clang:
        pytest.skip("ROCm compilers not found")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    common = ["-O1", "-g", "-std=c++17"]
    # sanitizers on the host pass only: each flag goes behind -Xarch_host on the hipcc lines
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    clang_san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    objs, procs = [], []
    for src, hip in [(os.path.join(CSRC, "abi.hip"), True), (os.path.join(CSRC, "pages.hip"), True),
                     (os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), True),
                     (os.path.join(CSRC, "pack.cpp"), False), (os.path.join(CSRC, "planner.cpp"), False)]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        if hip:
            cmd = [hipcc, "--offload-arch=gfx950", *common, *inc, *host_san, "-x", "hip", "-c", src, "-o", obj]
        else:
            cmd = [clang, *common, *inc, *clang_san, "-c", src, "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate()[0].decode(errors="replace")
        assert p.returncode == 0, out
    exe = str(tmp_path / "host_sanitize_driver")
    link = [clang, *clang_san, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lpthread",
            f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    res = subprocess.run(link, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
