"""Build libmoe_apq.so in-tree with hipcc for gfx950.

Usage: python -m any_precision_expert_router_amd.csrc.build  (or call ``build()``).
Every call recompiles (the build check must exercise the compiler each time).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_apq.so"
SOURCES = ["apq_gate_up.hip", "apq_down.hip", "apq_plain.hip", "abi.hip", "route.hip", "apq_ffn.hip",
           "probe.hip", "stats.hip", "pages.hip", "substitute.hip", "lynx.hip", "scratch.hip",
           "pack.cpp", "planner.cpp"]
ARCH = os.environ.get("MOE_APQ_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Never emit packed-fp32 VALU ops (they are not trusted on the test machines).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def build(verbose: bool = False, jobs: int = 8) -> str:
    out = os.path.join(PKG, LIB_NAME)
    # a failed build must not leave the previous library behind for tests to load
    if os.path.exists(out):
        os.remove(out)
    with tempfile.TemporaryDirectory(prefix="moe_apq_build_") as tmp:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            cmd = [hipcc(), *HIPCC_FLAGS, "-save-temps=obj", "-I", INCLUDE, "-I", HERE, "-c",
                   os.path.join(HERE, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        for p in procs:
            _wait(p)
        _check_isa(tmp)
        tmp_out = os.path.join(tmp, LIB_NAME)
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out, "-lpthread"]
        if verbose:
            print(" ".join(link), flush=True)
        res = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout.decode(errors="replace"))
        shutil.move(tmp_out, out)
    return out


def _check_isa(tmp: str) -> None:
    """Fail the build if the device assembly has a DPP wait-state hazard (see isa_check.py)."""
    import glob
    sys.path.insert(0, HERE)
    import isa_check
    total = 0
    for path in sorted(glob.glob(os.path.join(tmp, f"*-hip-amdgcn-amd-amdhsa-{ARCH}.s"))):
        n, problems = isa_check.check(path)
        total += n
        if problems:
            raise RuntimeError(f"DPP hazards in {os.path.basename(path)}:\n" + "\n".join(problems[:20]))
        spills = isa_check.scratch_users(path)
        if spills:
            raise RuntimeError(f"register spills (scratch memory) in {os.path.basename(path)}: {spills}")
        flat = isa_check.flat_accesses(path)
        if flat:
            raise RuntimeError(f"flat memory instructions in {os.path.basename(path)}: {flat[:5]}")
    if total == 0:
        raise RuntimeError("no DPP instructions found in the device assembly: ISA check did not run")


def _wait(item):
    src, proc = item
    stdout, _ = proc.communicate()
    text = stdout.decode(errors="replace")
    # hipcc's host pass does not know the packed-fp32 feature flag: harmless, filter it
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    if proc.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(lines))
    if lines:
        print("\n".join(lines), file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
