"""Build the HIP library ``lib/librmsnorm_bi.so`` for gfx950 (in-tree).

hipcc cross-compiles without a GPU.  Flags that matter for the results:
  -ffp-contract=off   a*b+c stays two rounded operations unless fmaf is
                      written out (the canonical dweight order relies on it)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed FP32 instructions are generated
The host-only plan code is compiled with g++ (it has no HIP dependency).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
from typing import List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "librmsnorm_bi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result", f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", f"-I{CSRC}"]

SOURCES_HIP = ["kernels.hip", "abi.cpp", "linear.hip", "linear_abi.cpp", "embedding.hip",
               "embedding_abi.cpp", "ceiling.hip"]
SOURCES_CXX = ["plan.cpp"]


def _run(cmd: List[str]):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ...")
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "not a recognized feature for this target"
    for line in (r.stdout + r.stderr).splitlines():
        if line.strip() and noise not in line:
            sys.stderr.write(line + "\n")


def build(verbose: bool = False, save_temps: Optional[str] = None) -> str:
    """Compile every source and link the shared library; returns its path."""
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    cmds = []
    for src in SOURCES_HIP:
        obj = os.path.join(obj_dir, src + ".o")
        cmd = [HIPCC, *HIP_FLAGS]
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        if save_temps:
            os.makedirs(save_temps, exist_ok=True)
            cmd += ["-save-temps=obj"]
            obj = os.path.join(save_temps, src + ".o")
        cmds.append((cmd + ["-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in SOURCES_CXX:
        obj = os.path.join(obj_dir, src + ".o")
        cmds.append((["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    if verbose:
        for cmd, _ in cmds:
            print(" ".join(cmd))
    # the translation units are independent: compile them side by side
    # (-save-temps writes shared intermediate names, so it stays serial)
    workers = 1 if save_temps else min(len(cmds), os.cpu_count() or 1, 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        list(pool.map(_run, [cmd for cmd, _ in cmds]))
    objs = [obj for _, obj in cmds]
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv,
                save_temps=(sys.argv[sys.argv.index("--save-temps") + 1]
                            if "--save-temps" in sys.argv else None)))
