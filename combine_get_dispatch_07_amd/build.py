"""Build libmoe_ep.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python combine_get_dispatch_07_amd/build.py        # or __graft_entry__.build()

Flags that matter for results:
* ``-ffp-contract=off`` (plus ``#pragma clang fp contract(off)`` in the
  kernels): combine multiplies then adds, never a fused multiply-add.
* ``-fhip-fp32-correctly-rounded-divide-sqrt``: the FP8 scale and the x / s
  quotients are IEEE correctly rounded divisions.
* ``-target-feature -packed-fp32-ops``: no packed fp32 instructions.
* fp32 denormals are kept (no flush-to-zero flag).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from typing import Iterable, Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRC = os.path.join(PKG_DIR, "csrc", "moe_ep.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_ep.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")
    return path


def build(out: Optional[str] = None, defines: Iterable[str] = (), extra_flags: Iterable[str] = (),
          verbose: bool = False) -> str:
    """Compile the library; returns the path of the built .so."""
    out = out or LIB_PATH
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", *[f"-D{d}" for d in defines], *extra_flags,
           SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in res.stderr.splitlines() if noise not in l and "ignoring feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "c_abi_client")


def build_c_client(out: Optional[str] = None) -> str:
    """Compile tests/c_abi_client.c, a plain C11 consumer of the C ABI (gcc, no HIP compiler),
    linked against the in-tree libmoe_ep.so and the ROCm HIP runtime."""
    out = out or C_CLIENT
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
           f"-I{rocm}/include", C_CLIENT_SRC, "-o", out + ".tmp", f"-L{PKG_DIR}", "-lmoe_ep", f"-L{rocm}/lib",
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../combine_get_dispatch_07_amd", f"-Wl,-rpath,{rocm}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(out + ".tmp", out)
    return out


HBM_CEILING_SRC = os.path.join(ROOT, "hbm_ceiling.hip")
HBM_CEILING = os.path.join(ROOT, "hbm_ceiling")
LAUNCH_FLOOR_SRC = os.path.join(ROOT, "launch_floor.hip")
LAUNCH_FLOOR = os.path.join(ROOT, "liblaunch_floor.so")


def _probe(src: str, out: str, extra) -> str:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *extra, src, "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(out + ".tmp", out)
    return out


def build_hbm_ceiling(out: Optional[str] = None) -> str:
    """Compile hbm_ceiling.hip (beside bench.py), the streaming-bandwidth probe bench.py reports
    beside the kernels' fraction of peak (a standalone HIP program, not part of the library)."""
    return _probe(HBM_CEILING_SRC, out or HBM_CEILING, [])


def build_launch_floor(out: Optional[str] = None) -> str:
    """Compile launch_floor.hip (beside bench.py): the shortest one-wave launches, which bench.py
    times next to the decode launches (a measurement aid, not part of the library)."""
    return _probe(LAUNCH_FLOOR_SRC, out or LAUNCH_FLOOR, ["-shared", "-fPIC"])


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_client())
    print(build_hbm_ceiling())
    print(build_launch_floor())
