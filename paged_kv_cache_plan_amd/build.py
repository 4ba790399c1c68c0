"""Build libpka.so (the C-ABI library) in-tree for gfx950.

    python -m paged_kv_cache_plan_amd.build

* the planner and the HIP-free entry points (plain C++17) with g++;
* the rest of the C ABI (host code against the HIP runtime) with g++ and
  the HIP headers;
* the kernels with ``hipcc --offload-arch=gfx950 -O3`` and packed-fp32
  instruction selection switched off (``-Xclang -target-feature -Xclang
  -packed-fp32-ops``); decode also without the atomic optimizer;
* everything is linked into ``paged_kv_cache_plan_amd/libpka.so``.

A host-only ``libpka_planner_host.so`` (the planner and the HIP-free entry
points of ``host_api.cpp``, no HIP) is also built with AddressSanitizer and
UndefinedBehaviorSanitizer, so that the planner tests can run against it
under the host sanitizers (``tests/test_planner_sanitized.py``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpka.so")
HOST_LIB_PATH = os.path.join(HERE, "libpka_planner_host.so")
ARCH = "gfx950"
KERNELS = ["prefill.hip", "decode.hip", "mixed.hip", "merge.hip", "append.hip", "scratch.hip"]
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
# decode takes its next unit with one lane's atomic whose result is awaited
# only at the unit's end; the atomic optimizer would read it back at once
# (a wait for every load in flight)
KERNEL_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
                # the ILP-first machine scheduler: measured 1-2% faster on the
                # short causal units of a ragged prefill batch, equal elsewhere
                "prefill.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
                # the one-grid mixed kernel holds both workers: the decode
                # worker's atomic as above, and the default scheduler (with
                # the ILP-first one its 8-wave decode part spilled)
                "mixed.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpka.so)")


def _rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def _run_all(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature: harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln
                 and "is not a recognized feature for this target" not in ln]
        if p.returncode != 0:
            failed.append((cmd, "\n".join(lines)))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        msg = "\n\n".join(" ".join(c) + "\n" + t for c, t in failed)
        raise RuntimeError("libpka build failed:\n" + msg)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(os.path.dirname(HERE), "include"), "-I", CSRC]
    planner_o = os.path.join(BUILD_DIR, "planner.o")
    host_api_o = os.path.join(BUILD_DIR, "host_api.o")
    api_o = os.path.join(BUILD_DIR, "api.o")
    cmds = [["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", *inc, "-c",
             os.path.join(CSRC, "planner.cpp"), "-o", planner_o],
            ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", *inc, "-c",
             os.path.join(CSRC, "host_api.cpp"), "-o", host_api_o],
            ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(_rocm(), "include"), *inc, "-c",
             os.path.join(CSRC, "api.cpp"), "-o", api_o]]
    kobjs = []
    for k in KERNELS:
        o = os.path.join(BUILD_DIR, k.replace(".hip", ".o"))
        kobjs.append(o)
        cmds.append([hipcc, *HIP_FLAGS, *KERNEL_FLAGS.get(k, []), *inc, "-c", os.path.join(CSRC, k), "-o", o])
    _run_all(cmds, verbose)
    tmp = LIB_PATH + ".tmp"
    _run_all([[hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
               planner_o, host_api_o, api_o, *kobjs]], verbose)
    os.replace(tmp, LIB_PATH)
    build_host_sanitized(verbose)
    return LIB_PATH


def build_host_sanitized(verbose: bool = False) -> str:
    """libpka_planner_host.so: planner.cpp + host_api.cpp under ASan and
    UBSan (host code only, g++; no GPU code is built with a sanitizer)."""
    inc = ["-I", os.path.join(os.path.dirname(HERE), "include"), "-I", CSRC]
    tmp = HOST_LIB_PATH + ".tmp"
    san = ["g++", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    srcs = [os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "host_api.cpp")]
    _run_all([[*san, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", *inc, *srcs, "-o", tmp]],
             verbose)
    os.replace(tmp, HOST_LIB_PATH)
    return HOST_LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
