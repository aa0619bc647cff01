"""Build the HIP libraries in-tree for gfx950.

* ``tree_structured_copy_amd/libtkv.so`` -- the C-ABI library (host core + kernels).
* ``workloads/libtkvgen.so``           -- the seeded input generator's device fill.

Host C++ is compiled with amdclang++, HIP sources with hipcc --offload-arch=gfx950.
Packed-fp32 instructions are disabled in every device compile.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIPCC = os.path.join(ROCM, "bin", "hipcc")
CXX = os.path.join(ROCM, "llvm", "bin", "clang++")
if not os.path.exists(CXX):
    CXX = shutil.which("amdclang++") or "g++"

DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The attention kernels never produce NaN (masked scores are -inf and every
# exp / rescale guards the -inf - -inf case), so max() needs no NaN canonicalisation.
ATTN_FLAGS = ["-fno-honor-nans"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
              "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]

LIB_SOURCES = ["tree.cpp", "plan.cpp", "capi.cpp", "attn.hip", "attn_rows.hip", "attn_merge.hip", "kv.hip",
               "static_ws.hip"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if p.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out)


def _compile(src: str, obj: str, verbose: bool):
    if src.endswith(".hip"):
        extra = ATTN_FLAGS if os.path.basename(src).startswith("attn") else []
        cmd = [HIPCC] + DEVICE_FLAGS + extra + ["-I" + INCLUDE, "-I" + CSRC, "-c", src, "-o", obj]
    else:
        cmd = [CXX] + HOST_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-c", src, "-o", obj]
    _run(cmd, verbose)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> dict:
    """Compile every HIP library.  Always recompiles.  Returns the built paths."""
    os.makedirs(BUILD, exist_ok=True)
    tasks = []
    objs = []
    for s in LIB_SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(BUILD, s.replace(".", "_") + ".o")
        tasks.append((src, obj))
        objs.append(obj)
    gen_src = os.path.join(ROOT, "workloads", "gen.hip")
    gen_obj = os.path.join(BUILD, "gen_hip.o")
    tasks.append((gen_src, gen_obj))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_compile, s, o, verbose) for s, o in tasks]
        for f in futs:
            f.result()
    lib = os.path.join(HERE, "libtkv.so")
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", lib + ".tmp"], verbose)
    os.replace(lib + ".tmp", lib)
    genlib = os.path.join(ROOT, "workloads", "libtkvgen.so")
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, gen_obj, "-o", genlib + ".tmp"], verbose)
    os.replace(genlib + ".tmp", genlib)
    # host-only fork-latency benchmark, linked against the library it measures
    fb = os.path.join(HERE, "fork_bench")
    _run([CXX, "-O2", "-std=c++17", "-I" + INCLUDE, os.path.join(HERE, "fork_bench.cpp"), "-L" + HERE, "-ltkv",
          "-Wl,-rpath,$ORIGIN", "-o", fb + ".tmp"], verbose)
    os.replace(fb + ".tmp", fb)
    # native recipe replayer (loop timings), linked against the library and the HIP runtime
    rb = os.path.join(HERE, "replay_bench")
    _run([CXX] + HOST_FLAGS + ["-I" + INCLUDE, os.path.join(HERE, "replay_bench.cpp"), "-L" + HERE, "-ltkv",
                               "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath,$ORIGIN",
                               "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", rb + ".tmp"], verbose)
    os.replace(rb + ".tmp", rb)
    return {"libtkv": lib, "libtkvgen": genlib, "fork_bench": fb, "replay_bench": rb}


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
