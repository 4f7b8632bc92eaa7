"""Build libkvpage.so for gfx950 in-tree with hipcc.

``python -m paged_kv_cache_07_amd.build`` (or ``build()``) compiles every HIP
source under ``csrc/`` to an object in ``_build/`` and links
``paged_kv_cache_07_amd/libkvpage.so``.  It always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvpage.so")
C_ABI_CHECK = os.path.join(ROOT, "tests", "cabi", "kvpage_c_abi_check")
SOURCES = ("api.hip", "queue.hip", "attn.hip", "merge.hip", "append.hip", "check.hip",
           "decide.hip")
ARCH = "gfx950"

# Leading kernel arguments preloaded into SGPRs at wave launch (gfx950), per
# source: each kernel's first loads then need no kernel-argument load before
# them.  The attention kernel's first-load buffers and B (3 arguments), the
# merge/finish kernels' row-metadata buffers and shape fields (9), the queue
# kernel's lengths and scan fields (5), the append kernel's lengths, free
# count, B and max_pages (4).  The compiler also emits the kernel-argument
# loads in a prologue that firmware without preloading runs instead.
PRELOAD_ARGS = {"attn.hip": 3, "merge.hip": 9, "queue.hip": 5, "append.hip": 4}

# The packed-FP32 feature is switched off: every float op stays scalar.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libkvpage.so")


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = FLAGS + list(extra_flags)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        pre = PRELOAD_ARGS.get(src)
        extra = ["-mllvm", f"-amdgpu-kernarg-preload-count={pre}"] if pre else []
        out = _run([cc, *flags, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        return obj, out

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(compile_one, SOURCES))
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    link_out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    # The standalone C ABI check (plain host code linked against the library,
    # no Python), run by the GPU tests.
    check_src = os.path.join(ROOT, "tests", "cabi", "c_abi_check.cpp")
    if os.path.exists(check_src):
        link_out += _run([cc, "-O2", "-std=c++17", "-I", INCLUDE, check_src, "-o", C_ABI_CHECK,
                          "-L", HERE, "-lkvpage", "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_07_amd"])
    if verbose:
        for _, out in results:
            if out.strip():
                print(out)
        if link_out.strip():
            print(link_out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
