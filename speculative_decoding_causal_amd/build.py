"""Build ``libgdn.so`` (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_rows.hip", "gdn_prefill.hip", "gdn_chunk.hip"]
# measurement kernels for the benchmark (include/gdn_bench.h), a library of
# their own so that the step's library holds only the step
BENCH_LIB = os.path.join(HERE, "libgdn_bench.so")
BENCH_SOURCES = ["bench_ceiling.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Host code only under AddressSanitizer (device code is never instrumented):
# load the result with GDN_LIBRARY=<path> and LD_PRELOAD=<clang asan runtime>.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, out: str = LIB, asan: bool = False,
          sources=SOURCES) -> str:
    """Compile every source and link ``libgdn.so`` (or ``out``); returns its
    path.  Sources compile in parallel."""
    objs, procs = [], []
    tag = ".asan" if asan else ""
    for src in sources:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + tag + ".o")
        cmd = ["hipcc", *HIPCC_FLAGS, *(ASAN_FLAGS if asan else []), "-x", "hip", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
        objs.append(obj)
    for cmd, p in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(p.returncode, cmd)
    tmp = out + ".tmp"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC",
           *(["-Xarch_host", "-fsanitize=address", "-shared-libasan"] if asan else []),
           "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    for obj in objs:
        os.remove(obj)
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    if "--asan" in args:
        i = args.index("--asan")
        print(build(verbose="-v" in args, out=os.path.abspath(args[i + 1]), asan=True))
    else:
        print(build(verbose="-v" in args))
        print(build(verbose="-v" in args, out=BENCH_LIB, sources=BENCH_SOURCES))
