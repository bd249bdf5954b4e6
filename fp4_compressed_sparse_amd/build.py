"""Build the CSA2 HIP library in-tree: fp4_compressed_sparse_amd/libcsa2.so.

hipcc cross-compiles for gfx950 without a GPU.  Every kernel source is
compiled into one translation unit (csrc/api.hip includes the others), so
the device flag word has a single definition without relocatable device
code.  Flags: -ffp-contract=off keeps every float32 multiply and add of the
pinned score order separate (fused forms are written explicitly where they
are exact); packed-fp32 instructions are disabled; the atomic optimizer is
off (every atomic in the kernels is already issued by one lane).

A second library, libcsa2_checked.so, is the same source built with
-DCSA2_CHECKED: scrambled workgroup order (CSA2_WG_ORDER) and device-side
index checks that raise CSA2_FLAG_CHECK.  The tests run it beside the
product library and require identical results.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libcsa2.so")
CHECKED_LIB = os.path.join(HERE, "libcsa2_checked.so")
SOURCES = ["api.hip", "quantize.hip", "index.hip", "headmax.hip", "attend.hip", "common.hpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep single-lane atomics as written: the wave-level atomic rewrite
    # reads the result back at once, which would stall the full scan's
    # work-counter prefetch
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc"),
]


def _variants():
    return [(LIB, []), (CHECKED_LIB, ["-DCSA2_CHECKED"])]


def build(verbose=False):
    """Compile libcsa2.so and libcsa2_checked.so (two hipcc processes at once)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = []
    for lib, extra in _variants():
        cmd = [hipcc] + FLAGS + extra + [os.path.join(HERE, "csrc", "api.hip"), "-o", lib + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((lib, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for lib, p in jobs:
        out = p.communicate()[0]
        msgs = [l for l in out.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l]
        if p.returncode != 0:
            sys.stderr.write("\n".join(msgs) + "\n")
            failed.append(os.path.basename(lib))
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("hipcc failed building " + ", ".join(failed))
    for lib, _ in jobs:
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
