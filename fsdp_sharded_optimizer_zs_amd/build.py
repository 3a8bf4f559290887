"""Build libzs.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzs.so")
SOURCES = ("zs_api.cpp", "zs_pipeline.cpp", "zs_ckpt.cpp", "zs_host.cpp", "zs_step.hip",
           "zs_move.hip", "zs_diag.hip", "zs_static.hip")

# -ffp-contract=off: no fused multiply-add in the step's arithmetic;
# correctly rounded fp32 divide and sqrt (the HIP default, stated);
# packed fp32 VALU ops disabled; symbols hidden except the C ABI.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libzs")


def build(out: str = LIB, defines: tuple = (), verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + FLAGS + ["-D" + d for d in defines] + ["-x", "hip"] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building %s" % out)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
