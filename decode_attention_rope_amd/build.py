"""Build libbgtq.so (HIP, gfx950) in-tree with hipcc.

    python -m decode_attention_rope_amd.build

Every source is compiled with floating-point contraction off (the energy,
allocation and quantize kernels must reproduce an exact rounding sequence;
decode uses explicit fused multiply-adds), IEEE-correct fp32 division and
square root, denormals kept, and packed-fp32 instruction selection disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libbgtq.so")
SOURCES = ["api.cpp", "lloyd_max.cpp", "kernels.hip", "diagnostic.hip"]

ARCH = os.environ.get("BGTQ_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Wall", "-Wno-unused-result",
]
DEVICE = [
    f"--offload-arch={ARCH}",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="bgtq_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *COMMON, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".hip"):
                cmd[1:1] = ["-x", "hip", *DEVICE]
            _run(cmd, verbose)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libbgtq.so")
        _run([cc, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib], verbose)
        shutil.move(tmp_lib, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
