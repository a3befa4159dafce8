"""Builds libqlora.so (the HIP kernels + C ABI) in-tree for gfx950.

    python bit_nf4_quantized_20_amd/build.py

hipcc cross-compiles for gfx950 without a GPU.  Every HIP source is compiled
with packed fp32 instructions disabled (-Xclang -target-feature -Xclang
-packed-fp32-ops), IEEE fp32 division and square root, and no fast-math.
"""

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqlora.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fno-fast-math", "-ffp-contract=fast",
        "-munsafe-fp-atomics",
        "-Wall", "-Wno-unused-function",
    ]


def build(verbose: bool = False) -> str:
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in sources:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc(), *flags(), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in res.stderr.splitlines()
                         if "packed-fp32-ops" not in l and "unused during compilation" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
        if errs.strip() and verbose:
            print(errs, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
