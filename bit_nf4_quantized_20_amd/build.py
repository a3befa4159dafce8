"""Builds libqlora.so (the HIP kernels + C ABI) in-tree for gfx950, and the
bench's measurement-support library libqlora_bench.so (bench_csrc/).

    python bit_nf4_quantized_20_amd/build.py             # libqlora.so, libqlora_bench.so
    python bit_nf4_quantized_20_amd/build.py --sanitize  # + _build/libqlora_san.so

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
BENCH_CSRC = os.path.join(HERE, "bench_csrc")
BENCH_LIB = os.path.join(HERE, "libqlora_bench.so")
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
    _link(sorted(glob.glob(os.path.join(CSRC, "*.hip"))), LIB, verbose)
    _link(sorted(glob.glob(os.path.join(BENCH_CSRC, "*.hip"))), BENCH_LIB, verbose, prefix="bench_")
    return LIB


def _link(sources, lib, verbose, prefix=""):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in sources:
        obj = os.path.join(objdir, prefix + os.path.basename(src) + ".o")
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
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, lib)


# Host-side sanitizers for the validation layer: the C-ABI entry points'
# argument checks (qlora_api.hip) are compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host pass only (each -fsanitize= behind
# -Xarch_host; the device code is built as usual) and linked with the other
# objects of the regular build into a separate library, which the CPU ABI
# tests load with the sanitizer runtime preloaded.
SAN_LIB = os.path.join(HERE, "_build", "libqlora_san.so")
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime matching hipcc's compiler."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def build_sanitized(verbose: bool = False) -> str:
    build(verbose)
    objdir = os.path.join(HERE, "_build")
    api = os.path.join(CSRC, "qlora_api.hip")
    san_obj = os.path.join(objdir, "qlora_api.hip.san.o")
    cmd = [hipcc(), *flags(), *SAN_HOST_FLAGS, "-c", api, "-o", san_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {api} (sanitized):\n{res.stderr}")
    objs = [os.path.join(objdir, os.path.basename(src) + ".o")
            for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))) if src != api]
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, san_obj, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + res.stderr)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
