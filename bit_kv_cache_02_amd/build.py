"""Build libkvq.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m bit_kv_cache_02_amd.build        (or build() from Python)

Every HIP source is compiled for gfx950 only; packed-fp32 instructions are
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).  MFMA accumulators
live in ordinary VGPRs (-amdgpu-mfma-vgpr-form), so the VALU can rescale them
without AGPR copies.  Kernels run with the IEEE mode bit off and NaNs assumed
absent (-fno-honor-nans -mno-amdgpu-ieee): min/max then need no NaN
canonicalisation and fuse with DPP moves.  Fast-math stays off, so divisions,
rounding and the add-then-subtract rounding tricks keep IEEE semantics.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["kvq_host.cpp", "kvq_append.hip", "kvq_decode.hip", "kvq_prefill.hip", "kvq_dequant.hip",
           "kvq_check.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-fno-honor-nans", "-mno-amdgpu-ieee",
         "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    objs = []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("link of libkvq.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
