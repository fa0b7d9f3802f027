"""Build libfp8q.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Run as `python -m blockwise_scaled_fp8_quant_amd.build` or through
`__graft_entry__.build()`.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8q.so")
SOURCES = ["quant.hip", "gemm.hip", "attention.hip", "moe.hip", "abi.cpp"]
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # no contraction: every fused multiply-add in the kernels is written out
    "-ffp-contract=off",
    # keep packed fp32 instructions out of the generated device code.  The
    # driver cannot forward -Xclang through -Xarch_device, so the host pass
    # sees the feature too and prints that it does not know it (HOST_NOTICE,
    # filtered below); the device pass applies it.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs, where the per-block scale FMAs can read them
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


HOST_NOTICE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def _compile(src, build_dir):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    err = "\n".join(l for l in r.stderr.splitlines() if l.strip() != HOST_NOTICE)
    return obj, err


def build(verbose=False):
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
