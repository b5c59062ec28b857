"""Build libfa_mi355x.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object in parallel, then linked into
exact_io_aware_10_amd/libfa_mi355x.so. Usage: python -m exact_io_aware_10_amd.build [-v]

Environment (optional): FA_EXTRA_CFLAGS (extra hipcc flags for every file), FA_LIB_OUT
(output library path), FA_BUILD_DIR (object directory).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.environ.get("FA_BUILD_DIR") or os.path.join(ROOT, "_build")
LIB = os.environ.get("FA_LIB_OUT") or os.path.join(HERE, "libfa_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-result",
] + os.environ.get("FA_EXTRA_CFLAGS", "").split()

# Per-file flags. The dQ kernel's softmax-side VALU work reads the S and dP accumulators
# directly, so its MFMA results are kept in VGPRs (in AGPRs they would be copied back for
# every tile); the dK/dV kernel keeps the default (its 128 gradient accumulators live in
# AGPRs).
# The forward kernel's row max reads MFMA results; without NaN semantics fmaxf needs no
# canonicalizing instruction per input (NaN inputs still propagate through exp and the sums).
FILE_FLAGS = {
    "fa_bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fa_fwd.hip": ["-fno-honor-nans"],
    "fa_fwd_fp8.hip": ["-fno-honor-nans"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
