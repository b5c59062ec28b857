"""Build libfa_mi355x.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object in parallel, then linked into
exact_io_aware_10_amd/libfa_mi355x.so. Usage: python -m exact_io_aware_10_amd.build [-v]
[--variant lds_poison|host_asan]

Environment (optional): FA_EXTRA_CFLAGS (extra hipcc flags for every file), FA_LIB_OUT
(output library path), FA_BUILD_DIR (object directory).

Debug variants (build_variant), each its own library (variant_path: under
exact_io_aware_10_amd/variants/, the sanitizer build under the object directory), loaded by
setting FA_LIBRARY to its path:
  lds_poison  every kernel fills its LDS with NaN patterns before use (-DFA_LDS_POISON)
  host_asan   host code built with AddressSanitizer and UndefinedBehaviorSanitizer (the
              argument checks of the C ABI; device code unchanged), for a process that
              preloads clang's ASan runtime
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
# every tile); the dK/dV kernel needs no such flag (at 256 registers per wave the compiler
# already keeps all its accumulators in VGPRs).
# The forward kernel's row max reads MFMA results; without NaN semantics fmaxf needs no
# canonicalizing instruction per input (NaN inputs still propagate through exp and the sums).
# Scheduler choices, each measured against the default (B4 H16 N8192 d128, alternating
# processes): the memory-clause strategy for dQ (-0.9%), the register-pressure trackers for
# dK/dV (-0.5%; also one spilled register instead of ten under the mask), the ILP strategy
# for the row-term kernel (-4%); the forward keeps the default (ILP +0.7%, memory clauses +9%).
FILE_FLAGS = {
    "fa_bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form",
                      "-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
    "fa_bwd_dkdv.hip": ["-mllvm", "-amdgpu-use-amdgpu-trackers"],
    "fa_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "fa_fwd.hip": ["-fno-honor-nans"],
    "fa_fwd_fp8.hip": ["-fno-honor-nans"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, verbose, build_dir=BUILD_DIR, extra=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o",
           obj]
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


VARIANTS = {
    "lds_poison": (["-DFA_LDS_POISON"], []),
    "host_asan": (["-Xarch_host", "-fsanitize=address",
                   "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer", "-g"],
                  ["-Xarch_host", "-fsanitize=address",
                   "-Xarch_host", "-fsanitize=undefined"]),
}
VARIANT_DIR = os.path.join(HERE, "variants")


def variant_path(name: str) -> str:
    # the sanitizer build serves CPU tests only and stays with the objects
    d = os.path.join(BUILD_DIR, name) if name == "host_asan" else VARIANT_DIR
    return os.path.join(d, f"libfa_mi355x_{name}.so")


def build_variant(name: str, verbose: bool = False, jobs: int = 8) -> str:
    """Build the debug variant `name` of the library (see the module docstring)."""
    cflags, ldflags = VARIANTS[name]
    bdir = os.path.join(BUILD_DIR, name)
    os.makedirs(bdir, exist_ok=True)
    os.makedirs(os.path.dirname(variant_path(name)), exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, bdir, cflags), sources()))
    out = variant_path(name)
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *ldflags, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if "--variant" in sys.argv:
        print(build_variant(sys.argv[sys.argv.index("--variant") + 1], verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
