"""Build the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so with g++."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

# x86-64-v3 (AVX2 + FMA) rather than -march=native: the library is built in one place and
# run on another host.
FLAGS = ["-O3", "-march=x86-64-v3", "-std=c++17", "-shared", "-fPIC", "-pthread", "-Wall"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["g++", *FLAGS, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


ASAN_LIB = os.path.join(os.path.dirname(HERE), "_build", "asan", "liboracle_asan.so")
# AddressSanitizer and UndefinedBehaviorSanitizer build for the sanitizer test (host code
# only; loaded with gcc's sanitizer runtimes preloaded)
ASAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-shared", "-fPIC",
              "-pthread", "-Wall"]


def build_asan(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(ASAN_LIB), exist_ok=True)
    tmp = ASAN_LIB + ".tmp"
    cmd = ["g++", *ASAN_FLAGS, "-fsanitize=address,undefined", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def build_from_text(source_text: str, out_path: str) -> str:
    """Compile a (modified) copy of the oracle source to out_path; used by the mutation test."""
    src = out_path + ".cpp"
    with open(src, "w", encoding="utf-8") as f:
        f.write(source_text)
    subprocess.run(["g++", *FLAGS, src, "-o", out_path], check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
