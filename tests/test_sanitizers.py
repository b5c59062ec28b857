"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The fp64 oracle is built with g++ -fsanitize=address,undefined (oracle/build.py,
build_asan) and its whole pin suite runs against that build in a child process that
preloads gcc's sanitizer runtimes. The C ABI's host code (the synchronous argument checks
of every entry point) is built with clang's sanitizers (exact_io_aware_10_amd/build.py,
variant host_asan) and tests/test_abi.py runs against it in a child process that preloads
clang's ASan runtime. A report of either sanitizer aborts the child and fails the test.
Each build is redone when one of its sources is newer than it."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _stale(lib, sources):
    return not os.path.exists(lib) or any(os.path.getmtime(s) > os.path.getmtime(lib)
                                          for s in sources)


def _run(args, env_extra, log_stem):
    env = dict(os.environ)
    env.update(env_extra)
    log = os.path.join(ROOT, "_build", log_stem)
    os.makedirs(os.path.dirname(log), exist_ok=True)
    for f in glob.glob(log + ".*"):
        os.remove(f)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:abort_on_error=1:log_path={log}"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={log}"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *args], cwd=ROOT, env=env, capture_output=True, text=True)
    reports = "".join(open(f, encoding="utf-8", errors="replace").read()
                      for f in glob.glob(log + ".*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports)
    return r.stdout


def test_oracle_pins_under_asan_ubsan():
    from oracle import build
    if _stale(build.ASAN_LIB, [build.SRC]):
        build.build_asan()
    lib = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                         text=True).stdout.strip()
    ub = subprocess.run(["g++", "-print-file-name=libubsan.so"], capture_output=True,
                        text=True).stdout.strip()
    if not (os.path.isabs(lib) and os.path.isabs(ub)):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    out = _run(["tests/test_oracle_pins.py"],
               {"ORACLE_LIB": build.ASAN_LIB, "LD_PRELOAD": f"{lib}:{ub}"}, "asan_oracle")
    assert " passed" in out


def test_abi_checks_under_asan_ubsan():
    from exact_io_aware_10_amd import build
    lib = build.variant_path("host_asan")
    srcs = build.sources() + glob.glob(os.path.join(build.CSRC, "*.h")) + [
        os.path.join(ROOT, "include", "fa.h"), build.__file__]
    if _stale(lib, srcs):
        build.build_variant("host_asan")
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    out = _run(["tests/test_abi.py"], {"FA_LIBRARY": lib, "LD_PRELOAD": rt[0]}, "asan_abi")
    assert " passed" in out
