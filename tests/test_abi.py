"""CPU-only checks of the C-ABI library: it loads, exports every function include/fa.h
declares, and rejects bad arguments synchronously (no GPU is touched by these calls)."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import exact_io_aware_10_amd as fa
    return fa.load_library()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["fa_status_string", "fa_fwd", "fa_bwd_workspace_size", "fa_bwd", "fa_bwd_prep",
         "fa_bwd_dkdv", "fa_bwd_dq", "fa_fwd_varlen", "fa_bwd_varlen",
         "fa_fwd_splitkv_workspace_size", "fa_fwd_splitkv", "fa_fwd_fp8", "fa_merge",
         "fa_noalloc_scratch_bytes", "fa_fwd_splitkv_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    import exact_io_aware_10_amd as fa
    assert fa.fa_status_string(0) == "ok"
    assert fa.fa_status_string(1) == "invalid argument"
    assert fa.fa_status_string(2) == "unsupported configuration"
    assert fa.fa_status_string(3) == "HIP launch error"
    assert fa.fa_status_string(99) == "unknown status"


FAKE = 1 << 20  # a 16-byte aligned, never dereferenced address (checks fail before launch)


def call_fwd(lib, q=FAKE, lse=FAKE, B=1, N=8, H=1, d=64, dt=1, scale=0.125, causal=0):
    return lib.fa_fwd(q, FAKE, FAKE, FAKE, lse, B, N, H, d, dt, ctypes.c_float(scale), causal,
                      None)


def test_fwd_argument_checks(lib):
    assert call_fwd(lib, q=None) == 1
    assert call_fwd(lib, q=FAKE + 2) == 1          # misaligned
    assert call_fwd(lib, lse=None) == 1
    assert call_fwd(lib, B=-1) == 1
    assert call_fwd(lib, dt=7) == 1
    assert call_fwd(lib, scale=float("nan")) == 1
    assert call_fwd(lib, scale=float("inf")) == 1
    assert call_fwd(lib, d=96) == 2
    assert call_fwd(lib, d=256) == 2
    assert call_fwd(lib, N=1 << 20, H=64, d=128) == 2   # N*H*d beyond the offset range
    assert call_fwd(lib, B=1 << 19, N=1 << 12) == 2     # B*N tokens beyond 2^31 - 1
    # 8 * ceil(B * H / 8) * ceil(N / 128) workgroups beyond 2^31 - 1, within the other limits
    assert call_fwd(lib, B=20000, N=16000, H=1024) == 2
    assert call_fwd(lib, B=0) == 0                    # empty problem: nothing to do
    assert call_fwd(lib, q=None, N=0) == 0


def test_bwd_argument_checks(lib):
    args = [FAKE] * 10
    f = ctypes.c_float(0.1)
    bad = list(args)
    bad[9] = None  # workspace
    assert lib.fa_bwd(*bad, 1, 8, 1, 64, 1, f, 0, None) == 1
    bad = list(args)
    bad[0] = None
    assert lib.fa_bwd(*bad, 1, 8, 1, 64, 1, f, 0, None) == 1
    assert lib.fa_bwd(*args, 1, 8, 1, 80, 1, f, 0, None) == 2
    assert lib.fa_bwd(*args, 0, 8, 1, 64, 1, f, 0, None) == 0
    assert lib.fa_bwd(*args, 1 << 19, 1 << 12, 1, 64, 1, f, 0, None) == 2  # B*N > 2^31 - 1
    for stage in (lib.fa_bwd_prep, lib.fa_bwd_dkdv, lib.fa_bwd_dq):
        assert stage(*bad, 1, 8, 1, 64, 1, f, 0, None) == 1
        assert stage(*args, 1, 8, 1, 80, 1, f, 0, None) == 2
        assert stage(*args, 1, 8, 1, 64, 1, ctypes.c_float(float("nan")), 0, None) == 1

def test_varlen_argument_checks(lib):
    f = ctypes.c_float(0.1)
    a = [FAKE] * 5
    assert lib.fa_fwd_varlen(*a, None, 2, 100, 64, 2, 64, 1, f, 1, None) == 1   # no cu_seqlens
    assert lib.fa_fwd_varlen(*a, FAKE, -1, 100, 64, 2, 64, 1, f, 1, None) == 1
    assert lib.fa_fwd_varlen(*a, FAKE, 2, 100, 64, 2, 72, 1, f, 1, None) == 2
    assert lib.fa_fwd_varlen(*a, FAKE, 2, 0, 64, 2, 64, 1, f, 1, None) == 0
    # workgroups of the packed launch, 8 * ceil(num_seqs * H / 8) * ceil(max_seqlen / 128),
    # beyond 2^31 - 1
    assert lib.fa_fwd_varlen(*a, FAKE, 17000, 100, 16000, 1024, 64, 1, f, 1, None) == 2


def test_workspace_is_linear_in_sequence_length(lib):
    """The backward's scratch grows like B*H*N, never N^2: compare it against the size of
    one head's full fp16 score matrix that the guide tabulates (§3.1)."""
    import exact_io_aware_10_amd as fa
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "guide_score_matrix_sizes.json"),
                       encoding="utf-8"))
    unit = {"MB": 2 ** 20, "GB": 2 ** 30}
    for row in g["rows"]:
        n = row["N"]
        s_bytes = row["size"] * unit[row["unit"]]
        assert s_bytes == n * n * g["bytes_per_element"]  # the table is the N*N*2 closed form
        ws = fa.fa_bwd_workspace_size(1, n, 1, 128)
        assert ws == 8 * n
        assert ws * 1024 <= s_bytes or n < 4096
    assert fa.fa_bwd_workspace_size(4, 4096, 16, 128) == 8 * 4 * 16 * 4096
    assert fa.fa_bwd_workspace_size(1, 8, 1, 96) == 0


def test_bwd_varlen_argument_checks(lib):
    f = ctypes.c_float(0.1)
    a = [FAKE] * 10
    assert lib.fa_bwd_varlen(*a, None, 2, 100, 64, 2, 64, 1, f, 1, None) == 1  # no cu_seqlens
    assert lib.fa_bwd_varlen(*a, FAKE, -1, 100, 64, 2, 64, 1, f, 1, None) == 1
    assert lib.fa_bwd_varlen(*a, FAKE, 2, 100, 64, 2, 72, 1, f, 1, None) == 2
    bad = list(a)
    bad[9] = None  # workspace
    assert lib.fa_bwd_varlen(*bad, FAKE, 2, 100, 64, 2, 64, 1, f, 1, None) == 1
    assert lib.fa_bwd_varlen(*a, FAKE, 2, 0, 64, 2, 64, 1, f, 1, None) == 0


def test_splitkv_argument_checks(lib):
    f = ctypes.c_float(0.1)
    a = [FAKE] * 6  # q, k, v, o, lse, workspace

    def call(*args, ptrs=a, scale=f):
        B, Nq, Nk, H, d, dt, causal, ns = args
        return lib.fa_fwd_splitkv(*ptrs, B, Nq, Nk, H, d, dt, scale, causal, ns, None)

    assert call(-1, 1, 64, 2, 64, 1, 0, 0) == 1      # negative batch
    assert call(1, 1, 0, 2, 64, 1, 0, 0) == 1        # no keys
    assert call(1, 1, 64, 2, 64, 1, 0, -1) == 1      # negative split count
    assert call(1, 1, 64, 2, 64, 1, 0, 4097) == 1    # too many splits
    assert call(1, 1, 64, 2, 64, 7, 0, 0) == 1       # unknown dtype
    assert call(1, 1, 64, 2, 64, 1, 0, 0, scale=ctypes.c_float(float("nan"))) == 1
    assert call(1, 1, 64, 2, 72, 1, 0, 0) == 2       # head dim
    assert call(1, 1, 1 << 24, 2, 128, 1, 0, 0) == 2  # key rows beyond the offset range
    # workgroups of the partials, B * H * S * ceil(Nq / 32), beyond 2^31 - 1
    assert call(1 << 20, 1, 1 << 17, 16, 64, 1, 0, 4096) == 2
    misaligned = list(a)
    misaligned[0] = FAKE + 2
    assert call(1, 1, 64, 2, 64, 1, 0, 0, ptrs=misaligned) == 1
    no_ws = list(a)
    no_ws[5] = None
    assert call(1, 1, 64, 2, 64, 1, 0, 0, ptrs=no_ws) == 1
    assert call(0, 1, 64, 2, 64, 1, 0, 0) == 0       # empty batch: nothing to do
    assert call(1, 0, 64, 2, 64, 1, 1, 0) == 0       # no query rows: nothing to do


def test_splitkv_workspace_size(lib):
    """(d + 2) fp32 per (b, h, split, query row): linear in the query rows, and independent
    of the number of keys beyond the split count."""
    import exact_io_aware_10_amd as fa
    ws = fa.fa_fwd_splitkv_workspace_size
    assert ws(1, 1, 8192, 1, 128, 4) == 4 * (128 + 2) * 4
    assert ws(4, 3, 8192, 16, 64, 8) == 4 * 16 * 8 * 3 * (64 + 2) * 4
    assert ws(1, 1, 100, 1, 64, 50) == 4 * (64 + 2) * 4   # at most ceil(Nk / 32) ranges
    assert ws(1, 1, 1 << 20, 1, 128, 4) == ws(1, 1, 1 << 12, 1, 128, 4)
    auto = ws(4, 1, 8192, 16, 128, 0)
    assert auto > 0 and auto % (4 * 16 * (128 + 2) * 4) == 0
    assert ws(1, 1, 64, 1, 96, 0) == 0 and ws(-1, 1, 64, 1, 64, 0) == 0
    # empty problems need no workspace (and the range count of an empty problem is defined)
    assert ws(0, 1, 64, 2, 64, 0) == 0 and ws(1, 0, 64, 2, 64, 0) == 0
    assert ws(1, 1, 64, 0, 64, 0) == 0


def test_fp8_argument_checks(lib):
    c = ctypes.c_float

    def call(q=FAKE, lse=FAKE, B=1, N=8, H=1, d=64, qd=1.0, kd=1.0, vd=1.0, scale=0.125,
             causal=0):
        return lib.fa_fwd_fp8(q, FAKE, FAKE, FAKE, lse, B, N, H, d, c(qd), c(kd), c(vd),
                              c(scale), causal, None)

    assert call(q=None) == 1
    assert call(q=FAKE + 8) == 1                  # misaligned
    assert call(lse=None) == 1
    assert call(B=-1) == 1
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert call(qd=bad) == 1
        assert call(kd=bad) == 1
        assert call(vd=bad) == 1
    assert call(scale=float("nan")) == 1
    assert call(qd=1e30, kd=1e30) == 1            # exponent scale overflows
    assert call(d=96) == 2
    assert call(N=1 << 20, H=64, d=128) == 2
    assert call(B=0) == 0
    assert call(q=None, N=0) == 0


def test_merge_argument_checks(lib):
    def call(oa=FAKE, la=FAKE, op=FAKE, lp=FAKE, out=FAKE, B=1, N=8, H=1, d=64, dt=1):
        return lib.fa_merge(oa, la, op, lp, out, B, N, H, d, dt, None)

    assert call(oa=None) == 1
    assert call(op=None) == 1
    assert call(la=None) == 1
    assert call(lp=FAKE + 2) == 1               # misaligned lse
    assert call(out=FAKE + 8) == 1              # misaligned output
    assert call(B=-1) == 1
    assert call(dt=5) == 1
    assert call(d=96) == 2
    assert call(N=1 << 20, H=64, d=128) == 2
    assert call(B=1 << 22, N=1 << 12) == 2      # workgroups beyond 2^31 - 1
    assert call(out=None, B=0) == 0             # empty: nothing to do


def test_splitkv_noalloc_argument_checks(lib):
    """The allocation-free split-KV entry point checks its arguments like fa_fwd_splitkv,
    before it touches any device; requests whose partials exceed the scratch array are
    refused as unsupported."""
    f = ctypes.c_float(0.1)
    call = lambda q=FAKE, B=1, Nq=1, Nk=8, H=1, d=64, dt=1, splits=0: \
        lib.fa_fwd_splitkv_noalloc(q, FAKE, FAKE, FAKE, FAKE, B, Nq, Nk, H, d, dt, f, 0,
                                   splits, None)
    lib.fa_noalloc_scratch_bytes.restype = ctypes.c_size_t
    assert lib.fa_noalloc_scratch_bytes() == 8 << 20
    assert call(q=None) == 1
    assert call(dt=5) == 1
    assert call(Nk=0) == 1
    assert call(d=96) == 2
    assert call(B=0) == 0
    # 16 heads x 4096 ranges x 130 fp32 values per partial row: 34 MB, beyond 8 MiB
    lib.fa_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    assert lib.fa_fwd_splitkv_workspace_size(1, 1, 500000, 16, 128, 4096) > 8 << 20
    assert call(Nk=500000, H=16, d=128, splits=4096) == 2
