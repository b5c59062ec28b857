"""GPU parity of fa_fwd and fa_fwd_varlen against the fp64 oracle (called through the C ABI
via the ctypes binding)."""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_10_amd import inputs
from parity import assert_close, to_device, f64_of

pytestmark = pytest.mark.gpu


def fa():
    import exact_io_aware_10_amd as m
    return m


def run_dense(B, N, H, d, dtype, causal, seed, scale=None):
    print(f"[fwd] B={B} N={N} H={H} d={d} {dtype} causal={causal} seed={seed} scale={scale}",
          flush=True)
    qb, kb, vb = inputs.attention_inputs(B, N, H, d, dtype, seed)
    q, k, v = (to_device(x, dtype) for x in (qb, kb, vb))
    o, lse = fa().fa_fwd(q, k, v, causal=causal, softmax_scale=scale)
    import torch
    torch.cuda.synchronize()
    return (qb, kb, vb), f64_of(o, dtype), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,N,H", [(1, 1, 1), (2, 17, 3), (1, 64, 1), (2, 129, 2), (1, 300, 2),
                                   (1, 1000, 1)])
def test_fwd_small(B, N, H, d, dtype, causal):
    scale = 1 / math.sqrt(d)
    (qb, kb, vb), o, lse = run_dense(B, N, H, d, dtype, causal, seed=N + d)
    w = lambda x: oracle.widen(x, dtype)
    ro, rlse = oracle.fwd(w(qb), w(kb), w(vb), scale, causal)
    assert_close("O", o, ro)
    assert_close("LSE", lse, rlse)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.5])
def test_fwd_scale_values(scale):
    B, N, H, d, dtype = 1, 200, 2, 64, "bf16"
    for causal in (False, True):
        (qb, kb, vb), o, lse = run_dense(B, N, H, d, dtype, causal, 7, scale)
        w = lambda x: oracle.widen(x, dtype)
        ro, rlse = oracle.fwd(w(qb), w(kb), w(vb), scale, causal)
        assert_close("O", o, ro)
        assert_close("LSE", lse, rlse)


def test_fwd_deterministic():
    import torch
    qb, kb, vb = inputs.attention_inputs(2, 700, 4, 128, "bf16", 3)
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    o1, l1 = fa().fa_fwd(q, k, v, causal=True)
    o2, l2 = fa().fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


# ---- the five workloads, every output element against the oracle (each call of the oracle
# covers the whole tensor: every (b, h) slice is an independent problem it computes in full)

def _check_all(qb, kb, vb, o, lse, dtype, causal):
    """Every element of O and LSE, plus the tolerances per (b, h) slice (so that a slice
    computed wrongly cannot hide in the averages of the others)."""
    d = qb.shape[-1]
    w = lambda x: oracle.widen(x, dtype)
    ro, rlse = oracle.fwd(w(qb), w(kb), w(vb), 1 / math.sqrt(d), causal)
    assert_close("O", o, ro)
    assert_close("LSE", lse, rlse)
    B, H = qb.shape[0], qb.shape[2]
    for b in range(B):
        for h in range(H):
            assert_close(f"O[{b},:,{h}]", o[b, :, h], ro[b, :, h], quiet=True)
            assert_close(f"LSE[{b},{h}]", lse[b, h], rlse[b, h], quiet=True)


@pytest.mark.parametrize("name", ["single_head_fwd", "gpt2_small_causal_fwd", "long_seq_fwd"])
def test_fwd_workload(name):
    wl = inputs.WORKLOADS[name]
    (qb, kb, vb), o, lse = run_dense(wl.B, wl.N, wl.H, wl.d, wl.dtype, wl.causal, seed=0)
    _check_all(qb, kb, vb, o, lse, wl.dtype, wl.causal)


# Dense launches without the mask and with at least two query blocks per CU (512 on MI355X)
# take the stream form: one workgroup per CU walking its blocks as one stream of key/value
# tiles. Items of one tile, of two tiles with a ragged last one, of 17 blocks x 33 tiles,
# d = 64 and fp16; every slice checked.
@pytest.mark.parametrize("B,N,H,d,dtype", [(32, 100, 16, 128, "bf16"), (32, 200, 16, 64, "f16"),
                                           (2, 4196, 16, 128, "bf16"), (4, 2048, 16, 64, "bf16")])
def test_fwd_stream(B, N, H, d, dtype):
    (qb, kb, vb), o, lse = run_dense(B, N, H, d, dtype, False, seed=N + H)
    _check_all(qb, kb, vb, o, lse, dtype, False)


# Causal dense launches of many query blocks (512 to 1200 items, more than the CUs), dealt
# longest first over whole slices per XCD: ragged four-tile blocks, a head count that does not
# split evenly over the XCDs (H = 30 at B = 2) and a ragged N at d = 128; every slice checked.
@pytest.mark.parametrize("B,N,H,d,dtype", [(32, 200, 16, 64, "bf16"), (1, 6400, 32, 64, "bf16"),
                                           (2, 5000, 30, 128, "bf16")])
def test_fwd_causal_many_blocks(B, N, H, d, dtype):
    (qb, kb, vb), o, lse = run_dense(B, N, H, d, dtype, True, seed=N + H + 1)
    _check_all(qb, kb, vb, o, lse, dtype, True)


def run_varlen(lens, H, d, dtype, causal, seed, max_seqlen=None):
    import torch
    cu = inputs.cu_seqlens(lens)
    T = int(cu[-1])
    print(f"[varlen] nseq={len(lens)} T={T} H={H} d={d} {dtype} causal={causal}", flush=True)
    qb, kb, vb = (inputs.normal_bits((T, H, d), dtype, seed + i) for i in range(3))
    q, k, v = (to_device(x, dtype) for x in (qb, kb, vb))
    cu_d = torch.from_numpy(cu).cuda()
    o, lse = fa().fa_fwd_varlen(q, k, v, cu_d, max_seqlen or max(lens), causal=causal)
    torch.cuda.synchronize()
    return cu, (qb, kb, vb), f64_of(o, dtype), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_varlen_small(d, causal):
    lens = [5, 1, 130, 64, 300, 0, 17]
    cu, (qb, kb, vb), o, lse = run_varlen(lens, 3, d, "bf16", causal, seed=11)
    w = lambda x: oracle.widen(x, "bf16")
    ro, rlse = oracle.fwd_varlen(w(qb), w(kb), w(vb), cu, 1 / math.sqrt(d), causal)
    assert_close("O", o, ro)
    assert_close("LSE", lse, rlse)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_varlen_many(d, causal):
    """Many packed sequences of mixed lengths (one to three 256-row query blocks) over five
    heads: the (sequence, head) pairs do not fill whole rounds of eight, so the last round
    of the packed work order has empty slots."""
    lens = inputs.varlen_lengths(6000, 17, 600, seed=7)
    assert (len(lens) * 5) % 8 != 0
    cu, (qb, kb, vb), o, lse = run_varlen(lens, 5, d, "bf16", causal, seed=13)
    w = lambda x: oracle.widen(x, "bf16")
    ro, rlse = oracle.fwd_varlen(w(qb), w(kb), w(vb), cu, 1 / math.sqrt(d), causal)
    assert_close("O", o, ro)
    assert_close("LSE", lse, rlse)


def test_fwd_varlen_workload():
    """The packed causal workload (T = 131072, H16, d128): every (sequence, head) pair
    against the oracle, and the tolerances per sequence."""
    wl = inputs.WORKLOADS["varlen_causal_fwd"]
    lens = inputs.varlen_lengths(wl.N, *wl.len_range, seed=0)
    cu, (qb, kb, vb), o, lse = run_varlen(lens, wl.H, wl.d, wl.dtype, wl.causal, seed=0)
    w = lambda x: oracle.widen(x, wl.dtype)
    ro, rlse = oracle.fwd_varlen(w(qb), w(kb), w(vb), cu, 1 / math.sqrt(wl.d), wl.causal)
    assert_close("O", o, ro)
    assert_close("LSE", lse, rlse)
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        assert_close(f"O seq {s} (len {b - a})", o[a:b], ro[a:b])
        assert_close(f"LSE seq {s}", lse[:, a:b], rlse[:, a:b])
