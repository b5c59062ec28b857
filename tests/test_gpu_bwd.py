"""GPU parity of fa_bwd against the fp64 oracle's gradients (called through the C ABI via
the ctypes binding). The GPU backward consumes the GPU forward's O and LSE; the oracle's
gradients are the exact ones, so the comparison covers the whole training path."""
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


def run(B, N, H, d, dtype, causal, seed, scale=None):
    import torch
    print(f"[bwd] B={B} N={N} H={H} d={d} {dtype} causal={causal} seed={seed} scale={scale}",
          flush=True)
    bits = inputs.attention_inputs(B, N, H, d, dtype, seed, with_dout=True)
    q, k, v, do = (to_device(x, dtype) for x in bits)
    o, lse = fa().fa_fwd(q, k, v, causal=causal, softmax_scale=scale)
    dq, dk, dv = fa().fa_bwd(q, k, v, o, lse, do, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return bits, [f64_of(t, dtype) for t in (dq, dk, dv)]


def oracle_grads(bits, dtype, scale, causal):
    q, k, v, do = (oracle.widen(x, dtype) for x in bits)
    o, lse = oracle.fwd(q, k, v, scale, causal)
    return oracle.bwd(q, k, v, o, lse, do, scale, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,N,H", [(1, 1, 1), (2, 17, 3), (1, 130, 2), (2, 300, 1), (1, 777, 1)])
def test_bwd_small(B, N, H, d, dtype, causal):
    scale = 1 / math.sqrt(d)
    bits, got = run(B, N, H, d, dtype, causal, seed=3 * N + d)
    ref = oracle_grads(bits, dtype, scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert_close(name, g, r)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.3])
def test_bwd_scale_values(scale):
    for causal in (False, True):
        bits, got = run(1, 150, 2, 64, "bf16", causal, seed=5, scale=scale)
        ref = oracle_grads(bits, "bf16", scale, causal)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert_close(name, g, r, rtol=2.0 ** -7)


def test_bwd_deterministic():
    import torch
    bits = inputs.attention_inputs(2, 520, 4, 128, "bf16", 9, with_dout=True)
    q, k, v, do = (to_device(x, "bf16") for x in bits)
    o, lse = fa().fa_fwd(q, k, v, causal=True)
    g1 = fa().fa_bwd(q, k, v, o, lse, do, causal=True)
    g2 = fa().fa_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bwd_workload_sampled():
    """B4 H16 N4096 d128 bf16 causal forward + backward; the oracle recomputes three
    complete (b, h) slices (each an independent problem) and every gradient is checked
    there; the gradient invariants are checked on every slice."""
    wl = inputs.WORKLOADS["train_causal_fwd_bwd"]
    scale = 1 / math.sqrt(wl.d)
    bits, got = run(wl.B, wl.N, wl.H, wl.d, wl.dtype, wl.causal, seed=0)
    dq, dk, dv = got
    w = lambda x: oracle.widen(x, wl.dtype)
    for b, h in [(0, 0), (wl.B - 1, wl.H - 1), (2, 7)]:
        sl = lambda x: x[b:b + 1, :, h:h + 1, :]
        ref = oracle_grads([sl(x) for x in bits], wl.dtype, scale, wl.causal)
        print(f"  slice b={b} h={h}", flush=True)
        for name, g, r in zip(("dQ", "dK", "dV"), (sl(dq), sl(dk), sl(dv)), ref):
            assert_close(name, g, r)
    # every dS row sums to zero -> sum_j dK_j = 0; P rows sum to one -> sum_j dV_j = sum_i dO_i
    do = w(bits[3])
    sum_dk = dk.sum(axis=1)
    sum_dv = dv.sum(axis=1)
    sum_do = do.sum(axis=1)
    assert np.max(np.abs(sum_dk)) < 0.5, np.max(np.abs(sum_dk))
    assert np.max(np.abs(sum_dv - sum_do)) < 0.5, np.max(np.abs(sum_dv - sum_do))


def run_varlen_bwd(lens, H, d, dtype, causal, seed):
    import torch
    cu = inputs.cu_seqlens(lens)
    T = int(cu[-1])
    print(f"[bwd varlen] nseq={len(lens)} T={T} H={H} d={d} {dtype} causal={causal}",
          flush=True)
    bits = [inputs.normal_bits((T, H, d), dtype, seed + i) for i in range(4)]
    q, k, v, do = (to_device(x, dtype) for x in bits)
    cu_d = torch.from_numpy(cu).cuda()
    o, lse = fa().fa_fwd_varlen(q, k, v, cu_d, max(lens), causal=causal)
    dq, dk, dv = fa().fa_bwd_varlen(q, k, v, o, lse, do, cu_d, max(lens), causal=causal)
    torch.cuda.synchronize()
    return cu, bits, [f64_of(t, dtype) for t in (dq, dk, dv)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_small(d, causal):
    lens = [5, 1, 130, 64, 300, 0, 17]
    cu, bits, got = run_varlen_bwd(lens, 3, d, "bf16", causal, seed=21)
    q, k, v, do = (oracle.widen(x, "bf16") for x in bits)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.fwd_varlen(q, k, v, cu, scale, causal)
    ref = oracle.bwd_varlen(q, k, v, o, lse, do, cu, scale, causal)
    # short causal sequences (lengths 1, 5, 17) give gradients up to |x| ~ 5, where bf16
    # output rounding alone costs up to 2^-9 |x|: two half-ulps of relative slack
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert_close(name, g, r, rtol=2.0 ** -7)


def test_bwd_varlen_workload_sampled():
    """The packed causal workload (T = 131072, H16, d128) through forward and backward; the
    oracle recomputes the shortest sequence, a mid-length one and the last (truncated) one,
    one head each, as complete problems."""
    wl = inputs.WORKLOADS["varlen_causal_fwd"]
    lens = inputs.varlen_lengths(wl.N, *wl.len_range, seed=0)
    cu, bits, got = run_varlen_bwd(lens, wl.H, wl.d, wl.dtype, wl.causal, seed=0)
    w = lambda x: oracle.widen(x, wl.dtype)
    scale = 1 / math.sqrt(wl.d)
    order = np.argsort(lens)
    for s, h in sorted({(int(order[0]), 0), (int(order[len(lens) // 3]), 7),
                        (len(lens) - 1, wl.H - 1)}):
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: x[a:b, h:h + 1, :][None]
        q, k, v, do = (w(sl(x)) for x in bits)
        o, lse = oracle.fwd(q, k, v, scale, wl.causal)
        ref = oracle.bwd(q, k, v, o, lse, do, scale, wl.causal)
        print(f"  seq {s} len {b - a} head {h}", flush=True)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert_close(name, g[a:b, h:h + 1][None], r)


def test_varlen_debug_checks(monkeypatch):
    """With FA_DEBUG set, both packed entry points copy cu_seqlens to the host and reject a
    malformed array (cu[0] != 0, a decrease, or a last entry other than the token count)
    with FA_ERR_INVALID_ARG before launching anything; a well-formed array gives the same
    bits as without the check. FA_DEBUG=0 switches the check off again."""
    import torch
    lens = [70, 1, 129, 0, 33]
    cu = inputs.cu_seqlens(lens)
    T, H, d = int(cu[-1]), 2, 64
    print(f"[varlen FA_DEBUG] lens={lens} H={H} d={d} bf16 causal", flush=True)
    bits = [inputs.normal_bits((T, H, d), "bf16", 60 + i) for i in range(4)]
    q, k, v, do = (to_device(x, "bf16") for x in bits)

    def run(c):
        o, lse = fa().fa_fwd_varlen(q, k, v, c, max(lens), causal=True)
        return (o, lse, *fa().fa_bwd_varlen(q, k, v, o, lse, do, c, max(lens), causal=True))

    monkeypatch.delenv("FA_DEBUG", raising=False)
    want = run(torch.from_numpy(cu).cuda())
    monkeypatch.setenv("FA_DEBUG", "1")
    got = run(torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    for w, g in zip(want, got):
        assert torch.equal(w, g)
    o, lse = want[0], want[1]
    bad = [cu.copy() for _ in range(3)]
    bad[0][0] = 1                      # does not start at 0
    bad[1][2], bad[1][3] = cu[3], cu[2]  # decreases
    bad[2][-1] = T - 1                 # does not end at the token count
    for c in bad:
        c_d = torch.from_numpy(c).cuda()
        with pytest.raises(fa().FAError) as e:
            fa().fa_fwd_varlen(q, k, v, c_d, max(lens), causal=True)
        assert e.value.code == 1
        with pytest.raises(fa().FAError) as e:
            fa().fa_bwd_varlen(q, k, v, o, lse, do, c_d, max(lens), causal=True)
        assert e.value.code == 1
    monkeypatch.setenv("FA_DEBUG", "0")
    again = run(torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    assert all(torch.equal(w, g) for w, g in zip(want, again))
