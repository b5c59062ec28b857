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
            assert_close(name, g, r, ulps=1)


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


def test_bwd_workload():
    """B4 H16 N4096 d128 bf16 causal forward + backward: every element of O, LSE, dQ, dK and
    dV against the oracle (its forward, then its backward from its own O and LSE), with the
    tolerances also per (b, h) slice; the gradient invariants on every slice."""
    import torch
    wl = inputs.WORKLOADS["train_causal_fwd_bwd"]
    scale = 1 / math.sqrt(wl.d)
    print(f"[bwd workload] B={wl.B} N={wl.N} H={wl.H} d={wl.d} causal={wl.causal}", flush=True)
    bits = inputs.attention_inputs(wl.B, wl.N, wl.H, wl.d, wl.dtype, 0, with_dout=True)
    q, k, v, do = (to_device(x, wl.dtype) for x in bits)
    o, lse = fa().fa_fwd(q, k, v, causal=wl.causal)
    grads = fa().fa_bwd(q, k, v, o, lse, do, causal=wl.causal)
    torch.cuda.synchronize()
    got = {"O": f64_of(o, wl.dtype), "LSE": lse.cpu().numpy().astype(np.float64)}
    got.update(zip(("dQ", "dK", "dV"), (f64_of(t, wl.dtype) for t in grads)))
    rq, rk, rv, rdo = (oracle.widen(x, wl.dtype) for x in bits)
    ro, rlse = oracle.fwd(rq, rk, rv, scale, wl.causal)
    ref = {"O": ro, "LSE": rlse}
    ref.update(zip(("dQ", "dK", "dV"), oracle.bwd(rq, rk, rv, ro, rlse, rdo, scale, wl.causal)))
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert_close(name, got[name], ref[name])
        for b in range(wl.B):
            for h in range(wl.H):
                sl = (b, h) if name == "LSE" else (b, slice(None), h)
                assert_close(f"{name}[{b},{h}]", got[name][sl], ref[name][sl], quiet=True)
    # every dS row sums to zero -> sum_j dK_j = 0; P rows sum to one -> sum_j dV_j = sum_i dO_i
    dk, dv = got["dK"], got["dV"]
    sum_dk = dk.sum(axis=1)
    sum_dv = dv.sum(axis=1)
    sum_do = rdo.sum(axis=1)
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
    # short causal sequences (lengths 1, 5, 17) give gradients of magnitude 4 and more, where
    # the bf16 output's own rounding costs up to 2^-6 = 0.0156 of the 2e-2 bound: one
    # half-ulp of the output is added to the bound (parity.py)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert_close(name, g, r, ulps=1)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_many(d, causal):
    """Many packed sequences of mixed lengths (one to five 128-key blocks) over five heads:
    the (sequence, head) pairs do not fill whole rounds of eight, so the last round of the
    packed work order has empty slots in both gradient kernels."""
    lens = inputs.varlen_lengths(6000, 17, 600, seed=7)
    assert (len(lens) * 5) % 8 != 0
    cu, bits, got = run_varlen_bwd(lens, 5, d, "bf16", causal, seed=23)
    q, k, v, do = (oracle.widen(x, "bf16") for x in bits)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.fwd_varlen(q, k, v, cu, scale, causal)
    ref = oracle.bwd_varlen(q, k, v, o, lse, do, cu, scale, causal)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert_close(name, g, r)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_max_seqlen_truncates(causal):
    """A sequence longer than max_seqlen is processed as its first max_seqlen tokens, in the
    forward and in both gradient kernels, and the other sequences are unaffected: each
    sequence's first min(L, max_seqlen) rows of O, LSE, dQ, dK and dV against the oracle on
    that many tokens alone."""
    import torch
    lens, mx, H, d, dt = [100, 700, 40, 301], 300, 2, 64, "bf16"
    cu = inputs.cu_seqlens(lens)
    T = int(cu[-1])
    print(f"[varlen truncation] lens={lens} max_seqlen={mx} causal={causal}", flush=True)
    bits = [inputs.normal_bits((T, H, d), dt, 31 + i) for i in range(4)]
    q, k, v, do = (to_device(x, dt) for x in bits)
    cu_d = torch.from_numpy(cu).cuda()
    o, lse = fa().fa_fwd_varlen(q, k, v, cu_d, mx, causal=causal)
    dq, dk, dv = fa().fa_bwd_varlen(q, k, v, o, lse, do, cu_d, mx, causal=causal)
    torch.cuda.synchronize()
    got = [f64_of(t, dt) for t in (o, dq, dk, dv)]
    lse = lse.cpu().numpy().astype(np.float64)
    w = [oracle.widen(x, dt) for x in bits]
    scale = 1 / math.sqrt(d)
    for s, L in enumerate(lens):
        a, n = int(cu[s]), min(L, mx)
        sq, sk, sv, sdo = (x[a:a + n][None] for x in w)
        ro, rlse = oracle.fwd(sq, sk, sv, scale, causal)
        ref = oracle.bwd(sq, sk, sv, ro, rlse, sdo, scale, causal)
        assert_close(f"O seq {s}", got[0][a:a + n], ro[0])
        assert_close(f"LSE seq {s}", lse[:, a:a + n], rlse[0])
        for name, g, r in zip(("dQ", "dK", "dV"), got[1:], ref):
            assert_close(f"{name} seq {s}", g[a:a + n], r[0])


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_stages_match_fa_bwd(causal):
    """The three stages that fa_bwd runs, called one by one through their own entry points
    with one workspace (row terms, then dK/dV, then dQ; the order a caller may change between
    the last two), give fa_bwd's gradients bit for bit, and each stage writes only its own
    outputs: gradient buffers a stage does not own keep a planted bit pattern."""
    import torch
    m = fa()
    B, N, H, d, dt = 2, 700, 3, 128, "bf16"
    print(f"[bwd stages] B={B} N={N} H={H} d={d} causal={causal}", flush=True)
    bits = inputs.attention_inputs(B, N, H, d, dt, 61, with_dout=True)
    q, k, v, do = (to_device(x, dt) for x in bits)
    o, lse = m.fa_fwd(q, k, v, causal=causal)
    ref = m.fa_bwd(q, k, v, o, lse, do, causal=causal)
    ws = torch.empty(max(m.fa_bwd_workspace_size(B, N, H, d), 16), dtype=torch.uint8,
                     device=q.device)
    fill = lambda: torch.full_like(q, 0).view(torch.int16).fill_(0x7fc1).view(q.dtype)
    for order in ("dkdv_first", "dq_first"):
        grads = (fill(), fill(), fill())
        m.fa_bwd_prep(q, k, v, o, lse, do, causal=causal, workspace=ws, grads=grads)
        torch.cuda.synchronize()
        for g in grads:  # the row terms go to the workspace only
            assert torch.all(g.view(torch.int16) == 0x7fc1)
        stages = [(m.fa_bwd_dkdv, (1, 2)), (m.fa_bwd_dq, (0,))]
        if order == "dq_first":
            stages.reverse()
        written = set()
        for stage, own in stages:
            stage(q, k, v, o, lse, do, causal=causal, workspace=ws, grads=grads)
            torch.cuda.synchronize()
            written.update(own)
            for i, g in enumerate(grads):
                if i not in written:
                    assert torch.all(g.view(torch.int16) == 0x7fc1), (order, i)
        for i, (g, r) in enumerate(zip(grads, ref)):
            assert torch.equal(g.view(torch.int16), r.view(torch.int16)), (order, i)


def test_bwd_varlen_workload():
    """The packed causal workload (T = 131072, H16, d128) through forward and backward; the
    oracle recomputes every sequence on two heads (the first and the last) as complete
    problems: dQ, dK and dV of every token there, with the tolerances per sequence too."""
    wl = inputs.WORKLOADS["varlen_causal_fwd"]
    lens = inputs.varlen_lengths(wl.N, *wl.len_range, seed=0)
    cu, bits, got = run_varlen_bwd(lens, wl.H, wl.d, wl.dtype, wl.causal, seed=0)
    w = lambda x: oracle.widen(x, wl.dtype)
    scale = 1 / math.sqrt(wl.d)
    heads = [0, wl.H - 1]
    q, k, v, do = (w(np.ascontiguousarray(x[:, heads])) for x in bits)
    o, lse = oracle.fwd_varlen(q, k, v, cu, scale, wl.causal)
    ref = oracle.bwd_varlen(q, k, v, o, lse, do, cu, scale, wl.causal)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g = g[:, heads]
        assert_close(f"{name} heads {heads}", g, r)
        for s in range(len(lens)):
            a, b = int(cu[s]), int(cu[s + 1])
            assert_close(f"{name} seq {s} (len {b - a})", g[a:b], r[a:b], quiet=True)


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
