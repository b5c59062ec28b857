"""GPU parity at the largest problem the library accepts: (N + 256) * H * d just below 2^30
elements per tensor (N = 524031, H = 16, d = 128: 2 GiB of bf16 per tensor), where byte
offsets come closest to the 32-bit range of the kernels' buffer addressing. The whole-tensor
oracle is out of reach at this size (N^2 d = 3.5e13 per head), so the oracle checks, for two
heads, chosen query rows (O, LSE, dQ against all the keys each row sees) and, under the
causal mask, the last 129 keys' dK and dV (the highest addresses; seen only by the last
rows); dV of every key enters a sum that holds at any size. The same size is used for the split-KV decode
(one query row against 524031 keys) on all heads."""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_10_amd import inputs
from parity import assert_close, bits_of, f64_of, to_device

pytestmark = pytest.mark.gpu

H, D = 16, 128
N_MAX = (1 << 30) // (H * D) - 256 - 1  # largest N with (N + 256) * H * d < 2^30


def fa():
    import exact_io_aware_10_amd as m
    return m


@pytest.mark.timeout(900)
def test_fwd_bwd_at_size_limit():
    import torch
    N, scale = N_MAX, 1 / math.sqrt(D)
    print(f"[limit fwd+bwd] B=1 N={N} H={H} d={D} bf16 causal", flush=True)
    bits = inputs.attention_inputs(1, N, H, D, "bf16", 21, with_dout=True)
    q, k, v, do = (to_device(x, "bf16") for x in bits)
    o, lse = fa().fa_fwd(q, k, v, causal=True)
    dq, dk, dv = fa().fa_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    print("  kernels done", flush=True)
    # over all keys of every head, sum_j dV_j = sum_i dO_i (each row's weights sum to one),
    # up to roundings of at most half an ulp (2^-9 relative, standard deviation 2^-9/sqrt(3)
    # of the value): of each stored dV_j, and of the weights that enter dV (their row sums
    # then differ from one by at most that much, weighting dO_i). Six standard deviations
    # of both sums bound the difference.
    f = lambda t: t[0].double()
    s_dv, s_do = f(dv).sum(0), f(do).sum(0)
    sd = 2.0 ** -9 / math.sqrt(3)
    bound = 6 * sd * (torch.linalg.vector_norm(f(dv), dim=0) +
                      torch.linalg.vector_norm(f(do), dim=0)) + 1e-3
    excess = float(((s_dv - s_do).abs() / bound).max())
    print(f"  sum dV - sum dO: at most {excess:.3f} of the bound", flush=True)
    assert excess <= 1.0
    w = lambda x: oracle.widen(x, "bf16")
    rows = np.array([0, 1, 777, 65535, 65536, N // 2, N - 129, N - 2, N - 1])
    tail = np.arange(N - 129, N)
    # 16-bit copies on the host; only the checked rows are widened
    got_o, got_dq, got_dk, got_dv = (bits_of(t) for t in (o, dq, dk, dv))
    got_lse = lse.cpu().numpy().astype(np.float64)
    for h in (0, H - 1):
        kh, vh = w(bits[1][0, :, h]), w(bits[2][0, :, h])
        ro, rl, rdq = oracle.rows(w(bits[0][0, rows, h]), kh, vh, rows, scale, True,
                                  w(bits[3][0, rows, h]))
        print(f"  head {h}: rows {list(rows)}", flush=True)
        assert_close("O rows", w(got_o[0, rows, h]), ro)
        assert_close("LSE rows", got_lse[0, h, rows], rl)
        assert_close("dQ rows", w(got_dq[0, rows, h]), rdq)
        to, tl, _ = oracle.rows(w(bits[0][0, tail, h]), kh, vh, tail, scale, True)
        tdk, tdv = oracle.tail_keys(w(bits[0][0, tail, h]), kh, vh, w(bits[3][0, tail, h]),
                                    to, tl, scale)
        assert_close("dK last keys", w(got_dk[0, tail, h]), tdk)
        assert_close("dV last keys", w(got_dv[0, tail, h]), tdv)


@pytest.mark.timeout(600)
def test_splitkv_at_size_limit():
    import torch
    Nk, scale = N_MAX, 1 / math.sqrt(D)
    print(f"[limit split-KV] B=1 Nq=1 Nk={Nk} H={H} d={D} bf16 causal", flush=True)
    qb = inputs.normal_bits((1, 1, H, D), "bf16", 30)
    kb = inputs.normal_bits((1, Nk, H, D), "bf16", 31)
    vb = inputs.normal_bits((1, Nk, H, D), "bf16", 32)
    q, k, v = (to_device(x, "bf16") for x in (qb, kb, vb))
    o, lse = fa().fa_fwd_splitkv(q, k, v, causal=True)
    torch.cuda.synchronize()
    w = lambda x: oracle.widen(x, "bf16")
    ro, rl = oracle.fwd_decode(w(qb), w(kb), w(vb), scale, True)
    assert_close("O", f64_of(o, "bf16"), ro)
    assert_close("LSE", lse.cpu().numpy().astype(np.float64), rl)


@pytest.mark.timeout(900)
def test_varlen_beyond_2gib():
    """Packed sequences past the first 2 GiB of each tensor: T = 1 100 000 tokens (lengths
    drawn as in the packed workload, seed 40), H16 d128 bf16 causal, forward and backward.
    The sequence limit applies per sequence; the sequences' base offsets are 64-bit. The
    oracle recomputes the first sequence that starts beyond 2^31 bytes (head 0) and the last
    one (head 15) as dense problems."""
    import torch
    T = 1_100_000
    lens = inputs.varlen_lengths(T, 64, 16384, 40)
    cu = inputs.cu_seqlens(lens)
    print(f"[limit varlen] T={T} nseq={len(lens)} H={H} d={D} bf16 causal", flush=True)
    bits = [inputs.normal_bits((T, H, D), "bf16", 41 + i) for i in range(4)]
    q, k, v, do = (to_device(x, "bf16") for x in bits)
    cu_d = torch.from_numpy(cu).cuda()
    o, lse = fa().fa_fwd_varlen(q, k, v, cu_d, max(lens), causal=True)
    dq, dk, dv = fa().fa_bwd_varlen(q, k, v, o, lse, do, cu_d, max(lens), causal=True)
    torch.cuda.synchronize()
    print("  kernels done", flush=True)
    start_bytes = cu[:-1].astype(np.int64) * H * D * 2
    beyond = int(np.argmax(start_bytes >= 1 << 31))
    assert start_bytes[beyond] >= 1 << 31
    scale = 1 / math.sqrt(D)
    w = lambda x: oracle.widen(x, "bf16")
    for s, h in ((beyond, 0), (len(lens) - 1, H - 1)):
        a, b = int(cu[s]), int(cu[s + 1])
        print(f"  sequence {s}: tokens {a}..{b} (byte offset {a * H * D * 2}), head {h}",
              flush=True)
        sl = lambda x: w(x[a:b, h:h + 1][None])
        qs, ks, vs, dos = (sl(x) for x in bits)
        ro, rl = oracle.fwd(qs, ks, vs, scale, True)
        rq, rk, rv = oracle.bwd(qs, ks, vs, ro, rl, dos, scale, True)
        g = lambda t: f64_of(t[a:b, h:h + 1], "bf16")[None]
        assert_close("O", g(o), ro)
        assert_close("LSE", lse[h, a:b].cpu().numpy().astype(np.float64)[None, None], rl)
        for name, t, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            assert_close(name, g(t), r)
