"""Pins for the fp64 CPU oracle: values the pages print, closed forms, invariants, brute
force and independent cross-checks. None of these re-types the oracle's own formulas."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from exact_io_aware_10_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _one_row_problem(scores, values):
    """q = [1], k_j = scores[j], scale 1, d = 1: s_j = scores[j]."""
    n = len(scores)
    q = np.zeros((1, n, 1, 1))
    q[0, 0, 0, 0] = 1.0
    k = np.asarray(scores, dtype=np.float64).reshape(1, n, 1, 1)
    v = np.asarray(values, dtype=np.float64).reshape(1, n, 1, 1)
    return q, k, v


# ---------------------------------------------------------------- worked examples (pages)

def test_narration_example_one_shot():
    g = _golden("narration_online_softmax_example.json")
    scores = [math.log(1), math.log(2), math.log(4), math.log(3)]
    q, k, v = _one_row_problem(scores, g["values"])
    o, lse = oracle.fwd(q, k, v, scale=1.0, causal=False)
    assert o[0, 0, 0, 0] == pytest.approx(g["one_shot"]["output"], abs=1e-12)
    assert o[0, 0, 0, 0] == pytest.approx(
        g["one_shot"]["weighted_sum"] / g["one_shot"]["weight_total"], abs=1e-12)
    # the row's log-sum-exp is ln(sum of exponentiated scores) = ln 10
    assert lse[0, 0, 0] == pytest.approx(math.log(g["one_shot"]["weight_total"]), abs=1e-12)


@pytest.mark.parametrize("form", ["deferred", "normalized"])
def test_narration_example_blocked(form):
    g = _golden("narration_online_softmax_example.json")
    scores = [math.log(1), math.log(2), math.log(4), math.log(3)]
    q, k, v = _one_row_problem(scores, g["values"])
    o, lse, trace = oracle.fwd_blocked(q, k, v, 1.0, False, block_q=1,
                                       block_k=g["block_size"], form=form)
    for jb, step in enumerate(g["after_block"]):
        m, l, state = trace[jb]
        assert math.exp(m) == pytest.approx(step["block_max_exp"], abs=1e-12)
        assert l == pytest.approx(step["denominator"], abs=1e-12)
        numer = state if form == "deferred" else state * l
        assert numer == pytest.approx(step["numerator"], abs=1e-12)
    assert math.exp(trace[0, 0] - trace[1, 0]) == pytest.approx(
        g["after_block"][1]["rescale_of_previous"], abs=1e-12)
    assert o[0, 0, 0, 0] == pytest.approx(g["output"], abs=1e-12)
    assert lse[0, 0, 0] == pytest.approx(math.log(10.0), abs=1e-12)


@pytest.mark.parametrize("form", ["deferred", "normalized"])
def test_guide_example(form):
    g = _golden("guide_online_softmax_example.json")
    tol = g["abs_tol"]
    x = g["scores"]
    n = len(x)
    # q = e1, k_j = x_j e1, V = identity: O row = softmax row
    q = np.zeros((1, n, 1, n))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, n, 1, n))
    k[0, :, 0, 0] = x
    v = np.eye(n).reshape(1, n, 1, n)
    o, lse = oracle.fwd(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0, 0, 0], g["one_shot"]["softmax"], atol=tol)
    m = g["one_shot"]["max"]
    assert math.exp(lse[0, 0, 0] - m) == pytest.approx(g["one_shot"]["sum"], abs=tol)
    ob, lseb, trace = oracle.fwd_blocked(q, k, v, 1.0, False, 1, g["block_size"], form)
    on = g["online"]
    assert trace[0, 0] == pytest.approx(on["m1"], abs=1e-12)
    assert trace[0, 1] == pytest.approx(on["l1"], abs=tol)
    assert trace[0, 1] * math.exp(trace[0, 0] - trace[1, 0]) == pytest.approx(
        on["rescaled_l1"], abs=tol)
    assert trace[1, 0] == pytest.approx(on["m2"], abs=1e-12)
    assert trace[1, 1] == pytest.approx(on["l2"], abs=tol)
    np.testing.assert_allclose(ob[0, 0, 0], g["one_shot"]["softmax"], atol=tol)


# ---------------------------------------------------------------- identities

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    """softmax rows sum to 1 (guide §2.4): with V = 1, every output entry is 1."""
    B, N, H, d = 2, 37, 3, 8
    q, k = _rand((B, N, H, d), 1), _rand((B, N, H, d), 2) * 3.0
    v = np.ones((B, N, H, d))
    o, _ = oracle.fwd(q, k, v, 0.7, causal)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("form", ["deferred", "normalized"])
def test_blocked_equals_unblocked(causal, form):
    """The tiled online algorithm reaches the plain definition (guide §5.2 exactness note)."""
    B, N, H, d = 1, 100, 2, 16
    q, k, v = _rand((B, N, H, d), 3), _rand((B, N, H, d), 4), _rand((B, N, H, d), 5)
    o_ref, lse_ref = oracle.fwd(q, k, v, 0.5, causal)
    for bk in (1, 2, 3, 7, 64, N):
        for bq in (1, 7, 64):
            o, lse, _ = oracle.fwd_blocked(q, k, v, 0.5, causal, bq, bk, form)
            scale_o = np.max(np.abs(o_ref))
            assert np.max(np.abs(o - o_ref)) <= 1e-12 * scale_o, (bk, bq)
            assert np.max(np.abs(lse - lse_ref) / np.maximum(1, np.abs(lse_ref))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    """Subtracting a per-row constant leaves softmax unchanged (guide §2.4): adding u to
    every key shifts each row's scores by scale*<q_i,u>, so O is unchanged and LSE_i
    moves by exactly that amount."""
    B, N, H, d = 1, 29, 2, 8
    scale = 0.8
    q, k, v = _rand((B, N, H, d), 6), _rand((B, N, H, d), 7), _rand((B, N, H, d), 8)
    u = _rand((d,), 9) * 2
    o1, lse1 = oracle.fwd(q, k, v, scale, causal)
    o2, lse2 = oracle.fwd(q, k + u, v, scale, causal)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    shift = scale * np.einsum("bnhd,d->bhn", q, u)
    np.testing.assert_allclose(lse2 - lse1, shift, atol=1e-12)


# ---------------------------------------------------------------- brute force and special cases

def _brute(q, k, v, scale, causal):
    """Direct per-row evaluation with exactly rounded sums (math.fsum), pure Python."""
    B, N, H, d = q.shape
    o = np.zeros((B, N, H, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                js = range(i + 1) if causal else range(N)
                s = [scale * math.fsum(float(q[b, i, h, c]) * float(k[b, j, h, c])
                                       for c in range(d)) for j in js]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for c in range(d):
                    o[b, i, h, c] = math.fsum(wj * float(v[b, j, h, c])
                                              for wj, j in zip(w, js)) / tot
                lse[b, h, i] = mx + math.log(tot)
    return o, lse


@pytest.mark.parametrize("N", [1, 2, 5, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_small(N, causal):
    B, H, d = 2, 2, 3
    q, k, v = _rand((B, N, H, d), 10 + N), _rand((B, N, H, d), 20 + N), _rand((B, N, H, d), 30)
    o, lse = oracle.fwd(q, k, v, 0.9, causal)
    ob, lseb = _brute(q, k, v, 0.9, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-13)


def test_special_cases():
    B, H, d = 1, 2, 4
    # N = 1: the only key gets all the weight; LSE is its score
    q, k, v = _rand((B, 1, H, d), 40), _rand((B, 1, H, d), 41), _rand((B, 1, H, d), 42)
    o, lse = oracle.fwd(q, k, v, 0.3, False)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse[0, :, 0], 0.3 * np.sum(q[0, 0] * k[0, 0], axis=-1), atol=1e-14)
    # causal row 0 sees only key 0
    N = 9
    q, k, v = _rand((B, N, H, d), 43), _rand((B, N, H, d), 44), _rand((B, N, H, d), 45)
    o, lse = oracle.fwd(q, k, v, 0.3, True)
    np.testing.assert_allclose(o[:, 0], v[:, 0], atol=1e-15)
    # K = 0: uniform weights over the visible keys, LSE = ln |J(i)|
    for causal in (False, True):
        o, lse = oracle.fwd(q, np.zeros_like(k), v, 0.3, causal)
        for i in range(N):
            cnt = i + 1 if causal else N
            np.testing.assert_allclose(o[0, i], v[0, :cnt].mean(axis=0), atol=1e-14)
            np.testing.assert_allclose(lse[0, :, i], math.log(cnt), atol=1e-14)


# ---------------------------------------------------------------- gradients

def _torch_reference(q, k, v, dout, scale, causal):
    """softmax(scale QK^T + mask) V in float64 on the CPU with autograd (stored P)."""
    import torch
    t = [torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True)
         for x in (q, k, v)]
    s = scale * (t[0] @ t[1].transpose(-1, -2))
    if causal:
        n = s.shape[-1]
        mask = torch.ones(n, n, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = p @ t[2]
    lse = torch.logsumexp(s, dim=-1)
    o.backward(torch.tensor(dout.transpose(0, 2, 1, 3)))
    back = lambda x: x.detach().numpy().transpose(0, 2, 1, 3)
    return back(o), lse.detach().numpy(), back(t[0].grad), back(t[1].grad), back(t[2].grad)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_autograd(causal):
    B, N, H, d = 2, 23, 2, 8
    scale = 1 / math.sqrt(d)
    q, k, v, do = (_rand((B, N, H, d), 50 + i) for i in range(4))
    o, lse = oracle.fwd(q, k, v, scale, causal)
    dq, dk, dv = oracle.bwd(q, k, v, o, lse, do, scale, causal)
    ro, rlse, rdq, rdk, rdv = _torch_reference(q, k, v, do, scale, causal)
    for a, b in ((o, ro), (lse, rlse), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    """dL/dX for L = sum(O * dO) by central differences, h = 1e-6."""
    B, N, H, d = 1, 6, 1, 3
    scale = 0.7
    q, k, v, do = (_rand((B, N, H, d), 60 + i) for i in range(4))
    o, lse = oracle.fwd(q, k, v, scale, causal)
    grads = oracle.bwd(q, k, v, o, lse, do, scale, causal)
    h = 1e-6

    def loss(qq, kk, vv):
        oo, _ = oracle.fwd(qq, kk, vv, scale, causal, nthreads=1)
        return float(np.sum(oo * do))

    for which, g in zip(range(3), grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            lp = loss(*args)
            args[which][idx] -= 2 * h
            lm = loss(*args)
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1e-3, np.max(np.abs(g)))
        assert err <= 1e-6, (which, err)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    """Each row of dS sums to zero (softmax Jacobian), so sum_j dK_j = 0; P rows sum to
    one, so sum_j dV_j = sum_i dO_i."""
    B, N, H, d = 2, 31, 2, 8
    q, k, v, do = (_rand((B, N, H, d), 70 + i) for i in range(4))
    o, lse = oracle.fwd(q, k, v, 0.4, causal)
    dq, dk, dv = oracle.bwd(q, k, v, o, lse, do, 0.4, causal)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)


# ---------------------------------------------------------------- varlen

@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_dense(causal):
    """Each packed sequence is an independent attention problem (fusion page, varlen)."""
    lens = [5, 1, 17, 8]
    cu = inputs.cu_seqlens(lens)
    T, H, d = int(cu[-1]), 3, 8
    q, k, v, do = (_rand((T, H, d), 80 + i) for i in range(4))
    o, lse = oracle.fwd_varlen(q, k, v, cu, 0.6, causal)
    dq, dk, dv = oracle.bwd_varlen(q, k, v, o, lse, do, cu, 0.6, causal)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        sl = lambda x: x[None, a:b]
        od, lsed = oracle.fwd(sl(q), sl(k), sl(v), 0.6, causal)
        np.testing.assert_allclose(o[a:b], od[0], atol=1e-14)
        np.testing.assert_allclose(lse[:, a:b], lsed[0], atol=1e-14)
        g = oracle.bwd(sl(q), sl(k), sl(v), od, lsed, sl(do), 0.6, causal)
        for x, y in zip((dq, dk, dv), g):
            np.testing.assert_allclose(x[a:b], y[0], atol=1e-14)


def test_varlen_rejects_bad_cu_seqlens():
    q = np.zeros((4, 1, 2))
    for cu in ([1, 4], [0, 3], [0, 3, 2, 4]):
        with pytest.raises(ValueError):
            oracle.fwd_varlen(q, q, q, np.array(cu, dtype=np.int32), 1.0, False)


def test_thread_count_does_not_change_results():
    B, N, H, d = 2, 70, 3, 8
    q, k, v, do = (_rand((B, N, H, d), 90 + i) for i in range(4))
    o1, l1 = oracle.fwd(q, k, v, 0.5, True, nthreads=1)
    o8, l8 = oracle.fwd(q, k, v, 0.5, True, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(l1, l8)
    g1 = oracle.bwd(q, k, v, o1, l1, do, 0.5, True, nthreads=1)
    g8 = oracle.bwd(q, k, v, o1, l1, do, 0.5, True, nthreads=8)
    assert all(np.array_equal(a, b) for a, b in zip(g1, g8))


# ---------------------------------------------------------------- input conversion

def test_widen_is_exact():
    assert oracle.widen(np.array([0x3F80, 0xC000, 0x3F81], np.uint16), "bf16").tolist() == \
        [1.0, -2.0, 1.0 + 2.0 ** -7]
    assert oracle.widen(np.array([0x3C00, 0xC000, 0x3C01], np.uint16), "f16").tolist() == \
        [1.0, -2.0, 1.0 + 2.0 ** -10]


def test_input_rounding_is_nearest_even():
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -1.5], np.float32)
    got = oracle.widen(inputs.round_to_bits(x, "bf16"), "bf16")
    assert got.tolist() == [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.5]
    y = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11], np.float32)
    assert oracle.widen(inputs.round_to_bits(y, "f16"), "f16").tolist() == [1.0, 1 + 2.0 ** -9]


def test_varlen_length_draw():
    for seed in (0, 1, 2):
        lens = inputs.varlen_lengths(131072, 64, 16384, seed)
        assert sum(lens) == 131072
        assert all(64 <= n <= 16384 for n in lens[:-1]) and 1 <= lens[-1] <= 16384


# ---------------------------------------------------------------- decode shapes (Nq != Nk)

@pytest.mark.parametrize("nsplit", [None, 1, 2, 3, 4])
def test_decode_narration_example(nsplit):
    # The narration's row as one query against four cached keys: the split form with key
    # blocks of two is exactly the two-block walk-through (after block two the numerator and
    # denominator relative to the running maximum 4 are 72.5 and 2.5).
    g = _golden("narration_online_softmax_example.json")
    scores = [math.log(1), math.log(2), math.log(4), math.log(3)]
    q, k, v = _one_row_problem(scores, g["values"])
    q = q[:, :1]
    if nsplit is None:
        o, lse = oracle.fwd_decode(q, k, v, 1.0, False)
    else:
        o, lse = oracle.fwd_decode_split(q, k, v, 1.0, False, nsplit)
    assert o[0, 0, 0, 0] == pytest.approx(g["output"], abs=1e-12)
    last = g["after_block"][-1]
    assert o[0, 0, 0, 0] == pytest.approx(last["numerator"] / last["denominator"], abs=1e-12)
    assert lse[0, 0, 0] == pytest.approx(
        math.log(last["block_max_exp"] * last["denominator"]), abs=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 7), (3, 7), (7, 7), (9, 5)])
@pytest.mark.parametrize("nsplit", [None, 3])
def test_decode_visible_counts(causal, nq, nk, nsplit):
    # q = 0 makes every visible key weigh the same; v_j = e_j then reads off which keys row i
    # saw: O_i = (1/n_i) on the first n_i coordinates, LSE_i = ln n_i. Query row i stands at
    # position nk - nq + i, so with the mask it sees n_i = clamp(nk - nq + i + 1, 0, nk) keys.
    d = max(nk, 2)
    q = np.zeros((1, nq, 1, d))
    k = _rand((1, nk, 1, d), 5)
    v = np.zeros((1, nk, 1, d))
    for j in range(nk):
        v[0, j, 0, j] = 1.0
    if nsplit is None:
        o, lse = oracle.fwd_decode(q, k, v, 0.7, causal)
    else:
        o, lse = oracle.fwd_decode_split(q, k, v, 0.7, causal, nsplit)
    for i in range(nq):
        n = min(max(nk - nq + i + 1, 0), nk) if causal else nk
        want = np.zeros(d)
        want[:n] = 1.0 / n if n else 0.0
        np.testing.assert_allclose(o[0, i, 0], want, atol=1e-14)
        if n:
            assert lse[0, 0, i] == pytest.approx(math.log(n), abs=1e-13)
        else:
            assert lse[0, 0, i] == -math.inf


@pytest.mark.parametrize("causal", [False, True])
def test_decode_square_is_the_plain_forward(causal):
    # with as many queries as keys the decode rule is the ordinary (causal) attention
    q, k, v = (_rand((2, 13, 3, 8), s) for s in (20, 21, 22))
    o1, l1 = oracle.fwd(q, k, v, 0.4, causal)
    o2, l2 = oracle.fwd_decode(q, k, v, 0.4, causal)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


def test_decode_constant_values():
    q = _rand((2, 3, 2, 6), 30) * 4
    k = _rand((2, 19, 2, 6), 31) * 4
    v = np.broadcast_to(np.arange(6.0) - 2.5, (2, 19, 2, 6)).copy()
    for causal in (False, True):
        for nsplit in (1, 4, 25):
            o, _ = oracle.fwd_decode_split(q, k, v, 0.9, causal, nsplit)
            np.testing.assert_allclose(o, np.broadcast_to(np.arange(6.0) - 2.5, o.shape),
                                       rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_split_equals_unsplit(causal):
    # the block-merge rule reproduces the one-shot softmax for any cut of the keys,
    # including cuts that leave trailing ranges empty
    q = _rand((2, 5, 3, 16), 40) * 2
    k = _rand((2, 37, 3, 16), 41) * 2
    v = _rand((2, 37, 3, 16), 42)
    o, lse = oracle.fwd_decode(q, k, v, 0.6, causal)
    for nsplit in (1, 2, 3, 7, 36, 37, 50):
        o2, l2 = oracle.fwd_decode_split(q, k, v, 0.6, causal, nsplit)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)


def test_decode_shift_invariance_and_large_scores():
    # adding c to every score of a row leaves O unchanged and moves LSE by c; scores near
    # 1000 do not overflow
    q = _rand((1, 4, 1, 8), 50)
    k = _rand((1, 23, 1, 8), 51)
    v = _rand((1, 23, 1, 8), 52)
    c = 1000.0
    q2 = np.concatenate([q, np.ones((1, 4, 1, 1))], axis=-1)
    k2 = np.concatenate([k, np.full((1, 23, 1, 1), c)], axis=-1)
    v2 = np.concatenate([v, np.zeros((1, 23, 1, 1))], axis=-1)
    for causal in (False, True):
        o, lse = oracle.fwd_decode_split(q, k, v, 1.0, causal, 4)
        o2, lse2 = oracle.fwd_decode_split(q2, k2, v2, 1.0, causal, 4)
        np.testing.assert_allclose(o2[..., :8], o, rtol=0, atol=1e-11)
        np.testing.assert_allclose(lse2, lse + c, rtol=0, atol=1e-9)


# ---------------------------------------------------------------- FP8 (e4m3) storage

def test_e4m3_codes():
    """Values the OCP E4M3 format fixes (1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits, no infinities): zero, the subnormals m * 2^-9, the smallest normal 2^-6, one,
    the largest finite 448, NaN at S.1111.111."""
    w = oracle.widen(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3F, 0x40, 0x77, 0x78,
                               0x7E, 0xFE, 0xB8], dtype=np.uint8), "e4m3")
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.875, 2.0, 240.0, 256.0,
            448.0, -448.0, -1.0]
    assert list(w) == want
    assert np.signbit(w[1])
    assert np.isnan(oracle.widen(np.array([0x7F, 0xFF], dtype=np.uint8), "e4m3")).all()
    allv = oracle.widen(np.arange(256, dtype=np.uint8), "e4m3")
    pos = allv[:127]
    assert np.all(np.diff(pos) > 0)                      # codes 0..126 increase strictly
    assert np.array_equal(allv[128:255], -pos)           # sign bit mirrors
    assert np.isfinite(allv).sum() == 254


def test_e4m3_widen_matches_torch():
    """Library cross-check: torch's float8_e4m3fn decodes every code to the same value."""
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    w = oracle.widen(codes, "e4m3")
    assert np.array_equal(np.isnan(w), np.isnan(t))
    assert np.array_equal(w[~np.isnan(w)], t[~np.isnan(t)])


def test_e4m3_input_rounding():
    """The input quantiser rounds to the nearest code, ties to the even code, and saturates
    at 448; it agrees with torch's conversion."""
    vals = oracle.widen(np.arange(127, dtype=np.uint8), "e4m3")
    mids = (vals[:-1] + vals[1:]) / 2
    got = oracle.widen(inputs.round_to_e4m3(mids.astype(np.float32)), "e4m3")
    lo, hi = np.arange(126), np.arange(1, 127)
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(got, vals[even])
    assert oracle.widen(inputs.round_to_e4m3(np.float32([1e6, -500.0])), "e4m3").tolist() == \
        [448.0, -448.0]
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal(20000).astype(np.float32) * 50
    t = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(inputs.round_to_e4m3(x), t.numpy())


def test_fp8_guide_example():
    """Guide §5.3 row (scores 1, 3, 2, 4) stored in e4m3: q = e1, k_j = x_j e1, V = I; the
    descales multiply to 1 on the scores (0.5 * 2) and scale V by 3."""
    g = _golden("guide_online_softmax_example.json")
    x = g["scores"]
    n = len(x)
    q = np.zeros((1, n, 1, n), dtype=np.float32)
    q[0, 0, 0, 0] = 2.0                   # 2 * 0.5 = 1
    k = np.zeros((1, n, 1, n), dtype=np.float32)
    k[0, :, 0, 0] = np.asarray(x) / 2.0   # (x / 2) * 2 = x
    v = np.eye(n, dtype=np.float32).reshape(1, n, 1, n)
    qc, kc, vc = (inputs.round_to_e4m3(t) for t in (q, k, v))
    o, lse = oracle.fwd_fp8(qc, kc, vc, 0.5, 2.0, 3.0, 1.0, False)
    np.testing.assert_allclose(o[0, 0, 0] / 3.0, g["one_shot"]["softmax"], atol=g["abs_tol"])
    assert math.exp(lse[0, 0, 0] - g["one_shot"]["max"]) == pytest.approx(
        g["one_shot"]["sum"], abs=g["abs_tol"])


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_descales(causal):
    """The value of a stored tensor is its descale times its codes' values: q_descale and
    k_descale act as a factor on the scores, v_descale as a factor on the output."""
    B, N, H, d = 1, 23, 2, 16
    (qc, kc, vc), (qd, kd, _) = inputs.fp8_inputs(B, N, H, d, 5)
    o1, l1 = oracle.fwd_fp8(qc, kc, vc, 1.0, 1.0, 1.0, 0.3 * 0.25 * 4.0, causal)
    o2, l2 = oracle.fwd_fp8(qc, kc, vc, 0.25, 4.0, 1.0, 0.3, causal)
    o3, l3 = oracle.fwd_fp8(qc, kc, vc, 0.25, 4.0, 0.125, 0.3, causal)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o3, 0.125 * o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, l1, rtol=0, atol=1e-12)
    # a descale on q alone changes the scores (not a no-op)
    o4, _ = oracle.fwd_fp8(qc, kc, vc, 2 * qd, kd, 1.0, 0.3, causal)
    o5, _ = oracle.fwd_fp8(qc, kc, vc, qd, kd, 1.0, 0.3, causal)
    assert np.abs(o4 - o5).max() > 1e-1


def test_fp8_inputs_recipe():
    """descale = amax / 448 per tensor, so the largest stored magnitude is 448 exactly."""
    (qc, kc, vc), ds = inputs.fp8_inputs(2, 64, 3, 32, 0)
    for c, s, i in zip((qc, kc, vc), ds, range(3)):
        x = np.random.default_rng(0 + i).standard_normal((2, 64, 3, 32), dtype=np.float32)
        assert s == pytest.approx(float(np.abs(x).max()) / 448, rel=1e-6)
        assert np.abs(oracle.widen(c, "e4m3")).max() == 448.0
        assert np.abs(oracle.widen(c, "e4m3") * s - x).max() <= 2.0 ** -4 * np.abs(x).max()


@pytest.mark.parametrize("scale", [0.05, 1.0, 6.0])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_error_bound_holds_for_rounded_weights(scale, causal):
    """The FP8 tolerance (tests/fp8_bound.py) against a direct simulation of its premise:
    every weight exp(s - max) scaled by 2^delta (delta >= 0, drawn per key), rounded to the
    nearest e4m3 code, and the output taken as the weighted mean of the rounded weights.
    The bound must hold everywhere and must not be vacuous."""
    from fp8_bound import fp8_bounds
    N, d = 96, 16
    rng = np.random.default_rng(11)
    (qc, kc, vc), (qd, kd, vd) = inputs.fp8_inputs(1, N, 1, d, 9)
    q, k, v = (oracle.widen(c, "e4m3")[0, :, 0, :] * s for c, s in zip((qc, kc, vc),
                                                                        (qd, kd, vd)))
    o, lse = oracle.fwd(q[None, :, None, :], k[None, :, None, :], v[None, :, None, :], scale,
                        causal)
    o, lse = o[0, :, 0, :], lse[0, 0]
    ob, lb = fp8_bounds(q, k, v, o, scale, causal)
    worst = 0.0
    for trial in range(4):
        s = scale * q @ k.T
        if causal:
            s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        delta = rng.uniform(0.0, 8.0, size=p.shape) * (trial > 0)
        big = (p * np.exp2(delta)).astype(np.float32)
        pr = oracle.widen(inputs.round_to_e4m3(big), "e4m3") / np.exp2(delta)
        o_sim = (pr @ v) / pr.sum(axis=1, keepdims=True)
        lse_sim = np.log(pr.sum(axis=1)) + m[:, 0]
        assert np.all(np.abs(o_sim - o) <= ob)
        assert np.all(np.abs(lse_sim - lse) <= lb)
        worst = max(worst, float((np.abs(o_sim - o) / ob).max()))
    print(f"worst error/bound {worst:.3f}")
    assert worst > 0.02, worst


# ---------------------------------------------------------------- merging partial results (O, LSE)

def test_merge_narration_example():
    """The narration's row (exponentiated scores 1, 2 | 4, 3, values 10, 20 | 30, 40) as two
    parts, each normalised over its own keys: merged O = 29 and LSE = ln 10 as printed."""
    g = _golden("narration_online_softmax_example.json")
    o1, l1 = (1 * 10 + 2 * 20) / 3, math.log(3)
    o2, l2 = (4 * 30 + 3 * 40) / 7, math.log(7)
    o, lse = oracle.merge(np.array([o1, o2]).reshape(2, 1, 1, 1, 1),
                          np.array([l1, l2]).reshape(2, 1, 1, 1))
    assert o[0, 0, 0, 0] == pytest.approx(g["output"], abs=1e-12)
    assert lse[0, 0, 0] == pytest.approx(math.log(g["one_shot"]["weight_total"]), abs=1e-12)


@pytest.mark.parametrize("parts", [2, 3, 5])
def test_merge_of_key_shards_is_the_whole(parts):
    """Attention of the same queries over disjoint key shards, merged, equals attention over
    all keys (the rule is exact in real arithmetic)."""
    B, N, H, d = 2, 30, 2, 8
    q = _rand((B, N, H, d), 40)
    k = _rand((B, N, H, d), 41)
    v = _rand((B, N, H, d), 42)
    ro, rl = oracle.fwd_decode(q, k, v, 0.4, False)
    cuts = np.linspace(0, N, parts + 1).astype(int)
    os, ls = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = oracle.fwd_decode(q, k[:, a:b], v[:, a:b], 0.4, False)
        os.append(o)
        ls.append(l)
    o, lse = oracle.merge(np.stack(os), np.stack(ls))
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_merge_empty_parts():
    """A part that saw no key (LSE = -inf) contributes nothing; all parts empty gives O = 0,
    LSE = -inf; the order of the parts does not matter."""
    o1 = _rand((1, 3, 1, 4), 50)
    l1 = _rand((1, 1, 3), 51)
    junk = _rand((1, 3, 1, 4), 52) * 100
    ninf = np.full((1, 1, 3), -np.inf)
    o, lse = oracle.merge(np.stack([o1, junk]), np.stack([l1, ninf]))
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(lse, l1, atol=1e-15)
    o, lse = oracle.merge(np.stack([junk, junk]), np.stack([ninf, ninf]))
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o2 = _rand((1, 3, 1, 4), 53)
    l2 = _rand((1, 1, 3), 54)
    a = oracle.merge(np.stack([o1, o2]), np.stack([l1, l2]))
    b = oracle.merge(np.stack([o2, o1]), np.stack([l2, l1]))
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-14)


# ---------------------------------------------------------------- row-subset functions

@pytest.mark.parametrize("causal", [False, True])
def test_rows_equal_whole_tensor_oracle(causal):
    """oracle.rows (O, LSE, dQ of chosen rows against all keys) gives the rows of the
    whole-tensor fwd and bwd, which the pins above fix."""
    N, H, d = 57, 2, 16
    q, k, v, do = (_rand((1, N, H, d), 60 + i) for i in range(4))
    o, lse = oracle.fwd(q, k, v, 0.3, causal)
    dq, _, _ = oracle.bwd(q, k, v, o, lse, do, 0.3, causal)
    pos = np.array([0, 1, 5, 31, N - 2, N - 1])
    for h in range(H):
        ro, rl, rdq = oracle.rows(q[0, pos, h], k[0, :, h], v[0, :, h], pos, 0.3, causal,
                                  do[0, pos, h])
        np.testing.assert_allclose(ro, o[0, pos, h], rtol=0, atol=1e-13)
        np.testing.assert_allclose(rl, lse[0, h, pos], rtol=0, atol=1e-13)
        np.testing.assert_allclose(rdq, dq[0, pos, h], rtol=0, atol=1e-13)


def test_tail_keys_equal_whole_tensor_oracle():
    """Under the causal mask the last R keys are seen only by the last R rows: their dK and
    dV from those rows alone equal the whole-tensor bwd's."""
    N, H, d, R = 64, 2, 8, 9
    q, k, v, do = (_rand((1, N, H, d), 70 + i) for i in range(4))
    o, lse = oracle.fwd(q, k, v, 0.5, True)
    _, dk, dv = oracle.bwd(q, k, v, o, lse, do, 0.5, True)
    tail = np.arange(N - R, N)
    for h in range(H):
        to, tl, _ = oracle.rows(q[0, tail, h], k[0, :, h], v[0, :, h], tail, 0.5, True)
        tdk, tdv = oracle.tail_keys(q[0, tail, h], k[0, :, h], v[0, :, h], do[0, tail, h],
                                    to, tl, 0.5)
        np.testing.assert_allclose(tdk, dk[0, tail, h], rtol=0, atol=1e-13)
        np.testing.assert_allclose(tdv, dv[0, tail, h], rtol=0, atol=1e-13)


def test_chunked_draws_are_one_stream():
    """inputs.normal_bits draws in chunks from one generator: the same bits as one draw."""
    ref = inputs.round_to_bits(
        np.random.default_rng(7).standard_normal(size=(3, 1001, 5), dtype=np.float32), "bf16")
    for chunk in (1, 7, 1000, 1 << 26):
        assert np.array_equal(inputs.normal_bits((3, 1001, 5), "bf16", 7, chunk=chunk), ref)
