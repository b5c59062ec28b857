"""GPU parity of fa_fwd_fp8 (FP8 forward, called through the C ABI via the ctypes binding)
against the fp64 oracle on the same stored e4m3 inputs and descales. The tolerances are
those of fp8_bound.py, derived from the rounding of P to e4m3: the per-element worst-case
bound everywhere and, on every slice of at least 512 rows, the bound on the summed squared
error (the one that discriminates at N = 8192); in addition the signed mean of the LSE
error over many rows must stay near 0 (nearest-even rounding has no bias; a few rows, e.g.
one four-key example, need not average out)."""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_10_amd import inputs
from fp8_bound import assert_rms_ok, assert_within_bound, fp8_bounds

pytestmark = pytest.mark.gpu


def fa():
    import exact_io_aware_10_amd as m
    return m


def run(codes, descales, causal, scale):
    import torch
    B, N, H, d = codes[0].shape
    print(f"[fp8] B={B} N={N} H={H} d={d} causal={causal} scale={scale} "
          f"descales={tuple(round(x, 6) for x in descales)}", flush=True)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(c)).cuda() for c in codes)
    o, lse = fa().fa_fwd_fp8(q, k, v, *descales, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    ob = o.view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.widen(ob, "bf16"), lse.cpu().numpy().astype(np.float64)


def check(codes, descales, o, lse, causal, scale, slices=None, rows=None):
    B, N, H, d = codes[0].shape
    scale = 1 / math.sqrt(d) if scale is None else scale
    vals = [oracle.widen(c, "e4m3") * s for c, s in zip(codes, descales)]
    slices = slices or [(b, h) for b in range(B) for h in range(H)]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    dl = []
    for b, h in slices:
        qs, ks, vs = (x[b, :, h, :] for x in vals)
        ro, rl = oracle.fwd(qs[None, :, None, :], ks[None, :, None, :], vs[None, :, None, :],
                            scale, causal)
        ro, rl = ro[0, rows, 0, :], rl[0, 0, rows]
        ob, lb, var = fp8_bounds(qs, ks, vs, ro, scale, causal, rows, with_var=True)
        assert_within_bound(f"O[{b},{h}]", o[b, rows, h, :], ro, ob)
        assert_within_bound(f"LSE[{b},{h}]", lse[b, h, rows], rl, lb)
        if len(rows) >= 512:
            assert_rms_ok(f"O[{b},{h}] squared error", o[b, rows, h, :], ro, var)
        dl.append(lse[b, h, rows] - rl)
    dl = np.concatenate(dl)
    print(f"  LSE signed mean error {dl.mean():.3e} over {dl.size} rows", flush=True)
    if dl.size >= 512:  # an average over many independently rounded rows
        assert abs(dl.mean()) <= 2.0 ** -8


# Unmasked launches with at least two query blocks per CU (512 on MI355X) take the stream
# form (one workgroup per CU walking its blocks as one tile stream): items of one tile, of
# two with a ragged last one, 17 blocks of 33 tiles, and d = 64; sampled slices (the
# full-size workloads below check every slice of the stream form).
@pytest.mark.parametrize("B,N,H,d", [(32, 100, 16, 128), (32, 200, 16, 64), (2, 4196, 16, 128),
                                     (4, 2048, 16, 64)])
def test_fp8_stream(B, N, H, d):
    codes, ds = inputs.fp8_inputs(B, N, H, d, seed=N + H)
    o, lse = run(codes, ds, False, None)
    check(codes, ds, o, lse, False, None,
          slices=[(0, 0), (B - 1, H - 1), (B // 2, 7), (1, 3)])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,N,H,d", [(1, 1, 1, 64), (1, 5, 1, 64), (2, 100, 2, 64),
                                     (1, 257, 2, 128), (2, 300, 3, 128), (1, 1000, 1, 128),
                                     (1, 600, 2, 64)])
def test_fp8_small(B, N, H, d, causal):
    codes, ds = inputs.fp8_inputs(B, N, H, d, seed=N + d)
    o, lse = run(codes, ds, causal, None)
    check(codes, ds, o, lse, causal, None)


def test_fp8_guide_example():
    """Guide §5.3 row (scores 1, 3, 2, 4) in e4m3 with V = I, padded to d = 64."""
    n, d = 4, 64
    x = [1.0, 3.0, 2.0, 4.0]
    q = np.zeros((1, n, 1, d), dtype=np.float32)
    q[0, :, 0, 0] = 2.0
    k = np.zeros((1, n, 1, d), dtype=np.float32)
    k[0, :, 0, 0] = np.asarray(x) / 2.0
    v = np.zeros((1, n, 1, d), dtype=np.float32)
    v[0, :, 0, :n] = np.eye(n)
    codes = [inputs.round_to_e4m3(t) for t in (q, k, v)]
    ds = (0.5, 2.0, 3.0)
    o, lse = run(codes, ds, False, 1.0)
    check(codes, ds, o, lse, False, 1.0)
    # every row holds 3 x the guide's softmax row (within e4m3's rounding of the weights)
    np.testing.assert_allclose(o[0, 0, 0, :n] / 3.0, [0.032, 0.237, 0.087, 0.644], atol=0.02)


@pytest.mark.parametrize("scale", [-0.05, 0.0, 0.2])
def test_fp8_scale_values(scale):
    codes, ds = inputs.fp8_inputs(1, 333, 2, 128, seed=21)
    o, lse = run(codes, ds, True, scale)
    check(codes, ds, o, lse, True, scale)


def test_fp8_descale_values():
    codes, (qd, kd, vd) = inputs.fp8_inputs(1, 500, 2, 64, seed=4)
    ds = (4 * qd, 0.5 * kd, 3.0 * vd)
    o, lse = run(codes, ds, False, None)
    check(codes, ds, o, lse, False, None)


@pytest.mark.parametrize("N", [129, 1023, 2049])
def test_fp8_ragged(N):
    codes, ds = inputs.fp8_inputs(1, N, 2, 128, seed=N)
    o, lse = run(codes, ds, True, None)
    check(codes, ds, o, lse, True, None)


def test_fp8_deterministic():
    import torch
    codes, ds = inputs.fp8_inputs(2, 700, 2, 128, seed=8)
    q, k, v = (torch.from_numpy(c).cuda() for c in codes)
    o1, l1 = fa().fa_fwd_fp8(q, k, v, *ds, causal=True)
    o2, l2 = fa().fa_fwd_fp8(q, k, v, *ds, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", sorted(inputs.FP8_WORKLOADS))
def test_fp8_workloads(name):
    """Full size, in the benchmark's launch configuration; every (b, h) slice checked."""
    wl = inputs.FP8_WORKLOADS[name]
    codes, ds = inputs.fp8_inputs(wl.B, wl.N, wl.H, wl.d, seed=0)
    o, lse = run(codes, ds, wl.causal, None)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    check(codes, ds, o, lse, wl.causal, None)
