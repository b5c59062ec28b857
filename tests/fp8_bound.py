"""Tolerance of the FP8 forward: a per-element bound on its error against exact attention
of the stored (descaled e4m3) values, and a bound on its expected squared error, both
derived from the arithmetic.

Where the FP8 path rounds. The scores are sums of products of two e4m3 values, each
product exact in fp32 (at most 8 significant bits), accumulated in fp32; exp2, the sums of
P V and of P, and the final division are fp32. The one coarse rounding is P -> e4m3 (3
mantissa bits) before P V, and the output's rounding to bf16.

The kernel's weights are P_j = 2^delta_j p_j with p_j = exp(s_j - max s) (so max p = 1,
l = sum p >= 1) and delta_j >= 0: the exponent's reference is at or below the row max at
every point of the loop. Rounding to nearest e4m3 errs by at most 2^-4 relative to the
value at or above 2^-6 (the smallest normal), by at most 2^-10 (half the subnormal spacing
2^-9) below it, and never by more than the value itself when it rounds to 0. In units of p
(delta = 0 is the worst case for the absolute term) each weight is p_j + eps_j with

    |eps_j| <= e_j = max(2^-4 p_j, min(p_j, 2^-10)).

The row sum the kernel divides by adds exactly the rounded weights, so its output is the
weighted mean O~ = sum (p_j + eps_j) v_j / sum (p_j + eps_j), and

    |O~ - O| = |sum eps_j (v_j - O)| / sum (p_j + eps_j) <= sum e_j |v_j - O| / (l - sum e_j)

(l - sum e_j >= 1 - 2^-4 because the largest weight has e = 2^-4). With
|v_j - O| <= |v_j| + |O| this is two matrix products. The bf16 output adds half an ulp,
2^-9 |O|; the bound uses 2^-8 |O| + 1e-6 to cover the fp32 arithmetic. For the LSE,
ln(sum (p + eps) / l) lies within -ln(1 - sum e / l) of 0; 1e-5 covers fp32.

The worst case adds every |eps_j| with the same sign; at N = 8192 keys it comes to about
2^-4 E|v|, several times O's own spread (0.018), so it cannot tell a wrong output from a
right one there. The squared error can. Round-to-nearest leaves an error spread over the
rounding interval of the value, which is at most [-e_j, e_j] wide: modelled as uniform
there, its variance is at most e_j^2 / 3, and the errors of different weights are
independent (each weight is a different exponential). To first order in eps the output's
error is then a sum of independent terms with

    E (O~_c - O_c)^2 <= sum_j (e_j^2 / 3) (v_jc - O_c)^2 / (l - sum e)^2 + (2^-8 O_c)^2 / 3

(the last term: the bf16 output's rounding, uniform within half an ulp <= 2^-8 |O|). Summed
over the rows and columns of a slice of many rows this is a sum of many independent
terms, so the measured sum of squared errors concentrates at or below the summed bound;
fp8_rms_ok compares the two.
"""
import numpy as np


def _t(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))


def fp8_bounds(q, k, v, o_ref, scale, causal, rows=None, block=512, with_var=False):
    """Per-element bound on |O_fp8 - O| and per-row bound on |LSE_fp8 - LSE| for one (b, h)
    slice. q: [Nq, d], k, v: [Nk, d] fp64 (descaled values); o_ref: [len(rows), d] exact
    output; rows: the query rows (indices into q, also their positions for the causal
    mask). With with_var, also returns the per-element bound on the expected squared error
    (the variance bound above). Computed with torch's CPU operations in fp64 (threaded)."""
    import torch
    qt, kt, vt = _t(q), _t(k), _t(v)
    av = vt.abs()
    v2 = vt * vt
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    ot = _t(o_ref)
    ob = torch.empty((len(rows), vt.shape[1]), dtype=torch.float64)
    lb = torch.empty(len(rows), dtype=torch.float64)
    var = torch.empty_like(ob) if with_var else None
    keys = torch.arange(kt.shape[0])
    for r0 in range(0, len(rows), block):
        rr = torch.from_numpy(rows[r0:r0 + block].astype(np.int64))
        s = scale * (qt[rr] @ kt.T)
        if causal:
            s = s.masked_fill(keys[None, :] > rr[:, None], -np.inf)
        m = s.max(dim=1, keepdim=True).values
        p = torch.exp(s - m)
        e = torch.maximum(2.0 ** -4 * p, torch.minimum(p, torch.tensor(2.0 ** -10)))
        l = p.sum(dim=1)
        se = e.sum(dim=1)
        oo = ot[r0:r0 + block]
        ao = oo.abs()
        num = e @ av + se[:, None] * ao
        ob[r0:r0 + block] = num / (l - se)[:, None] + 2.0 ** -8 * ao + 1e-6
        lb[r0:r0 + block] = -torch.log1p(-se / l) + 1e-5
        if with_var:
            e2 = e * e
            # sum_j e_j^2 (v_jc - O_c)^2 = (e2 v^2)_c - 2 O_c (e2 v)_c + O_c^2 sum_j e_j^2
            sq = e2 @ v2 - 2.0 * oo * (e2 @ vt) + oo * oo * e2.sum(dim=1, keepdim=True)
            var[r0:r0 + block] = (sq.clamp_min(0.0) / 3.0 / ((l - se) ** 2)[:, None]
                                  + (2.0 ** -8 * oo) ** 2 / 3.0 + 1e-12)
    if with_var:
        return ob.numpy(), lb.numpy(), var.numpy()
    return ob.numpy(), lb.numpy()


def assert_within_bound(name, got, ref, bound):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape == bound.shape, (name, got.shape, ref.shape, bound.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    ratio = err / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    print(f"  {name}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} "
          f"max err/bound={ratio.max():.3f} mean err/bound={ratio.mean():.3f} "
          f"at {tuple(int(i) for i in worst)}", flush=True)
    assert ratio.max() <= 1.0, (name, worst, float(err[worst]), float(bound[worst]))
    return float(ratio.max())


def fp8_rms_ratio(got, ref, var):
    """Sum of squared errors over the summed variance bound (<= 1 for a correct output of
    many rows)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape == var.shape
    return float(np.sum((got - ref) ** 2) / np.sum(var))


def assert_rms_ok(name, got, ref, var):
    r = fp8_rms_ratio(got, ref, var)
    rms = float(np.sqrt(np.mean((np.asarray(got) - np.asarray(ref)) ** 2)))
    print(f"  {name}: rms err={rms:.3e} rms bound={float(np.sqrt(np.mean(var))):.3e} "
          f"sum sq err / sum var bound={r:.3f}", flush=True)
    assert r <= 1.0, (name, r)
    return r
