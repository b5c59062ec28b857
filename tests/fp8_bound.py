"""Tolerance of the FP8 forward: a per-element bound on its error against exact attention
of the stored (descaled e4m3) values, derived from the arithmetic.

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
"""
import numpy as np


def fp8_bounds(q, k, v, o_ref, scale, causal, rows=None, block=512):
    """Per-element bound on |O_fp8 - O| and per-row bound on |LSE_fp8 - LSE| for one (b, h)
    slice. q: [Nq, d], k, v: [Nk, d] fp64 (descaled values); o_ref: [Nq, d] exact output;
    rows: the query rows (indices into q, also their positions for the causal mask)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    av = np.abs(np.asarray(v, dtype=np.float64))
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    ob = np.empty((len(rows), k.shape[1] if k.ndim == 2 else av.shape[1]))
    lb = np.empty(len(rows))
    for r0 in range(0, len(rows), block):
        rr = rows[r0:r0 + block]
        s = scale * (q[rr] @ k.T)
        if causal:
            s = np.where(np.arange(k.shape[0])[None, :] > rr[:, None], -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        e = np.maximum(2.0 ** -4 * p, np.minimum(p, 2.0 ** -10))
        l = p.sum(axis=1)
        se = e.sum(axis=1)
        ao = np.abs(np.asarray(o_ref, dtype=np.float64)[r0:r0 + block])
        num = e @ av + se[:, None] * ao
        ob[r0:r0 + block] = num / (l - se)[:, None] + 2.0 ** -8 * ao + 1e-6
        lb[r0:r0 + block] = -np.log1p(-se / l) + 1e-5
    return ob, lb


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
