"""The FP8 forward's tolerances (tests/fp8_bound.py) at the workload's size, on the CPU.

At N = 8192 keys (one (b, h) slice of the FP8 workloads, d = 128, 1024 of its rows) the
weights exp(s - max s) are rounded to e4m3 at random reference offsets 2^delta (delta in
[0, 8], the kernel's lagging reference max) and the output is their weighted mean, rounded
to bf16: a direct simulation of the premise of both bounds. That output must pass the
worst-case bound and the squared-error bound. Outputs with a plausible mistake must fail
the squared-error bound, although (the reason it exists) most of them pass the worst-case
bound there: the output scaled by 0.7, one 128-key tile of V replaced by the next tile's
rows, and an all-zero output."""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_10_amd import inputs
from fp8_bound import fp8_bounds, fp8_rms_ratio


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_rms_bound_discriminates(causal):
    N, d = 8192, 128
    rows = np.arange(0, N, 8)
    (qc, kc, vc), ds = inputs.fp8_inputs(1, N, 1, d, 0)
    q, k, v = (oracle.widen(c, "e4m3")[0, :, 0, :] * s for c, s in zip((qc, kc, vc), ds))
    scale = 1 / math.sqrt(d)
    o, _ = oracle.fwd(q[None, :, None], k[None, :, None], v[None, :, None], scale, causal)
    o = o[0, rows, 0]
    ob, _, var = fp8_bounds(q, k, v, o, scale, causal, rows, with_var=True)

    rng = np.random.default_rng(1)
    s = scale * q[rows] @ k.T
    if causal:
        s = np.where(np.arange(N)[None, :] > rows[:, None], -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    delta = rng.uniform(0.0, 8.0, size=p.shape)
    pr = oracle.widen(inputs.round_to_e4m3((p * np.exp2(delta)).astype(np.float32)),
                      "e4m3") / np.exp2(delta)
    bf16 = lambda x: oracle.widen(inputs.round_to_bits(x.astype(np.float32), "bf16"), "bf16")
    o_sim = bf16((pr @ v) / pr.sum(axis=1, keepdims=True))
    v_bad = v.copy()
    v_bad[1024:1152] = v[1152:1280]
    o_tile = bf16((pr @ v_bad) / pr.sum(axis=1, keepdims=True))

    worst = lambda x: float((np.abs(x - o) / ob).max())
    r_sim = fp8_rms_ratio(o_sim, o, var)
    print(f"simulated: worst {worst(o_sim):.3f}, squared {r_sim:.3f}")
    assert worst(o_sim) <= 1.0 and r_sim <= 0.75
    for name, bad in (("x0.7", 0.7 * o_sim), ("wrong V tile", o_tile), ("zeros", 0 * o)):
        r = fp8_rms_ratio(bad, o, var)
        print(f"{name}: worst {worst(bad):.3f}, squared {r:.3f}")
        assert r > 10.0, (name, r)
    if not causal:  # the worst-case bound alone lets these through at this size
        assert worst(0.7 * o_sim) <= 1.0 and worst(o_tile) <= 1.0
