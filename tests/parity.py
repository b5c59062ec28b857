"""Helpers shared by the GPU parity tests: moving 16-bit patterns to and from the device
and the tolerance checks.

Tolerances (per tensor, against the fp64 oracle on the same stored inputs): max-abs error
<= 2e-2 and mean-abs error <= 2e-3 for O, LSE, dQ, dK and dV; in addition the relative
Frobenius error of each tensor must be <= 1e-2, which catches errors that the absolute
bounds would let through when the tensor itself is small (O at N = 8192 has a standard
deviation of about 0.018). The relative check is skipped when the reference's RMS is
below 1e-4 (an exactly-zero gradient, e.g. dQ with a single visible key).

Tests at softmax scales other than 1/sqrt(d) (not one of the five workloads) can produce
gradients of magnitude 4 or more. From |x| = 4 on, rounding the output to bf16 alone costs
up to half an ulp, 2^-6 = 0.0156 on [4, 8) and 2^-5 = 0.031 on [8, 16), most or more than
all of the absolute bound, while the arithmetic before it (P and dS rounded to bf16 as
matrix-core operands, 2^-9 relative each) grows with the scale. Those tests pass ulps=1:
the bound becomes MAX_ABS plus the output's own rounding, half an ulp of bf16 at |ref|,
per element (negligible below |ref| = 1). Checks of results that are themselves roundings
of partial results (the ring tests) pass a relative term rtol instead, stated where used.
"""
import numpy as np

import oracle

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_FRO = 1e-2


def half_ulp_bf16(x):
    """Half an ulp of bf16 (8 significant bits) at |x|: 2^(floor(log2 |x|) - 8); 0 at 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8.0), 0.0)


def torch_dtype(dtype):
    import torch
    return {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_device(bits, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).cuda()


def bits_of(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t, dtype):
    """Device 16-bit tensor -> exact fp64 numpy array."""
    return oracle.widen(bits_of(t), dtype)


def err_stats(got, ref, diff=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    e = got - ref if diff is None else diff
    if not e.size:
        return {"max_abs": 0.0, "mean_abs": 0.0, "rel_fro": 0.0}
    d = np.abs(e)
    fro = np.linalg.norm(e.ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300)
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean()), "rel_fro": float(fro)}


def assert_close(name, got, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS, rel_fro=REL_FRO,
                 rtol=0.0, ulps=0, quiet=False):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = got - ref
    s = err_stats(got, ref, diff)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    ad = np.abs(diff)
    if rtol or ulps:
        excess = float(np.max(ad - rtol * np.abs(ref) - ulps * half_ulp_bf16(ref))) \
            if ref.size else 0.0
    else:
        excess = s["max_abs"]
    if not quiet:
        at = ""
        if ref.size:
            w = np.unravel_index(int(np.argmax(ad)), ref.shape)
            at = (f" worst at {tuple(int(i) for i in w)} ref={float(ref[w]):.4f} "
                  f"half-ulp={float(half_ulp_bf16(ref[w])):.2e}")
        print(f"  {name}: max_abs={s['max_abs']:.3e} mean_abs={s['mean_abs']:.3e} "
              f"rel_fro={s['rel_fro']:.3e} ref_rms={rms:.3e} max|ref|="
              f"{float(np.max(np.abs(ref))) if ref.size else 0:.3e}{at}", flush=True)
    assert excess <= max_abs, (name, s, excess)
    assert s["mean_abs"] <= mean_abs, (name, s)
    if rms >= 1e-4:
        assert s["rel_fro"] <= rel_fro, (name, s)
    return s
