"""Helpers shared by the GPU parity tests: moving 16-bit patterns to and from the device
and the tolerance checks.

Tolerances (per tensor, against the fp64 oracle on the same stored inputs): max-abs error
<= 2e-2 and mean-abs error <= 2e-3 for O, LSE, dQ, dK and dV; in addition the relative
Frobenius error of each tensor must be <= 1e-2, which catches errors that the absolute
bounds would let through when the tensor itself is small (O at N = 8192 has a standard
deviation of about 0.018). The relative check is skipped when the reference's RMS is
below 1e-4 (an exactly-zero gradient, e.g. dQ with a single visible key).

Tests at softmax scales other than 1/sqrt(d) (not one of the five workloads) can produce
gradients of magnitude 10 or more, where rounding the output to bf16 alone costs up to
half an ulp = 2^-9 |x|; they pass rtol = 2^-7 (two half-ulps), applied elementwise on top
of the absolute bound.
"""
import numpy as np

import oracle

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_FRO = 1e-2


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


def err_stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    fro = np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300)
    return {"max_abs": float(d.max()) if d.size else 0.0,
            "mean_abs": float(d.mean()) if d.size else 0.0,
            "rel_fro": float(fro) if d.size else 0.0}


def assert_close(name, got, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS, rel_fro=REL_FRO,
                 rtol=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    s = err_stats(got, ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    excess = float(np.max(np.abs(got - ref) - rtol * np.abs(ref))) if ref.size else 0.0
    print(f"  {name}: max_abs={s['max_abs']:.3e} mean_abs={s['mean_abs']:.3e} "
          f"rel_fro={s['rel_fro']:.3e} ref_rms={rms:.3e} max|ref|="
          f"{float(np.max(np.abs(ref))) if ref.size else 0:.3e}", flush=True)
    assert excess <= max_abs, (name, s, excess)
    assert s["mean_abs"] <= mean_abs, (name, s)
    if rms >= 1e-4:
        assert s["rel_fro"] <= rel_fro, (name, s)
    return s
