"""fp64 CPU oracle for exact attention: TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package. The product library never loads it, and it shares no code with the GPU path.

It follows the definition of attention on the page "FlashAttention 详解（零基础入门）"
(§2.3 scores S = QK^T scaled, §2.4 safe softmax, §2.5 O = PV), the tiled algorithm of the
same page (§5.2-§5.4 online softmax, §6.2 Q-outer / K,V-inner loop), the deferred
normalisation of the narration script "FlashAttention 短片讲解稿" (segment 第二招 · 在线
Softmax), and the causal mask and varlen packing of "FlashAttention 与算子融合" (fusion
table, 工程实践). The arithmetic lives in oracle.cpp; this module converts the stored
16-bit input bits to fp64 and calls it through ctypes.

Every function here is pinned by tests/test_oracle_pins.py against values printed on the
pages, closed forms, invariants, brute force and an autograd cross-check.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB points the test suite at another build of oracle.cpp (the mutation
        # test plants mistakes in copies of the source and checks that the pins fail).
        path = os.environ.get("ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        L, D, I = ctypes.c_long, ctypes.c_double, ctypes.c_int
        lib.oracle_fwd.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, D, I, I]
        lib.oracle_fwd_blocked.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, D, I, L, L, I, dp, I]
        lib.oracle_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, L, L, L, L, D, I, I]
        lib.oracle_fwd_varlen.argtypes = [dp, dp, dp, dp, dp, ip, L, L, L, L, D, I, I]
        lib.oracle_fwd_decode.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, D, I, I]
        lib.oracle_fwd_decode_split.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L, D, I, L, I]
        lib.oracle_bwd_varlen.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, ip, L, L, L, L,
                                          D, I, I]
        lib.oracle_merge.argtypes = [dp, dp, dp, dp, L, L, L, I]
        lp = ctypes.POINTER(ctypes.c_long)
        lib.oracle_rows.argtypes = [dp, dp, dp, dp, lp, dp, dp, dp, L, L, L, D, I, I]
        lib.oracle_tail_keys.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, L, L, L, D, I]
        for f in ("oracle_fwd", "oracle_fwd_blocked", "oracle_bwd", "oracle_fwd_varlen",
                  "oracle_bwd_varlen", "oracle_fwd_decode", "oracle_fwd_decode_split",
                  "oracle_merge", "oracle_rows", "oracle_tail_keys"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on (its affinity), at most
    OMP_NUM_THREADS where that is set (a GPU host's share of its CPUs per GPU), else at most
    16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = 16
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "") or 16)
    except ValueError:
        pass
    return max(1, min(n, cap))


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored floats given as bit patterns.

    bf16 is the upper half of an IEEE binary32; fp16 is IEEE binary16 (both as uint16).
    e4m3 is the OCP FP8 E4M3 format (uint8): sign bit, 4 exponent bits with bias 7, 3
    mantissa bits; exponent field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN and
    there are no infinities (largest finite 448). All widen to binary64 without rounding.
    """
    if dtype == "e4m3":
        b = np.ascontiguousarray(bits, dtype=np.uint8).astype(np.int64)
        e, m = (b >> 3) & 15, b & 7
        mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return np.where(b >> 7, -mag, mag)
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (code {rc})")


def fwd(q, k, v, scale, causal, nthreads=None):
    """Plain definition. q, k, v: fp64 [B, N, H, d]. Returns (O [B,N,H,d], LSE [B,H,N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    rc = _load().oracle_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), B, N, H, d, float(scale),
                            int(bool(causal)), nthreads or default_threads())
    _check(rc, "oracle_fwd")
    return o, lse


def fwd_fp8(q_codes, k_codes, v_codes, q_descale, k_descale, v_descale, scale, causal,
            nthreads=None):
    """Attention of FP8-stored tensors: each tensor's value is its descale times the e4m3
    code's value (widened exactly), then the plain definition in fp64. Returns (O, LSE)."""
    q = widen(q_codes, "e4m3") * float(q_descale)
    k = widen(k_codes, "e4m3") * float(k_descale)
    v = widen(v_codes, "e4m3") * float(v_descale)
    return fwd(q, k, v, scale, causal, nthreads)


def fwd_blocked(q, k, v, scale, causal, block_q, block_k, form, nthreads=None):
    """Tiled algorithm. form: "normalized" (guide §5.4 / §6.2) or "deferred" (narration).

    Returns (O, LSE, trace) where trace[jb] = (m, l, state[0]) for row 0 of slice (0, 0)
    after key block jb; state is O in the normalised form and the unnormalised numerator
    in the deferred form.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    nkb = max(1, -(-N // block_k))
    trace = np.full((nkb, 3), np.nan)
    f = {"normalized": 0, "deferred": 1}[form]
    rc = _load().oracle_fwd_blocked(_p(q), _p(k), _p(v), _p(o), _p(lse), B, N, H, d,
                                    float(scale), int(bool(causal)), int(block_q), int(block_k),
                                    f, _p(trace), nthreads or default_threads())
    _check(rc, "oracle_fwd_blocked")
    return o, lse, trace


def bwd(q, k, v, o, lse, dout, scale, causal, nthreads=None):
    """Gradients from the saved O and LSE. All [B,N,H,d] fp64 except lse [B,H,N]."""
    q, k, v, o, lse, dout = map(_f64, (q, k, v, o, lse, dout))
    B, N, H, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    rc = _load().oracle_bwd(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dout), _p(dq), _p(dk),
                            _p(dv), B, N, H, d, float(scale), int(bool(causal)),
                            nthreads or default_threads())
    _check(rc, "oracle_bwd")
    return dq, dk, dv


def fwd_decode(q, k, v, scale, causal, nthreads=None):
    """Decode shapes. q: fp64 [B, Nq, H, d]; k, v: [B, Nk, H, d]. Query row i stands at
    position Nk - Nq + i (causal: sees keys j <= Nk - Nq + i). Returns (O [B,Nq,H,d],
    LSE [B,H,Nq])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    assert k.shape == (B, Nk, H, d) and v.shape == k.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    rc = _load().oracle_fwd_decode(_p(q), _p(k), _p(v), _p(o), _p(lse), B, Nq, Nk, H, d,
                                   float(scale), int(bool(causal)), nthreads or default_threads())
    _check(rc, "oracle_fwd_decode")
    return o, lse


def fwd_decode_split(q, k, v, scale, causal, nsplit, nthreads=None):
    """fwd_decode by key splits combined with the block-merge rule (same results up to
    rounding)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    assert k.shape == (B, Nk, H, d) and v.shape == k.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    rc = _load().oracle_fwd_decode_split(_p(q), _p(k), _p(v), _p(o), _p(lse), B, Nq, Nk, H, d,
                                         float(scale), int(bool(causal)), int(nsplit),
                                         nthreads or default_threads())
    _check(rc, "oracle_fwd_decode_split")
    return o, lse


def merge(o_parts, lse_parts, nthreads=None):
    """Merge partial results over disjoint key sets of the same query rows (the block-merge
    rule with m_s = LSE_s, l_s = 1). o_parts: fp64 [P, B, N, H, d]; lse_parts: [P, B, H, N].
    Returns (O [B, N, H, d], LSE [B, H, N])."""
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    P, B, N, H, d = o_parts.shape
    assert lse_parts.shape == (P, B, H, N)
    rows = B * N * H
    op = np.ascontiguousarray(o_parts.reshape(P, rows, d))
    lp = np.ascontiguousarray(lse_parts.transpose(0, 1, 3, 2).reshape(P, rows))
    o = np.empty((rows, d))
    lse = np.empty(rows)
    rc = _load().oracle_merge(_p(op), _p(lp), _p(o), _p(lse), P, rows, d,
                              nthreads or default_threads())
    _check(rc, "oracle_merge")
    return o.reshape(B, N, H, d), np.ascontiguousarray(lse.reshape(B, N, H).transpose(0, 2, 1))


def rows(q_rows, k, v, pos, scale, causal, dout_rows=None, nthreads=None):
    """Rows of one (batch, head) slice too large for the whole-tensor functions. q_rows
    [R, d] at positions pos (int [R]) of a slice with keys and values k, v [N, d]; dout_rows
    [R, d] or None. Returns (O [R, d], LSE [R], dQ [R, d] or None) by the plain definition."""
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    R, d = q_rows.shape
    N = k.shape[0]
    assert k.shape == (N, d) and v.shape == (N, d)
    posa = np.ascontiguousarray(pos, dtype=np.int64)
    assert posa.shape == (R,)
    o = np.empty((R, d))
    lse = np.empty(R)
    dq = None
    dptr = None
    if dout_rows is not None:
        dout_rows = _f64(dout_rows)
        assert dout_rows.shape == (R, d)
        dq = np.empty((R, d))
        dptr = _p(dout_rows)
    rc = _load().oracle_rows(_p(q_rows), _p(k), _p(v), dptr,
                             posa.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), _p(o), _p(lse),
                             _p(dq) if dq is not None else None, R, N, d, float(scale),
                             int(causal), nthreads or default_threads())
    _check(rc, "oracle_rows")
    return o, lse, dq


def tail_keys(q_tail, k, v, dout_tail, o_tail, lse_tail, scale, nthreads=None):
    """dK, dV [R, d] of the last R keys of a causal slice (k, v [N, d]) from its last R rows
    (q_tail, dout_tail, o_tail [R, d], lse_tail [R])."""
    q_tail, k, v = _f64(q_tail), _f64(k), _f64(v)
    dout_tail, o_tail, lse_tail = _f64(dout_tail), _f64(o_tail), _f64(lse_tail)
    R, d = q_tail.shape
    N = k.shape[0]
    assert k.shape == (N, d) and v.shape == (N, d) and lse_tail.shape == (R,)
    dk = np.empty((R, d))
    dv = np.empty((R, d))
    rc = _load().oracle_tail_keys(_p(q_tail), _p(k), _p(v), _p(dout_tail), _p(o_tail),
                                  _p(lse_tail), _p(dk), _p(dv), R, N, d, float(scale),
                                  nthreads or default_threads())
    _check(rc, "oracle_tail_keys")
    return dk, dv


def _cu(cu_seqlens):
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    return cu, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def fwd_varlen(q, k, v, cu_seqlens, scale, causal, nthreads=None):
    """Packed sequences. q, k, v: fp64 [T, H, d]. Returns (O [T,H,d], LSE [H,T])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, d = q.shape
    cu, cup = _cu(cu_seqlens)
    o = np.zeros_like(q)
    lse = np.full((H, T), np.nan)
    rc = _load().oracle_fwd_varlen(_p(q), _p(k), _p(v), _p(o), _p(lse), cup, len(cu) - 1, T,
                                   H, d, float(scale), int(bool(causal)),
                                   nthreads or default_threads())
    _check(rc, "oracle_fwd_varlen")
    return o, lse


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, scale, causal, nthreads=None):
    """Packed-sequence gradients; layouts as fwd_varlen."""
    q, k, v, o, lse, dout = map(_f64, (q, k, v, o, lse, dout))
    T, H, d = q.shape
    cu, cup = _cu(cu_seqlens)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    rc = _load().oracle_bwd_varlen(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dout), _p(dq),
                                   _p(dk), _p(dv), cup, len(cu) - 1, T, H, d, float(scale),
                                   int(bool(causal)), nthreads or default_threads())
    _check(rc, "oracle_bwd_varlen")
    return dq, dk, dv
