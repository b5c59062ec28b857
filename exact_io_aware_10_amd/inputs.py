"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the CPU oracle.

This module holds no attention arithmetic: it draws i.i.d. N(0, 1) values in fp32 on the
CPU, rounds them to bf16 or fp16 with round-to-nearest-even, and returns the 16-bit
patterns. Each side turns the same bits into its own operands (the oracle widens them to
fp64; the GPU path copies them to device memory). It also draws the packed-sequence
lengths and names the five workloads.

Seeds: Q, K, V and dO use default_rng(seed + 0, 1, 2, 3); sequence lengths use
default_rng(seed + 4).

FP8 inputs draw the same N(0, 1) values and store each tensor as OCP FP8 E4M3 codes with one
per-tensor descale factor: descale = amax / 448 (448 is e4m3's largest finite value) in
fp32, code = e4m3(x / descale) rounded to nearest even. The value the attention sees is
descale * (code's value).
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array -> uint16 bit patterns of bf16 or fp16, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        # in 32-bit words: u + 0x7FFF + lsb stays below 2^32 for every finite value and
        # infinity (u <= 0xFF800000); NaN patterns are kept NaN
        u = x.view(np.uint32)
        r = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            r[nan] = (u[nan] >> 16).astype(np.uint16) | np.uint16(0x40)
        return r
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def _e4m3_positive_values() -> np.ndarray:
    """Values of the e4m3 codes 0x00..0x7E (sign 0): 1 sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; 0x7F is NaN."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e - 10.0))


def round_to_e4m3(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint8 e4m3 codes, round to nearest even (ties to the even code),
    magnitudes above 448 saturated to 448."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    vals = _e4m3_positive_values()
    a = np.minimum(np.abs(x).astype(np.float64), vals[-1])
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))


def fp8_tensor(shape, seed: int):
    """One N(0, 1) tensor as (e4m3 codes uint8, descale float) with descale = amax / 448."""
    x = np.random.default_rng(seed).standard_normal(size=shape, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 1.0
    descale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    return round_to_e4m3(x / descale), float(descale)


def fp8_inputs(B, N, H, d, seed):
    """Q, K, V as e4m3 codes [B, N, H, d] (seeds +0, +1, +2) and their descale factors."""
    qs = [fp8_tensor((B, N, H, d), seed + i) for i in range(3)]
    return [c for c, _ in qs], [s for _, s in qs]


def normal_bits(shape, dtype: str, seed: int, chunk: int = 1 << 26) -> np.ndarray:
    """N(0, 1) draws of default_rng(seed) in row-major order, rounded to dtype. Drawn and
    rounded `chunk` values at a time from the one generator (the same stream as a single
    draw), so a tensor of 2^30 values needs no multi-gigabyte temporaries."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        out[a:b] = round_to_bits(rng.standard_normal(size=b - a, dtype=np.float32), dtype)
    return out.reshape(shape)


def attention_inputs(B, N, H, d, dtype, seed, with_dout=False):
    """Q, K, V (and dO) as uint16 bit patterns, shape [B, N, H, d]."""
    shape = (B, N, H, d)
    out = [normal_bits(shape, dtype, seed + i) for i in range(3)]
    if with_dout:
        out.append(normal_bits(shape, dtype, seed + 3))
    return out


def varlen_lengths(total_tokens: int, lo: int, hi: int, seed: int):
    """Draw lengths uniform in [lo, hi] until they cover total_tokens; truncate the last."""
    rng = np.random.default_rng(seed + 4)
    lens = []
    acc = 0
    while acc < total_tokens:
        n = int(rng.integers(lo, hi, endpoint=True))
        n = min(n, total_tokens - acc)
        lens.append(n)
        acc += n
    return lens


def cu_seqlens(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int  # per-sequence length (dense) or total tokens (varlen)
    H: int
    d: int
    dtype: str
    causal: bool
    varlen: bool = False
    backward: bool = False
    len_range: Optional[tuple] = None


WORKLOADS = {
    "single_head_fwd": Workload("single_head_fwd", 1, 512, 1, 64, "f16", False),
    "gpt2_small_causal_fwd": Workload("gpt2_small_causal_fwd", 1, 1024, 12, 64, "bf16", True),
    "long_seq_fwd": Workload("long_seq_fwd", 4, 8192, 16, 128, "bf16", False),
    "varlen_causal_fwd": Workload("varlen_causal_fwd", 1, 131072, 16, 128, "bf16", True,
                                  varlen=True, len_range=(64, 16384)),
    "train_causal_fwd_bwd": Workload("train_causal_fwd_bwd", 4, 4096, 16, 128, "bf16", True,
                                     backward=True),
}


# FP8 forward workloads (e4m3 inputs, bf16 output): the long-sequence shape, without and
# with the causal mask.
FP8_WORKLOADS = {
    "long_seq_fp8": Workload("long_seq_fp8", 4, 8192, 16, 128, "e4m3", False),
    "long_seq_causal_fp8": Workload("long_seq_causal_fp8", 4, 8192, 16, 128, "e4m3", True),
}


def decode_inputs(B, Nq, Nk, H, d, dtype, seed):
    """Q [B, Nq, H, d] and K, V [B, Nk, H, d] as uint16 bit patterns (seeds +0, +1, +2)."""
    return (normal_bits((B, Nq, H, d), dtype, seed), normal_bits((B, Nk, H, d), dtype, seed + 1),
            normal_bits((B, Nk, H, d), dtype, seed + 2))


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Nq: int  # query rows per sequence (the newest tokens)
    Nk: int  # cached keys and values per sequence
    H: int
    d: int
    dtype: str
    causal: bool


# Decode shapes: one new token after the wiki's batch 4 x 16 heads x 8k sequences, and one
# new token against a single 128k-token context (the long row of the wiki's comparison of
# standard and tiled attention).
DECODE_WORKLOADS = {
    "decode_8k": DecodeWorkload("decode_8k", 4, 1, 8192, 16, 128, "bf16", True),
    "decode_128k": DecodeWorkload("decode_128k", 1, 1, 131072, 16, 128, "bf16", True),
}
