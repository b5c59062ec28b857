"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the CPU oracle.

This module holds no attention arithmetic: it draws i.i.d. N(0, 1) values in fp32 on the
CPU, rounds them to bf16 or fp16 with round-to-nearest-even, and returns the 16-bit
patterns. Each side turns the same bits into its own operands (the oracle widens them to
fp64; the GPU path copies them to device memory). It also draws the packed-sequence
lengths and names the five workloads.

Seeds: Q, K, V and dO use default_rng(seed + 0, 1, 2, 3); sequence lengths use
default_rng(seed + 4).
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array -> uint16 bit patterns of bf16 or fp16, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        lsb = (u >> 16) & 1
        return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal_bits(shape, dtype: str, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return round_to_bits(rng.standard_normal(size=shape, dtype=np.float32), dtype)


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


# Decode shapes: no page gives one, so these follow the benchmark's own sequences: one new
# token after the 8192-token prefill of the long-sequence workload, and one new token against
# the packed workload's 131072 tokens as a single long context.
DECODE_WORKLOADS = {
    "decode_8k": DecodeWorkload("decode_8k", 4, 1, 8192, 16, 128, "bf16", True),
    "decode_128k": DecodeWorkload("decode_128k", 1, 1, 131072, 16, 128, "bf16", True),
}
