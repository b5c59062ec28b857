"""fa_fwd_splitkv_noalloc (its workspace in the library's static scratch array, nothing
allocated by the library) against fa_fwd_splitkv with a caller's workspace: bit-identical
outputs on two calls in a row, the second with a smaller input, both also within the parity
bounds against the fp64 oracle; a request beyond the scratch array is refused."""
import math

import numpy as np
import pytest

import oracle
from exact_io_aware_10_amd import inputs
from parity import assert_close, f64_of, to_device

pytestmark = pytest.mark.gpu

# the decode_8k shape (one new token, B4 H16, 8192 keys), then a smaller request: five query
# rows of fp16 against 1000 keys, three key ranges
CASES = [(4, 1, 8192, 16, 128, "bf16", True, 0), (1, 5, 1000, 2, 64, "f16", True, 3)]


def test_noalloc_matches_workspace_entry_point():
    import torch
    import exact_io_aware_10_amd as fa
    assert fa.fa_noalloc_scratch_bytes() == 8 << 20
    for B, Nq, Nk, H, d, dtype, causal, splits in CASES:
        print(f"[noalloc] B={B} Nq={Nq} Nk={Nk} H={H} d={d} {dtype} causal={causal} "
              f"splits={splits}", flush=True)
        assert fa.fa_fwd_splitkv_workspace_size(B, Nq, Nk, H, d, splits) <= 8 << 20
        qb, kb, vb = inputs.decode_inputs(B, Nq, Nk, H, d, dtype, seed=Nq + Nk)
        q, k, v = (to_device(x, dtype) for x in (qb, kb, vb))
        o1, l1 = fa.fa_fwd_splitkv_noalloc(q, k, v, causal=causal, num_splits=splits)
        o2, l2 = fa.fa_fwd_splitkv(q, k, v, causal=causal, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)
        w = lambda x: oracle.widen(x, dtype)
        ro, rlse = oracle.fwd_decode(w(qb), w(kb), w(vb), 1 / math.sqrt(d), causal)
        assert_close("O", f64_of(o1, dtype), ro)
        assert_close("LSE", l1.cpu().numpy().astype(np.float64), rlse)


def test_noalloc_refuses_requests_beyond_the_scratch_array():
    import torch
    import exact_io_aware_10_amd as fa
    B, Nq, Nk, H, d = 1, 64, 8192, 16, 128  # 256 ranges x 64 rows x 16 heads: 136 MB
    assert fa.fa_fwd_splitkv_workspace_size(B, Nq, Nk, H, d, 4096) > 8 << 20
    q = torch.zeros((B, Nq, H, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Nk, H, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_splitkv_noalloc(q, k, k, num_splits=4096)
    assert e.value.code == 2
