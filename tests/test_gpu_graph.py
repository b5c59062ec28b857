"""The hot path recorded into a HIP graph (torch.cuda.CUDAGraph): the entry points only
launch kernels on the caller's stream (no allocation, memset or synchronisation inside the
library), so a whole step can be captured once and replayed. One graph holds a dense causal
forward and backward, a packed forward and backward, a split-KV decode and a ring merge;
it is replayed three times, with eager calls of the same step and synchronisations between
the replays, and every replay must give the eager results bit for bit."""
import numpy as np
import pytest

from exact_io_aware_10_amd import inputs
from parity import to_device

pytestmark = pytest.mark.gpu


def fa():
    import exact_io_aware_10_amd as m
    return m


def test_graph_replay_matches_eager():
    import torch
    m = fa()
    print("[graph] dense B1 H12 N1024 d64 causal; packed lens [100,1,300,77] H4 d128 causal; "
          "split-KV B2 Nk5000 H4 d128; merge B1 N700 H4 d128", flush=True)
    q, k, v, do = (to_device(x, "bf16") for x in
                   inputs.attention_inputs(1, 1024, 12, 64, "bf16", 3, with_dout=True))
    lens = [100, 1, 300, 77]
    cu = torch.from_numpy(inputs.cu_seqlens(lens)).cuda()
    T = sum(lens)
    qv, kv, vv, dov = (to_device(inputs.normal_bits((T, 4, 128), "bf16", 70 + i), "bf16")
                       for i in range(4))
    qd = to_device(inputs.normal_bits((2, 1, 4, 128), "bf16", 80), "bf16")
    kd = to_device(inputs.normal_bits((2, 5000, 4, 128), "bf16", 81), "bf16")
    vd = to_device(inputs.normal_bits((2, 5000, 4, 128), "bf16", 82), "bf16")
    o_part = to_device(inputs.normal_bits((1, 700, 4, 128), "bf16", 83), "bf16")
    rng = np.random.default_rng(84)
    lse_part = torch.from_numpy(rng.normal(size=(1, 4, 700)).astype(np.float32)).cuda()
    o_acc0 = torch.from_numpy(rng.normal(size=(1, 700, 4, 128)).astype(np.float32)).cuda()
    lse_acc0 = torch.from_numpy(rng.normal(size=(1, 4, 700)).astype(np.float32)).cuda()
    o_acc, lse_acc = torch.empty_like(o_acc0), torch.empty_like(lse_acc0)

    def reset():
        o_acc.copy_(o_acc0)
        lse_acc.copy_(lse_acc0)

    def step():
        o, lse = m.fa_fwd(q, k, v, causal=True)
        grads = m.fa_bwd(q, k, v, o, lse, do, causal=True)
        ov, lv = m.fa_fwd_varlen(qv, kv, vv, cu, max(lens), causal=True)
        gv = m.fa_bwd_varlen(qv, kv, vv, ov, lv, dov, cu, max(lens), causal=True)
        od, ld = m.fa_fwd_splitkv(qd, kd, vd, causal=True)
        out = torch.empty_like(o_part)
        m.fa_merge(o_acc, lse_acc, o_part, lse_part, out=out)
        return [o, lse, *grads, ov, lv, *gv, od, ld, o_acc, lse_acc, out]

    reset()
    want = [t.clone() for t in step()]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one call on the capture stream before capturing
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g):
        outs = step()
    torch.cuda.synchronize()
    for r in range(3):
        reset()
        g.replay()
        torch.cuda.synchronize()
        for i, (w, x) in enumerate(zip(want, outs)):
            assert torch.equal(w, x), f"replay {r}: output {i} differs from the eager step"
        print(f"  replay {r}: {len(outs)} outputs equal to the eager step", flush=True)
        reset()
        again = step()  # eager work between replays
        torch.cuda.synchronize()
        assert all(torch.equal(w, x) for w, x in zip(want, again))
