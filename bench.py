"""Benchmark of the exact-attention hot path on one MI355X.

One step = one forward (fa_fwd) plus one backward (fa_bwd) of exact attention at
B=4, H=16, N=8192, d=128, bf16, no mask, on seeded synthetic N(0,1) inputs that are
resident in device memory before timing starts.

Prints ONE JSON line: the metric is attention TFLOP/s of forward + backward with the
algorithmic FLOP count 4*B*H*N^2*d for the forward (guide page "FlashAttention 与算子融合",
IO table: 4 B h s^2 d) and 10*B*H*N^2*d for the backward (five N x N x d products:
recomputed S, dV, dP, dQ, dK), halved with the causal mask. Extra fields carry the
forward-only rate, each kernel's live HIP-event timing, the roofline of the dominant
kernel against MI355X's dense bf16 MFMA peak, and the fp64 CPU oracle timed on a bounded
sample of the same workload (the CPU baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --copy-calibration MIB ...   also runs one plain device-to-device
                                                     copy of MIB MiB before the timed
                                                     region (reference kernel for the HBM
                                                     byte counters FETCH_SIZE/WRITE_SIZE)
       python bench.py --rocprof-summary DB [DB2]   prints a per-kernel table from
                                                     rocprofv3 result databases (kernel
                                                     trace, and counters if collected)
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak (vendor figure, no sparsity)
WORKLOAD = dict(name="long_seq_fwd_bwd", B=4, N=8192, H=16, d=128, dtype="bf16", causal=False)


def fwd_flops(B, N, H, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def bwd_flops(B, N, H, d, causal):
    f = 10.0 * B * H * N * N * d
    return f / 2 if causal else f


def cpu_baseline(wl, budget_s=15.0):
    """fp64 oracle (forward + backward) on a bounded sample of the workload: the first
    `rows` query rows of one (b, h) slice for the forward, and the backward of one slice
    at a shortened length. Reported as TFLOP/s of algorithmic work done on the host."""
    import oracle
    from exact_io_aware_10_amd import inputs

    d, dtype = wl["d"], wl["dtype"]
    scale = 1 / math.sqrt(d)
    nth = oracle.default_threads()
    w = lambda x: oracle.widen(x, dtype)
    # forward sample: one full-length (b, h) slice, N keys, all N rows (independent rows)
    n_fwd = wl["N"]
    qb, kb, vb, dob = inputs.attention_inputs(1, n_fwd, 1, d, dtype, 0, with_dout=True)
    q, k, v, do = w(qb), w(kb), w(vb), w(dob)
    done_flops = 0.0
    t0 = time.perf_counter()
    o, lse = oracle.fwd(q, k, v, scale, wl["causal"], nthreads=nth)
    done_flops += fwd_flops(1, n_fwd, 1, d, wl["causal"])
    t_fwd = time.perf_counter() - t0
    # backward sample: one slice at a length that keeps the whole sample near budget_s
    n_bwd = 2048 if t_fwd > budget_s / 4 else 4096
    sl = lambda x: np.ascontiguousarray(x[:, :n_bwd])
    o2, lse2 = oracle.fwd(sl(q), sl(k), sl(v), scale, wl["causal"], nthreads=nth)
    t1 = time.perf_counter()
    oracle.bwd(sl(q), sl(k), sl(v), o2, lse2, sl(do), scale, wl["causal"], nthreads=nth)
    t_bwd = time.perf_counter() - t1
    done_flops += bwd_flops(1, n_bwd, 1, d, wl["causal"])
    secs = t_fwd + t_bwd
    return {"value": round(done_flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": nth,
            "kind": "oracle",
            "sample": f"fp64 oracle on one (b,h) slice: forward at N={n_fwd} "
                      f"({t_fwd:.1f} s) + backward at N={n_bwd} ({t_bwd:.1f} s), d={d}, "
                      f"same algorithmic FLOP count as the GPU metric"}


def rocprof_summary(paths):
    """Per-kernel summary of rocprofv3 SQLite output: calls, average duration, and the
    average per-dispatch value of every collected counter."""
    import glob
    import sqlite3
    for path in paths:
        dbs = (glob.glob(os.path.join(path, "**", "*.db"), recursive=True)
               if os.path.isdir(path) else glob.glob(path))
        for db in sorted(dbs):
            c = sqlite3.connect(db)
            tabs = {r[0] for r in c.execute("select name from sqlite_master")}
            print(f"# {os.path.basename(db)}")
            if "kernels" in tabs and c.execute("select count(*) from kernels").fetchone()[0]:
                rows = c.execute("select name, count(*), avg(duration), sum(duration) from "
                                 "kernels group by name order by sum(duration) desc").fetchall()
                tot = sum(r[3] for r in rows) or 1
                print(f"{'calls':>5} {'avg_us':>10} {'pct':>6}  kernel")
                for name, n, avg, sm in rows:
                    print(f"{n:>5} {avg / 1e3:>10.2f} {100 * sm / tot:>6.2f}  {name[:110]}")
            if "counters_collection" in tabs or "pmc_events" in tabs:
                try:
                    q = ("select kernel_name, counter_name, avg(value), count(*) from "
                         "counters_collection group by kernel_name, counter_name "
                         "order by kernel_name, counter_name")
                    rows = c.execute(q).fetchall()
                except sqlite3.Error:
                    rows = []
                for name, cn, val, n in rows:
                    print(f"  {cn:<32} {val:>16.1f} per dispatch ({n} samples)  {name[:80]}")


def copy_calibration(mib):
    """One plain device copy of `mib` MiB (reads and writes that many bytes)."""
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def main():
    if "--rocprof-summary" in sys.argv:
        rocprof_summary(sys.argv[sys.argv.index("--rocprof-summary") + 1:])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the attention of each (batch, head) is independent: several GPUs would each "
              f"run this same kernel on their share of the heads)", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_io_aware_10_amd as fa
    from exact_io_aware_10_amd import inputs

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    wl = WORKLOAD
    B, N, H, d, dtype, causal = wl["B"], wl["N"], wl["H"], wl["d"], wl["dtype"], wl["causal"]
    dev = torch.device("cuda:0")
    bits = inputs.attention_inputs(B, N, H, d, dtype, seed=0, with_dout=True)
    q, k, v, do = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
                   for x in bits)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(fa.fa_bwd_workspace_size(B, N, H, d), 16), dtype=torch.uint8,
                     device=dev)
    have_bwd = True

    def step(ev=None):
        nonlocal have_bwd
        if ev is not None:
            ev[0].record()
        fa.fa_fwd(q, k, v, causal=causal, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        if have_bwd:
            try:
                fa.fa_bwd(q, k, v, o, lse, do, causal=causal, workspace=ws)
            except fa.FAError:
                have_bwd = False
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    ms = sum(step_ms) / len(step_ms)
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    bwd_avg = sum(bwd_ms) / len(bwd_ms)
    ff = fwd_flops(B, N, H, d, causal)
    bf = bwd_flops(B, N, H, d, causal) if have_bwd else 0.0
    tflops = (ff + bf) / (ms * 1e-3) / 1e12
    fwd_tflops = ff / (fwd_avg * 1e-3) / 1e12

    # dominant kernel: the one with the largest share of the step
    kernels = {"fa_fwd_kernel": (fwd_avg, ff)}
    if have_bwd:
        kernels["fa_bwd"] = (bwd_avg, bf)
    dom = max(kernels, key=lambda n: kernels[n][0])
    dms, dflops = kernels[dom]
    achieved = dflops / (dms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "avg_launch_ms": round(dms, 4)}

    out = {
        "metric": "attention TFLOP/s fwd+bwd, B4 H16 N8192 d128 bf16 (fwd-only in fwd_tflops)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["name"], "B": B, "N": N, "H": H, "d": d, "causal": causal,
                   "step": "fa_fwd + fa_bwd" if have_bwd else "fa_fwd only"},
        "fwd_tflops": round(fwd_tflops, 2), "fwd_ms": round(fwd_avg, 4),
        "bwd_ms": round(bwd_avg, 4) if have_bwd else None,
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_pct_of_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "wall_s": round(wall, 3),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
