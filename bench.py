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

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-clock]
       python bench.py --copy-calibration MIB ...   also runs one plain device-to-device
                                                     copy of MIB MiB before the timed
                                                     region (reference kernel for the HBM
                                                     byte counters FETCH_SIZE/WRITE_SIZE)
       python bench.py --rocprof-summary DB [DB2]   prints a per-kernel table from
                                                     rocprofv3 result databases (kernel
                                                     trace, and counters if collected)
       python bench.py --traffic-summary FETCH_DB WRITE_DB KERNEL MIB
                                                    prints the HBM traffic summary of
                                                    KERNEL from a FETCH_SIZE run and a
                                                    WRITE_SIZE run that both included a
                                                    --copy-calibration MIB copy
       python bench.py --configs                    prints forward and backward times of
                                                    the five parity configurations
       python bench.py --mfma-summary DB            prints, per kernel, the matrix-core
                                                    busy fraction from one run with
                                                    --kernel-trace and the counters
                                                    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA,
                                                    GRBM_GUI_ACTIVE
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
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA peak (vendor figure, no sparsity)
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E peak bandwidth (vendor figure)
BF16_FLOP_PER_CLK_CU = 4096  # dense bf16 MFMA FLOP per clock per CU (4 SIMDs)
CSRC = os.path.join(ROOT, "exact_io_aware_10_amd", "csrc")
KERNEL_SOURCES = {  # the files whose text determines each kernel's code (build.py: flags)
    "decode_kernel": ["fa_decode.hip", "fa_decode.h", "fa_bwd_common.h", "fa_device.h",
                      "fa_internal.h", "../build.py"],
    "decode1_kernel": ["fa_decode.hip", "fa_decode.h", "fa_bwd_common.h", "fa_device.h",
                       "fa_internal.h", "../build.py"],
    "fwd_kernel": ["fa_fwd.hip", "fa_device.h", "fa_internal.h", "../build.py"],
    "fwd_fp8_kernel": ["fa_fwd_fp8.hip", "fa_device.h", "fa_internal.h", "../build.py"],
    "merge_kernel": ["fa_merge.hip", "fa_device.h", "fa_internal.h", "../build.py"],
    "bwd_prep_kernel": ["fa_bwd.hip", "fa_bwd_common.h", "fa_device.h", "fa_internal.h",
                        "../build.py"],
    "bwd_dkdv_kernel": ["fa_bwd_dkdv.hip", "fa_bwd_common.h", "fa_device.h", "fa_internal.h",
                        "../build.py"],
    "bwd_dq_kernel": ["fa_bwd_dq.hip", "fa_bwd_common.h", "fa_device.h", "fa_internal.h",
                      "../build.py"],
}
WORKLOAD = dict(name="long_seq_fwd_bwd", B=4, N=8192, H=16, d=128, dtype="bf16", causal=False)


def fwd_flops(B, N, H, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def bwd_flops(B, N, H, d, causal):
    f = 10.0 * B * H * N * N * d
    return f / 2 if causal else f


def host_cores():
    """(threads the oracle uses, CPUs this process may run on, CPUs of the host)."""
    import oracle
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    return oracle.default_threads(), aff, os.cpu_count() or aff


def parse_sclk_mhz(text):
    """Shader clock in MHz from the output of `rocm-smi --showgpuclocks [--json]`: the first
    card's value of a key naming sclk ("(1640Mhz)", "1 (158Mhz)"), or None if there is none."""
    import re
    num = re.compile(r"(\d+(?:\.\d+)?)\s*mhz", re.I)
    try:  # the JSON object may follow warning lines
        data = json.loads(text[text.index("{"):])
    except ValueError:
        data = None
    if isinstance(data, dict):
        for card in sorted(data):
            fields = data[card]
            if not isinstance(fields, dict):
                continue
            for key, val in fields.items():
                m = num.search(str(val)) if "sclk" in key.lower() else None
                if m:
                    return float(m.group(1))
    for line in text.splitlines():
        m = num.search(line) if "sclk" in line.lower() else None
        if m:
            return float(m.group(1))
    return None


def sustained_clock(step, seconds=2.0, limit_s=30.0):
    """Runs `step` back to back for about `seconds` (at most `limit_s`) and reads the shader
    clock with rocm-smi half-way through, from a second thread (a child process: this one
    keeps the GPU busy). One reading at one moment of the step loop, whichever kernel runs
    then. Returns MHz, or None where rocm-smi is missing or says nothing."""
    import subprocess
    import threading
    import torch
    got = {}

    def probe():
        time.sleep(seconds / 2)
        try:
            r = subprocess.run(["rocm-smi", "--showgpuclocks", "--json"], capture_output=True,
                               text=True, timeout=20)
            got["mhz"] = parse_sclk_mhz(r.stdout)
        except (OSError, subprocess.SubprocessError):
            got["mhz"] = None

    th = threading.Thread(target=probe, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while (th.is_alive() or time.perf_counter() - t0 < seconds) and \
            time.perf_counter() - t0 < limit_s:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    th.join(timeout=1.0)
    return got.get("mhz")


def cpu_baseline(wl, bits, fwd_slices=16, bwd_slices=4):
    """The fp64 oracle timed on the host on a bounded sample of the same workload: the
    forward of the first `fwd_slices` (b, h) slices of the benchmark's inputs, then forward +
    backward of the first `bwd_slices` slices (each slice one complete attention problem).
    Reported as algorithmic TFLOP/s of that sample (same FLOP counts as the GPU metric).
    Sampled because the whole forward alone takes about 52 s on 16 host threads (measured
    on an MI355X host), beyond the ~10-30 s the CPU leg of the benchmark may take; the GPU
    parity tests run the oracle on the whole forward."""
    import oracle

    d, dtype, causal, N = wl["d"], wl["dtype"], wl["causal"], wl["N"]
    scale = 1 / math.sqrt(d)
    nth, aff, ncpu = host_cores()
    w = lambda x: oracle.widen(x, dtype)
    B, H = wl["B"], wl["H"]
    slices = [(b, h) for b in range(B) for h in range(H)]
    sl = lambda x, b, h: np.ascontiguousarray(x[b:b + 1, :, h:h + 1, :])
    # the forward of fwd_slices slices in one call (the oracle's threads span them)
    hs = slices[:fwd_slices]
    take = lambda x: np.concatenate([sl(x, b, h) for b, h in hs], axis=2)
    q, k, v = (w(take(x)) for x in bits[:3])
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, scale, causal, nthreads=nth)
    fwd_s = time.perf_counter() - t0
    del q, k, v
    secs = 0.0
    for b, h in slices[:bwd_slices]:
        q, k, v, do = (w(sl(x, b, h)) for x in bits)
        t0 = time.perf_counter()
        o, lse = oracle.fwd(q, k, v, scale, causal, nthreads=nth)
        oracle.bwd(q, k, v, o, lse, do, scale, causal, nthreads=nth)
        secs += time.perf_counter() - t0
    ff1, bf1 = fwd_flops(1, N, 1, d, causal), bwd_flops(1, N, 1, d, causal)
    flops = fwd_slices * ff1 + bwd_slices * (ff1 + bf1)
    return {"value": round(flops / (fwd_s + secs) / 1e12, 6), "unit": "TFLOP/s",
            "cores": nth, "kind": "oracle",
            "fwd_tflops": round(fwd_slices * ff1 / fwd_s / 1e12, 6),
            "host_cpus_allowed": aff, "host_cpus": ncpu,
            "sample": f"fp64 oracle forward of {fwd_slices} of the {B * H} (b,h) slices of the "
                      f"benchmark's inputs (N={N}, d={d}; {fwd_s:.1f} s), then forward + "
                      f"backward of {bwd_slices} slices ({secs:.1f} s), on {nth} host threads "
                      f"(the process may run on {aff} of the host's {ncpu} CPUs; the thread "
                      f"count is the GPU's share of them, OMP_NUM_THREADS, or at most 16)"}


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    profiles/<kernel>_long_seq_traffic.txt (FETCH_SIZE and WRITE_SIZE, each scaled by what
    the same counter reads for a plain copy of known size), or None when that summary is
    missing or was taken on other kernel source than the current one."""
    return measured_traffic_for(f"{kernel}_long_seq", kernel)


def measured_traffic_for(stem, kernel):
    """measured_traffic for the summary profiles/<stem>_traffic.txt."""
    path = os.path.join(ROOT, "profiles", f"{stem}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k_, v_ = line.split(":", 1)
                vals[k_.strip()] = v_.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def measured_mfma_busy(kernel, stem="long_seq"):
    """Share of the dispatch's cycles in which a SIMD's matrix core is busy, for `kernel`,
    from the committed rocprofv3 counter summary profiles/mfma_busy_<stem>.txt (its
    busy/active column), or None when that summary is missing or was taken on other kernel
    source than the current one."""
    path = os.path.join(ROOT, "profiles", f"mfma_busy_{stem}.txt")
    if not os.path.exists(path):
        return None
    want = kernel_source_hash(kernel)
    ok = False
    with open(path, encoding="utf-8") as f:
        for line in f:
            if line.startswith("# source hash:"):
                ok = f"{kernel}={want}" in line
            elif ok and not line.startswith("#") and f"{kernel}<" in line:
                cols = line.split()
                try:
                    return float(cols[6])
                except (IndexError, ValueError):
                    return None
    return None


def rocprof_summary(paths):
    """Per-kernel summary of rocprofv3 SQLite output: calls, average duration, and the
    average per-dispatch value of every collected counter."""
    import glob
    import sqlite3
    for path in paths:
        dbs = (glob.glob(os.path.join(path, "**", "*.db"), recursive=True)
               if os.path.isdir(path) else glob.glob(path))
        for db in sorted(dbs):
            print(f"# source hash: " + ", ".join(f"{k}={kernel_source_hash(k)}"
                                                 for k in KERNEL_SOURCES))
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


def _counter_values(db_path, counter):
    """{kernel name: [per-dispatch values of `counter`]} from one rocprofv3 database."""
    import glob
    import sqlite3
    dbs = (glob.glob(os.path.join(db_path, "**", "*.db"), recursive=True)
           if os.path.isdir(db_path) else [db_path])
    out = {}
    for db in dbs:
        c = sqlite3.connect(db)
        cols = [r[1] for r in c.execute("pragma table_info(counters_collection)")]
        key = "dispatch_id" if "dispatch_id" in cols else "rowid"
        for name, val in c.execute(f"select kernel_name, sum(value) from counters_collection "
                                   f"where counter_name = ? group by {key}, kernel_name",
                                   (counter,)):
            out.setdefault(name, []).append(val)
    return out


def traffic_summary(fetch_db, write_db, kernels, mib):
    """HBM bytes per launch of the kernels named in `kernels` (comma-separated; the first names
    the source hash), summed: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over the
    dispatches of each kernel), each scaled by (known bytes of the calibration copy) / (what the
    same counter read for it). The calibration copy is the largest copyBuffer dispatch of the
    run; smaller ones are the program's own host-to-device copies."""
    fetch = _counter_values(fetch_db, "FETCH_SIZE")
    write = _counter_values(write_db, "WRITE_SIZE")
    names = kernels.split(",")

    def pick(d, key):
        vals = [v for k, vs in d.items() if key in k for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of {key} in the counter database")
        return vals

    copy_bytes = mib * (1 << 20)
    cf, cw = max(pick(fetch, "copyBuffer")), max(pick(write, "copyBuffer"))
    f_fetch, f_write = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    print(f"kernel: {kernels}")
    print(f"kernel_source_sha256_16: {kernel_source_hash(names[0])}")
    print(f"calibration_copy_bytes: {copy_bytes}")
    print(f"copy_fetch_size_kib: {cf:.1f}")
    print(f"copy_write_size_kib: {cw:.1f}")
    print(f"fetch_scale: {f_fetch:.4f}")
    print(f"write_scale: {f_write:.4f}")
    rd = wr = 0.0
    for n in names:
        kf, kw = pick(fetch, n), pick(write, n)
        kf, kw = sum(kf) / len(kf), sum(kw) / len(kw)
        print(f"{n}.fetch_size_kib_per_dispatch: {kf:.1f}")
        print(f"{n}.write_size_kib_per_dispatch: {kw:.1f}")
        rd += kf * 1024 * f_fetch
        wr += kw * 1024 * f_write
    print(f"hbm_read_bytes_per_launch: {rd:.0f}")
    print(f"hbm_write_bytes_per_launch: {wr:.0f}")
    print(f"hbm_bytes_per_launch: {rd + wr:.0f}")


def mfma_summary(db_path, simds=1024, xcds=8):
    """Matrix-core use per kernel from one rocprofv3 run that collected the kernel trace and
    the counters SQ_VALU_MFMA_BUSY_CYCLES (summed over all SIMDs), SQ_INSTS_MFMA and
    GRBM_GUI_ACTIVE (summed over the XCDs). Per dispatch: MFMA busy cycles per SIMD, active
    cycles per XCD, the clock they imply over the traced duration, and busy / active. MI355X:
    256 CUs of 4 SIMDs in 8 XCDs."""
    import glob
    import sqlite3
    busy = _counter_values(db_path, "SQ_VALU_MFMA_BUSY_CYCLES")
    insts = _counter_values(db_path, "SQ_INSTS_MFMA")
    act = _counter_values(db_path, "GRBM_GUI_ACTIVE")
    dbs = (glob.glob(os.path.join(db_path, "**", "*.db"), recursive=True)
           if os.path.isdir(db_path) else [db_path])
    dur = {}
    for db in dbs:
        for name, d in sqlite3.connect(db).execute("select name, duration from kernels"):
            dur.setdefault(name, []).append(d)
    mean = lambda v: sum(v) / len(v)
    print(f"# source hash: " + ", ".join(f"{k}={kernel_source_hash(k)}" for k in KERNEL_SOURCES))
    print(f"# {simds} SIMDs, {xcds} XCDs")
    print(f"{'calls':>5} {'avg_us':>9} {'mfma_insts':>12} {'busy_per_simd':>14} "
          f"{'active_per_xcd':>15} {'clock_GHz':>9} {'busy/active':>11}  kernel")
    for name in sorted(busy, key=lambda n: -mean(busy[n])):
        b = mean(busy[name])
        if b <= 0 or name not in act or name not in dur:
            continue
        a, t = mean(act[name]) / xcds, mean(dur[name])
        n = mean(insts[name]) if name in insts else float("nan")
        print(f"{len(busy[name]):>5} {t / 1e3:>9.1f} {n:>12.4g} {b / simds:>14.0f} "
              f"{a:>15.0f} {a / t:>9.3f} {b / simds / a:>11.3f}  {name[:100]}")


def configs_table(iters=50, warmup=10):
    """The five parity configurations, each forward and backward call timed with HIP events
    on the current stream: median of `iters` calls after `warmup`. FLOP counts as the
    benchmark's (4 N^2 d per (b, h) forward, 2.5 times that backward, halved under the mask;
    sum of L^2 over the sequences when packed). Prints a text table, not the JSON line."""
    import torch
    import exact_io_aware_10_amd as fa
    from exact_io_aware_10_amd import inputs
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}

    def median_ms(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

    print(f"{'configuration':<68} {'fwd_us':>8} {'fwd_TF/s':>9} {'%peak':>6} {'bwd_us':>8} "
          f"{'bwd_TF/s':>9} {'fwd+bwd_TF/s':>12}")
    for name, wl in inputs.WORKLOADS.items():
        to = lambda x: torch.from_numpy(x.view(np.int16)).view(tdt[wl.dtype]).cuda()
        bits = inputs.attention_inputs(1 if wl.varlen else wl.B, wl.N, wl.H, wl.d, wl.dtype,
                                       0, with_dout=True)
        mask = " causal" if wl.causal else ""
        if wl.varlen:
            lens = inputs.varlen_lengths(wl.N, *wl.len_range, 0)
            cu = torch.from_numpy(inputs.cu_seqlens(lens)).cuda()
            q, k, v, do = (to(x)[0] for x in bits)
            ff = 4.0 * wl.H * wl.d * sum(L * L for L in lens) / (2 if wl.causal else 1)
            fwd = lambda: fa.fa_fwd_varlen(q, k, v, cu, max(lens), causal=wl.causal)
            o, lse = fwd()
            bwd = lambda: fa.fa_bwd_varlen(q, k, v, o, lse, do, cu, max(lens), causal=wl.causal)
            desc = f"packed T={wl.N} ({len(lens)} seqs) H{wl.H} d{wl.d} {wl.dtype}{mask}"
        else:
            q, k, v, do = (to(x) for x in bits)
            ff = fwd_flops(wl.B, wl.N, wl.H, wl.d, wl.causal)
            fwd = lambda: fa.fa_fwd(q, k, v, causal=wl.causal)
            o, lse = fwd()
            bwd = lambda: fa.fa_bwd(q, k, v, o, lse, do, causal=wl.causal)
            desc = f"B{wl.B} H{wl.H} N{wl.N} d{wl.d} {wl.dtype}{mask}"
        tf, tb = median_ms(fwd), median_ms(bwd)
        print(f"{name + ': ' + desc:<68} {tf * 1e3:>8.1f} {ff / tf / 1e9:>9.1f} "
              f"{100 * ff / tf / 1e9 / PEAK_BF16_TFLOPS:>6.1f} {tb * 1e3:>8.1f} "
              f"{2.5 * ff / tb / 1e9:>9.1f} {3.5 * ff / (tf + tb) / 1e9:>12.1f}", flush=True)


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


def decode_bytes(B, Nq, Nk, H, d):
    """Compulsory bytes of one split-KV decode call: K and V once, Q and O once (2 bytes per
    element), LSE (4 bytes per row)."""
    return 2.0 * 2 * B * Nk * H * d + 2.0 * 2 * B * Nq * H * d + 4.0 * B * H * Nq


def decode_cpu_baseline(wl, bits, min_s=10.0):
    """The fp64 oracle on the whole decode workload, repeated for at least min_s seconds."""
    import oracle
    w = [oracle.widen(x, wl.dtype) for x in bits]
    nth = oracle.default_threads()
    scale = 1 / np.sqrt(wl.d)
    reps, secs = 0, 0.0
    while secs < min_s:
        t0 = time.perf_counter()
        oracle.fwd_decode(w[0], w[1], w[2], scale, wl.causal, nthreads=nth)
        secs += time.perf_counter() - t0
        reps += 1
    rate = decode_bytes(wl.B, wl.Nq, wl.Nk, wl.H, wl.d) * reps / secs / 1e9
    return {"value": round(rate, 3), "unit": "GB/s", "cores": nth, "kind": "oracle",
            "sample": f"fp64 oracle decode of the whole workload, {reps} runs in {secs:.1f} s "
                      f"on {nth} host threads"}


def decode_main(args):
    """One JSON line for a decode workload: fa_fwd_splitkv (decode kernel + combine kernel)
    timed with HIP events on its stream, as HBM bandwidth of the compulsory bytes."""
    import torch
    import exact_io_aware_10_amd as fa
    from exact_io_aware_10_amd import inputs

    if args.workload not in inputs.DECODE_WORKLOADS:
        print(f"unknown workload {args.workload}", file=sys.stderr)
        sys.exit(2)
    wl = inputs.DECODE_WORKLOADS[args.workload]
    B, Nq, Nk, H, d = wl.B, wl.Nq, wl.Nk, wl.H, wl.d
    bits = inputs.decode_inputs(B, Nq, Nk, H, d, wl.dtype, 0)
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in bits)
    ws = torch.empty(max(fa.fa_fwd_splitkv_workspace_size(B, Nq, Nk, H, d, 0), 16),
                     dtype=torch.uint8, device="cuda")
    call = lambda: fa.fa_fwd_splitkv(q, k, v, causal=wl.causal, num_splits=0, workspace=ws)
    for _ in range(max(args.warmup, 10)):
        call()
    torch.cuda.synchronize()
    steps = max(args.steps, 50)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
    nbytes = decode_bytes(B, Nq, Nk, H, d)
    gbps = nbytes / (ms * 1e-3) / 1e9
    splits = fa.fa_fwd_splitkv_workspace_size(B, Nq, Nk, H, d, 0) // (B * H * Nq * (d + 2) * 4)
    dk = "decode1_kernel" if Nq == 1 else "decode_kernel"  # the first kernel of the call
    out = {
        "metric": f"split-KV decode HBM GB/s of compulsory bytes, B{B} Nq{Nq} Nk{Nk} H{H} d{d} "
                  f"bf16",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": max(args.warmup, 10), "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "Nq": Nq, "Nk": Nk, "H": H, "d": d,
                   "causal": wl.causal, "splits": int(splits),
                   "step": "fa_fwd_splitkv (decode kernel + combine kernel)"},
        "roofline": {"bound": "hbm", "kernel": f"{dk} + combine_kernel",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic_for(f"splitkv_{wl.name}", dk),
                     "avg_launch_ms": round(ms, 5)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = decode_cpu_baseline(wl, bits)
    print(json.dumps(out))


def fp8_cpu_baseline(wl, codes, descales, min_s=10.0, max_slices=64):
    """The fp64 oracle's FP8 forward (widen the e4m3 codes, apply the descales, plain
    definition) on whole (b, h) slices of the benchmark's inputs, for at least min_s
    seconds or max_slices slices; algorithmic TFLOP/s of the forward."""
    import oracle
    nth = oracle.default_threads()
    scale = 1 / math.sqrt(wl.d)
    done, secs = 0, 0.0
    for b in range(wl.B):
        for h in range(wl.H):
            if secs >= min_s or done >= max_slices:
                break
            sl = [np.ascontiguousarray(c[b:b + 1, :, h:h + 1, :]) for c in codes]
            t0 = time.perf_counter()
            oracle.fwd_fp8(*sl, *descales, scale, wl.causal, nthreads=nth)
            secs += time.perf_counter() - t0
            done += 1
    flops = done * fwd_flops(1, wl.N, 1, wl.d, wl.causal)
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": nth,
            "kind": "oracle",
            "sample": f"fp64 oracle FP8 forward of {done} of the {wl.B * wl.H} (b,h) slices "
                      f"of the benchmark's inputs (N={wl.N}, d={wl.d}), {secs:.1f} s on {nth} "
                      f"host threads"}


def fp8_main(args):
    """One JSON line for an FP8 forward workload: fa_fwd_fp8 timed with HIP events on its
    stream; algorithmic forward FLOP/s against the dense fp8 MFMA peak."""
    import torch
    import exact_io_aware_10_amd as fa
    from exact_io_aware_10_amd import inputs

    wl = inputs.FP8_WORKLOADS[args.workload]
    B, N, H, d = wl.B, wl.N, wl.H, wl.d
    codes, ds = inputs.fp8_inputs(B, N, H, d, 0)
    q, k, v = (torch.from_numpy(c).cuda() for c in codes)
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    call = lambda: fa.fa_fwd_fp8(q, k, v, *ds, causal=wl.causal, out=o, lse=lse)
    for _ in range(max(args.warmup, 5)):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    ff = fwd_flops(B, N, H, d, wl.causal)
    tflops = ff / (ms * 1e-3) / 1e12
    out = {
        "metric": f"attention TFLOP/s fwd, B{B} H{H} N{N} d{d} fp8 e4m3 inputs, bf16 output"
                  + (", causal" if wl.causal else ""),
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": max(args.warmup, 5), "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "N": N, "H": H, "d": d, "causal": wl.causal,
                   "step": "fa_fwd_fp8"},
        "roofline": {"bound": "mfma", "kernel": "fwd_fp8_kernel", "achieved": round(tflops, 2),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic_for(f"fwd_fp8_kernel_{wl.name}",
                                                     "fwd_fp8_kernel"),
                     "avg_launch_ms": round(ms, 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = fp8_cpu_baseline(wl, codes, ds)
    print(json.dumps(out), flush=True)


RING = dict(name="ring_step_16k", B=1, H=16, d=128, chunk=16384, devices=8)


def merge_bytes(B, N, H, d):
    """Compulsory bytes of one fa_merge: o_acc read and written (fp32), o_part read and the
    rounded output written (2 bytes), and per row lse_acc read and written, lse_part read."""
    return B * N * H * (4.0 * d * 2 + 2.0 * d * 2 + 12.0)


def ring_cpu_baseline(q, k, v, c, d, min_s=10.0):
    """The fp64 oracle on a sample of the ring step: for one head after another (until at
    least min_s seconds have passed, at most all of them), the forward of the chunk against
    one K/V chunk, then the merge into a running result."""
    import oracle
    nth = oracle.default_threads()
    H = q.shape[2]
    secs, heads = 0.0, 0
    while heads < H and (heads == 0 or secs < min_s):
        w = [oracle.widen(np.ascontiguousarray(x[:, :, heads:heads + 1, :]), "bf16")
             for x in (q, k, v)]
        t0 = time.perf_counter()
        o, lse = oracle.fwd(w[0], w[1], w[2], 1 / math.sqrt(d), False, nthreads=nth)
        oracle.merge(np.stack([o, o]), np.stack([lse, lse]), nthreads=nth)
        secs += time.perf_counter() - t0
        heads += 1
    return {"value": round(heads * fwd_flops(1, c, 1, d, False) / secs / 1e12, 6),
            "unit": "TFLOP/s", "cores": nth, "kind": "oracle",
            "sample": f"fp64 oracle forward + merge of {heads} of the {H} heads of one ring "
                      f"step (chunk {c}, d={d}), {secs:.1f} s on {nth} host threads"}


def ring_main(args):
    """One JSON line for one device's step of ring attention: fa_fwd of the local query chunk
    against one K/V chunk, then fa_merge into the running fp32 result. Both timed with HIP
    events on their stream."""
    import torch
    import exact_io_aware_10_amd as fa
    from exact_io_aware_10_amd import inputs

    r = RING
    B, H, d, c = r["B"], r["H"], r["d"], r["chunk"]
    bits = inputs.attention_inputs(B, c, H, d, "bf16", 0)
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in bits)
    o_s = torch.empty_like(q)
    l_s = torch.empty((B, H, c), dtype=torch.float32, device="cuda")
    o_acc = torch.zeros((B, c, H, d), dtype=torch.float32, device="cuda")
    l_acc = torch.full((B, H, c), -math.inf, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)

    def step(ev=None):
        if ev:
            ev[0].record()
        fa.fa_fwd(q, k, v, out=o_s, lse=l_s)
        if ev:
            ev[1].record()
        fa.fa_merge(o_acc, l_acc, o_s, l_s, out=out)
        if ev:
            ev[2].record()

    for _ in range(max(args.warmup, 5)):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    f_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    m_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms = sum(e[0].elapsed_time(e[2]) for e in evs) / args.steps
    ff = fwd_flops(B, c, H, d, False)
    mb = merge_bytes(B, c, H, d)
    out_line = {
        "metric": f"ring-attention step TFLOP/s, one device: chunk {c} of a "
                  f"{c * r['devices']}-token ring of {r['devices']}, B{B} H{H} d{d} bf16",
        "value": round(ff / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": max(args.warmup, 5), "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": r["name"], "B": B, "H": H, "d": d, "chunk": c,
                   "devices": r["devices"], "causal": False,
                   "step": "fa_fwd (chunk x chunk) + fa_merge"},
        "fwd_ms": round(f_ms, 4), "merge_ms": round(m_ms, 4),
        "merge_roofline": {"bound": "hbm", "kernel": "merge_kernel",
                           "achieved": round(mb / (m_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": round(mb / (m_ms * 1e-3) / 1e9 /
                                                         PEAK_HBM_GBPS, 4),
                           "traffic": measured_traffic_for(f"merge_kernel_{r['name']}",
                                                           "merge_kernel"),
                           "bytes_per_launch": mb, "avg_launch_ms": round(m_ms, 4)},
        "roofline": {"bound": "mfma", "kernel": "fwd_kernel",
                     "achieved": round(ff / (f_ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ff / (f_ms * 1e-3) / 1e12 /
                                                      PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic_for(f"fwd_kernel_{r['name']}", "fwd_kernel"),
                     "avg_launch_ms": round(f_ms, 4)},
    }
    if not args.no_cpu_baseline:
        out_line["cpu_baseline"] = ring_cpu_baseline(*bits, c, d)
    print(json.dumps(out_line), flush=True)


def main():
    if "--rocprof-summary" in sys.argv:
        rocprof_summary(sys.argv[sys.argv.index("--rocprof-summary") + 1:])
        return
    if "--mfma-summary" in sys.argv:
        mfma_summary(sys.argv[sys.argv.index("--mfma-summary") + 1])
        return
    if "--traffic-summary" in sys.argv:
        i = sys.argv.index("--traffic-summary")
        fdb, wdb, kern, mib = sys.argv[i + 1:i + 5]
        traffic_summary(fdb, wdb, kern, int(mib))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # about 0.8 s of untimed steps at the benchmark shape: long enough for the chip's clock to
    # settle under the power limit (the first few steps after idle ran up to 2% faster on one
    # MI355X and 2% slower on another), so the timed steps measure sustained throughput
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the sustained-clock reading after the timed region")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--configs", action="store_true",
                    help="print a table of the five parity configurations (forward and "
                         "backward times, TFLOP/s) instead of the JSON line")
    ap.add_argument("--workload", default=WORKLOAD["name"],
                    help="long_seq_fwd_bwd (default), a decode workload (decode_8k, "
                         "decode_128k), an FP8 forward workload (long_seq_fp8, "
                         "long_seq_causal_fp8) or one device's ring-attention step "
                         "(ring_step_16k)")
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
    if args.configs:
        configs_table()
        return
    if args.workload in inputs.FP8_WORKLOADS:
        fp8_main(args)
        return
    if args.workload == RING["name"]:
        ring_main(args)
        return
    if args.workload != WORKLOAD["name"]:
        decode_main(args)
        return
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
    grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    # the step: forward, then the backward's three stages (exactly what fa_bwd runs), with
    # an event between launches so each kernel is timed live on the stream it runs on
    stages = [
        ("fwd_kernel", lambda: fa.fa_fwd(q, k, v, causal=causal, out=o, lse=lse)),
        ("bwd_prep_kernel", lambda: fa.fa_bwd_prep(q, k, v, o, lse, do, causal=causal,
                                                   workspace=ws, grads=grads)),
        ("bwd_dkdv_kernel", lambda: fa.fa_bwd_dkdv(q, k, v, o, lse, do, causal=causal,
                                                   workspace=ws, grads=grads)),
        ("bwd_dq_kernel", lambda: fa.fa_bwd_dq(q, k, v, o, lse, do, causal=causal,
                                               workspace=ws, grads=grads)),
    ]

    def step(ev=None):
        for i, (_, fn) in enumerate(stages):
            if ev is not None:
                ev[i].record()
            fn()
        if ev is not None:
            ev[len(stages)].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    avg = lambda xs: sum(xs) / len(xs)
    kms = {name: avg([e[i].elapsed_time(e[i + 1]) for e in evs])
           for i, (name, _) in enumerate(stages)}
    ms = avg([e[0].elapsed_time(e[len(stages)]) for e in evs])
    ff = fwd_flops(B, N, H, d, causal)
    bf = bwd_flops(B, N, H, d, causal)
    tflops = (ff + bf) / (ms * 1e-3) / 1e12
    fwd_tflops = ff / (kms["fwd_kernel"] * 1e-3) / 1e12
    bwd_ms = kms["bwd_prep_kernel"] + kms["bwd_dkdv_kernel"] + kms["bwd_dq_kernel"]

    # algorithmic work per launch: the backward's five N x N x d products are S, dP, dV, dK
    # (all in the dK/dV kernel) and dQ (the dQ kernel's only new product; it recomputes S
    # and dP); the prep kernel is bandwidth work (reads O, dO, LSE; writes two row terms)
    work = {
        "fwd_kernel": ("mfma", ff),
        "bwd_dkdv_kernel": ("mfma", 0.8 * bf),
        "bwd_dq_kernel": ("mfma", 0.2 * bf),
        "bwd_prep_kernel": ("hbm", 2.0 * 2 * B * N * H * d + 4.0 * B * H * N + 8.0 * B * H * N),
    }
    per_kernel = {}
    for name, t in kms.items():
        bound, amount = work[name]
        rate = amount / (t * 1e-3)
        per_kernel[name] = {"ms": round(t, 4), "bound": bound,
                            ("tflops" if bound == "mfma" else "gbps"):
                                round(rate / (1e12 if bound == "mfma" else 1e9), 2)}
    for name in per_kernel:
        busy = measured_mfma_busy(name)
        traffic = measured_traffic(name)
        per_kernel[name]["mfma_busy"] = busy
        per_kernel[name]["hbm_bytes"] = traffic
        per_kernel[name]["hbm_gbps"] = (round(traffic / (kms[name] * 1e-3) / 1e9, 1)
                                        if traffic else None)
    dom = max(kms, key=kms.get)
    bound, amount = work[dom]
    if bound == "mfma":
        achieved, peak, unit = amount / (kms[dom] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = amount / (kms[dom] * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"
    roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(dom), "avg_launch_ms": round(kms[dom], 4)}

    out = {
        "metric": "attention TFLOP/s fwd+bwd, B4 H16 N8192 d128 bf16 (fwd-only in fwd_tflops)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["name"], "B": B, "N": N, "H": H, "d": d, "causal": causal,
                   "step": "fa_fwd + fa_bwd (prep, dkdv, dq)"},
        "fwd_tflops": round(fwd_tflops, 2), "fwd_ms": round(kms["fwd_kernel"], 4),
        "bwd_ms": round(bwd_ms, 4),
        "bwd_tflops": round(bf / (bwd_ms * 1e-3) / 1e12, 2),
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_pct_of_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "kernels": per_kernel,
        "kernel_counters": "mfma_busy: matrix-core busy share of each kernel's cycles "
                           "(profiles/mfma_busy_long_seq.txt); hbm_bytes: HBM bytes per "
                           "launch (profiles/<kernel>_long_seq_traffic.txt), hbm_gbps = "
                           "hbm_bytes / this run's launch time; null where the committed "
                           "counters were taken on other kernel source",
        "wall_s": round(wall, 3),
        "roofline": roofline,
    }
    if not args.no_clock:
        # after the timed region: the chip runs these kernels below the 2.4 GHz that the
        # vendor peak assumes (power-limited), so give the peak at the clock it sustained too
        mhz = sustained_clock(step)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        clock = {"sclk_mhz": mhz, "cus": cus,
                 "how": "rocm-smi --showgpuclocks, one reading half-way through 2 s of "
                        "back-to-back steps after the timed region; bf16 peak at that clock = CUs x clock "
                        "x 4096 FLOP (one 32x32x16 MFMA per SIMD per 32 cycles)"}
        if mhz:
            pk = cus * mhz * 1e6 * BF16_FLOP_PER_CLK_CU / 1e12
            clock.update(bf16_peak_at_sclk=round(pk, 1),
                         step_frac_at_sclk=round(tflops / pk, 4),
                         fwd_frac_at_sclk=round(fwd_tflops / pk, 4))
        out["clock"] = clock
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, bits)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
