"""Benchmark of the fused attention hot path on one MI355X.

One step = one pass of the whole hot path over resident synthetic inputs:
  * the fused forward on the long causal GQA prefill (B=1, Hq=32, Hkv=8,
    L=8192, D=128, bf16, causal), and
  * the paged decode (64 sequences, Hq=12, Hkv=2, D=128, bf16, context
    lengths uniform in [512, 4096], 16-token blocks, permuted block table).
The per-workload detail also times the paged prefill (16 sequences of 512 new
tokens over paged contexts of 512-4096 tokens, same model shape).
`value` is the forward's throughput in TFLOP/s (4*B*Hq*Lq*Lk*D, halved for
causal), averaged over the timed launches with HIP events on the launch
stream; the decode's HBM GB/s is reported beside it, from a batch of decode
calls issued back to back (as a decode loop issues them) between one pair of
events, with the per-call figure inside the step loop shown too.  The decode
rotates through KV-pool replicas totalling >= 1 GiB so no timed call finds
its K/V in the 256 MB last-level cache.

Before the W warmup steps, untimed steps run for one second so that the timed
ones see the shader clock it settles to under sustained load.  The decode is
also compared with a plain streaming read on the same device
(attn_hbm_read_probe, the attainable HBM rate) of its own size, rotated over
2 GiB, and of 2 GiB; the shader clock is sampled with rocm-smi while a batch of
forward launches runs.  The per-workload detail times each forward over input
replicas totalling at least 1 GiB (up to 64), one per launch in turn, calling
the C ABI with arguments marshalled once per replica; every detail timing
follows half a second of untimed launches of the same workload.

    python bench.py [--gpus 1] [--steps K=100] [--warmup W=10] [--no-cpu] [--no-detail]

Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s + % bf16 MFMA peak (L=2048/8192); paged decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
KV_ROTATION_BYTES = 1 << 30
SETTLE_S = 1.0              # untimed steps before the warmup: the shader clock settles under sustained load
DETAIL_SETTLE_S = 0.5       # untimed launches before each per-workload detail timing


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_flops(B, Hq, Lq, Lk, D, causal):
    f = 4.0 * B * Hq * Lq * Lk * D
    return f / 2 if causal else f


def window_pairs(Lq, Lk, W, causal):
    import numpy as np
    i = np.arange(Lq) + (Lk - Lq)
    hi = np.minimum(i, Lk - 1) if causal else np.minimum(i + W, Lk - 1)
    lo = np.maximum(i - W, 0)
    return int(np.maximum(hi - lo + 1, 0).sum())


def decode_bytes(ctx, Hq, Hkv, D, esize=2):
    import numpy as np
    ctx = np.asarray(ctx, dtype=np.int64)
    S = len(ctx)
    kv = int(ctx.sum()) * Hkv * D * 2 * esize
    return kv + S * Hq * D * esize * 2 + S * Hq * 4 + 4 * int((-(-ctx // 16)).sum()) + 4 * S


FWD_SOURCES = [os.path.join(ROOT, "transformer_attention_09_amd", "csrc", f)
               for f in ("fwd.hip", "common.h", "internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_fwd_kernel_gqa8k_causal.txt")
CALIB_BYTES = 512 << 20   # read, and written, by the calibration multiply


def sources_sha256(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_record():
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary, if it was taken on the current forward kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#") and not line.startswith(" "):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    if rec.get("source_sha256") != sources_sha256(FWD_SOURCES):
        return None
    try:
        return {"workload": rec["workload"], "fetch_bytes": float(rec["fetch_bytes_per_launch"]),
                "write_bytes": float(rec["write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


def write_traffic_record(fetch_csv, write_csv, command):
    """Reduce two rocprofv3 --pmc counter tables (FETCH_SIZE, then WRITE_SIZE,
    both in KiB per dispatch) of a `--copy-calibration` bench run to HBM bytes
    per launch.  Each counter is scaled by the factor that maps its reading on
    the calibration multiply (CALIB_BYTES read and CALIB_BYTES written) to
    those known byte counts."""
    import csv
    import collections

    def per_kernel(path, counter):
        vals = collections.defaultdict(list)
        per = collections.defaultdict(float)
        names = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                per[r["Dispatch_Id"]] += float(r["Counter_Value"])
                names[r["Dispatch_Id"]] = r["Kernel_Name"]
        for d, v in per.items():
            vals[names[d]].append(v)
        return vals

    def pick(vals, key):
        hits = [k for k in vals if key in k and "FillFunctor" not in k]
        if not hits:
            raise SystemExit(f"no dispatch of a kernel matching {key!r}")
        return hits[0], vals[hits[0]]

    out = ["# HBM traffic per launch from rocprofv3 --pmc (FETCH_SIZE and WRITE_SIZE, KiB per dispatch),",
           "# each scaled by its reading on an elementwise multiply that reads and writes 512 MiB.",
           f"workload: gqa8k_causal",
           f"source_sha256: {sources_sha256(FWD_SOURCES)}"]
    for counter, path, tag in (("FETCH_SIZE", fetch_csv, "fetch"), ("WRITE_SIZE", write_csv, "write")):
        vals = per_kernel(path, counter)
        cname, cv = pick(vals, "elementwise")   # the multiply (the fill before it only writes)
        scale = (CALIB_BYTES / 1024.0) / cv[0]
        out.append(f"{tag}_calibration_kernel: {cname[:80]}")
        out.append(f"{tag}_calibration_kib: {cv[0]:.1f} (expected {CALIB_BYTES / 1024:.0f})")
        out.append(f"{tag}_scale: {scale:.4f}")
        for key in ("fwd_kernel", "decode_split_kernel", "decode_combine_kernel"):
            kname, kv = pick(vals, key)
            avg = sum(kv) / len(kv)
            label = {"fwd_kernel": "", "decode_split_kernel": "decode_split_",
                     "decode_combine_kernel": "decode_combine_"}[key]
            out.append(f"{label}{tag}_kib_per_dispatch_raw: {avg:.1f} over {len(kv)} dispatches")
            out.append(f"{label}{tag}_bytes_per_launch: {avg * 1024 * scale:.0f}")
    out.append("commands:")
    for c in command:
        out.append("  " + c)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def host_cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, dcfg, target_s=15.0):
    """The fp64 oracle, as it stands, timed on this host's cores.

    Forward: a bounded sample of the same workload (every query head, an
    evenly spaced subset of query rows sized to about target_s seconds), flops
    counted as for the GPU.  Decode: the whole paged-decode workload, bytes
    counted as for the GPU.  BLAS (the only multi-threaded part of the oracle)
    runs on as many threads as this process may use: the CPUs in its affinity
    mask, capped by OMP_NUM_THREADS when that is set."""
    import numpy as np
    import threadpoolctl

    import oracle
    from workloads import dense_inputs, paged_inputs

    affinity = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    threads = min(affinity, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else affinity

    q, k, v = dense_inputs(cfg)
    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))

    def run(rows):
        t0 = time.perf_counter()
        oracle.attention(q64, k64, v64, cfg.scale, cfg.causal, cfg.window, rows=rows)
        return time.perf_counter() - t0

    def flops(rows):
        i = np.asarray(rows) + (cfg.Lk - cfg.Lq)
        vis = np.minimum(i, cfg.Lk - 1) + 1 if cfg.causal else np.full(len(rows), cfg.Lk)
        return 4.0 * cfg.B * cfg.Hq * cfg.D * float(vis.sum())

    pin = paged_inputs(dcfg)
    with threadpoolctl.threadpool_limits(threads):
        probe = np.arange(0, cfg.Lq, cfg.Lq // 64)
        t_probe = run(probe)
        n = int(min(cfg.Lq, max(64, len(probe) * target_s / max(t_probe, 1e-3))))
        rows = np.unique(np.linspace(0, cfg.Lq - 1, n).astype(np.int64))
        t = run(rows)
        t0 = time.perf_counter()
        oracle.decode_paged(pin.q, pin.k_cache, pin.v_cache, pin.block_table, pin.ctx_lens, dcfg.block_size,
                            dcfg.scale)
        t_dec = time.perf_counter() - t0
    d_bytes = decode_bytes(pin.ctx_lens.numpy(), dcfg.Hq, dcfg.Hkv, dcfg.D)
    return {"value": flops(rows) / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{cfg.name}: {len(rows)} of {cfg.Lq} query rows (evenly spaced), all {cfg.Hq} heads, "
                      f"{t:.1f} s; flops counted as for the GPU (visible keys only)",
            "seconds": t,
            "affinity_cpus": affinity,
            "cpu_model": host_cpu_model(),
            "decode": {"value": d_bytes / t_dec / 1e9, "unit": "GB/s", "seconds": t_dec,
                       "sample": f"{dcfg.name}: all {dcfg.num_seqs} sequences, bytes counted as for the GPU"}}


def read_ceiling(ta, torch, dev, stream, nbytes=2 << 30, reps=5, piece=None):
    """Attainable HBM read rate on this device: plain streaming reads
    (attn_hbm_read_probe) of a 2 GiB buffer, averaged over a few back-to-back
    runs; with `piece`, reads of `piece` bytes each, rotating over the pieces
    of the buffer so that no read finds its data in the 256 MB last-level
    cache (the decode's own size and rotation)."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    size = nbytes if piece is None else (piece // 16) * 16
    parts = [buf[i * size:(i + 1) * size] for i in range(nbytes // size)]
    n = len(parts) * (1 if piece is None else 4)
    reps = reps if piece is None else max(reps, n)
    for i in range(2):
        ta.attn_hbm_read_probe(parts[i % len(parts)], sink, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        ta.attn_hbm_read_probe(parts[i % len(parts)], sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del parts, buf
    return size / (ms * 1e-3) / 1e9


def under_profiler() -> bool:
    """Is this process running under rocprofv3 (its tool library preloaded)?"""
    return any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", "")


def sclk_under_load(run_batch):
    """Shader clock (MHz) reported by rocm-smi while a batch of forward launches
    is running; None if the tool is not available.  Not sampled under a
    profiler: its preloaded library would start the GPU in the child process
    before rocm-smi's interpreter replaces it."""
    import re
    import subprocess
    if under_profiler():
        return None
    run_batch()
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=60)
    except (OSError, subprocess.SubprocessError):
        return None
    m = re.search(r"sclk clock level:\s*\d+:\s*\((\d+)\s*Mhz\)", r.stdout)
    return int(m.group(1)) if m else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-detail", action="store_true", help="skip the extra per-workload numbers")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one elementwise multiply that reads and writes 512 MiB, a dispatch of "
                         "known traffic for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE readings")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic record from two rocprofv3 counter tables and exit (no GPU)")
    ap.add_argument("--traffic-command", action="append", default=[],
                    help="command line to note in the traffic record (repeatable)")
    args = ap.parse_args()
    if args.traffic_record:
        write_traffic_record(args.traffic_record[0], args.traffic_record[1], args.traffic_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards with no exchange over batch/KV-head groups or sequences; "
              "multi-GPU runs are out of scope)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import transformer_attention_09_amd as ta
    from workloads import CONFIGS, dense_inputs, paged_inputs, prefill_inputs

    torch.cuda.set_device(0)
    ta.load_library()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- inputs, resident in HBM before timing
    fcfg = CONFIGS["gqa8k_causal"]
    q, k, v = (t.to(dev) for t in dense_inputs(fcfg))
    out = torch.empty_like(q)
    lse = torch.empty((fcfg.B, fcfg.Hq, fcfg.Lq), dtype=torch.float32, device=dev)
    f_flops = causal_flops(fcfg.B, fcfg.Hq, fcfg.Lq, fcfg.Lk, fcfg.D, fcfg.causal)

    dcfg = CONFIGS["paged_decode"]
    pin = paged_inputs(dcfg)
    kv_bytes = pin.k_cache.numel() * pin.k_cache.element_size() * 2
    n_rep = max(2, math.ceil(KV_ROTATION_BYTES / kv_bytes))
    kcs = [pin.k_cache.to(dev) for _ in range(n_rep)]
    vcs = [pin.v_cache.to(dev) for _ in range(n_rep)]
    dq = pin.q.to(dev)
    bt = pin.block_table.to(dev)
    cl = pin.ctx_lens.to(dev)
    dout = torch.empty_like(dq)
    dlse = torch.empty((dcfg.num_seqs, dcfg.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(ta.attn_decode_paged_workspace_size(dcfg.num_seqs, dcfg.Hq, dcfg.D, pin.max_blocks_per_seq),
                     dtype=torch.uint8, device=dev)
    d_bytes = decode_bytes(pin.ctx_lens.numpy(), dcfg.Hq, dcfg.Hkv, dcfg.D)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        ta.attn_fwd(q, k, v, out=out, lse=lse, scale=fcfg.scale, causal=True, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        r = i % n_rep
        ta.attn_decode_paged(dq, kcs[r], vcs[r], bt, cl, out=dout, lse=dlse, scale=dcfg.scale, workspace=ws,
                             stream=stream)
        if ev is not None:
            ev[2].record(stream)

    # The shader clock under sustained MFMA load takes a few hundred
    # milliseconds to settle (the first launches of a run are the slowest), so
    # untimed steps run for SETTLE_S seconds before the W warmup steps.
    t_settle, n_settle = time.perf_counter(), 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(25):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(n_settle + i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(n_settle + args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_all = [e[0].elapsed_time(e[1]) for e in evs]
    d_all = [e[1].elapsed_time(e[2]) for e in evs]
    f_ms, d_step_ms = float(np.mean(f_all)), float(np.mean(d_all))
    f_med, d_step_med = float(np.median(f_all)), float(np.median(d_all))
    f_tflops = f_flops / (f_ms * 1e-3) / 1e12

    # The decode's rate: the same calls back to back (a decode loop), still
    # rotating over the KV-pool replicas, between one pair of events.  Inside
    # the step loop each decode call also carries the marker of the event
    # recorded after the forward (about 5 us before the first decode kernel
    # starts), which a decode loop does not have; that per-call figure is
    # reported beside it.
    # The batch calls the C ABI directly with the arguments marshalled once
    # per KV replica: a decode call's kernels take about as long as the
    # binding's per-call checks in Python, which would otherwise set the pace.
    n_dec = max(args.steps, 100)
    lib = ta.load_library()
    dec_args = [(dq.data_ptr(), kcs[r].data_ptr(), vcs[r].data_ptr(), bt.data_ptr(), cl.data_ptr(), 16,
                 dout.data_ptr(), dlse.data_ptr(), dcfg.num_seqs, dcfg.Hq, dcfg.Hkv, dcfg.D,
                 pin.max_blocks_per_seq, pin.num_blocks, float(dcfg.scale), ta.ATTN_BF16, ws.data_ptr(),
                 ws.numel(), stream.cuda_stream) for r in range(n_rep)]
    for i in range(n_rep):
        st_ = lib.attn_decode_paged(*dec_args[i])
        if st_ != 0:
            raise RuntimeError(f"attn_decode_paged: {ta.attn_status_string(st_)}")
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record(stream)
    for i in range(n_dec):
        lib.attn_decode_paged(*dec_args[i % n_rep])
    d1.record(stream)
    torch.cuda.synchronize()
    d_ms = d0.elapsed_time(d1) / n_dec
    d_gbs = d_bytes / (d_ms * 1e-3) / 1e9
    log(f"forward {fcfg.name}: {f_ms * 1e3:.1f} us/launch, {f_tflops:.1f} TFLOP/s "
        f"({100 * f_tflops / PEAK_BF16_TFLOPS:.1f}% of peak)")
    log(f"decode: {d_ms * 1e3:.1f} us/call back to back (split + combine), {d_gbs:.0f} GB/s "
        f"({100 * d_gbs / PEAK_HBM_GBS:.1f}% of peak), {n_rep} KV replicas; "
        f"{d_step_ms * 1e3:.1f} us/call inside the step loop")

    trec = traffic_record()

    # shader clock while the forward runs (a batch of about 0.5 s of launches)
    n_batch = max(1, int(500.0 / max(f_ms, 1e-3)))

    def fwd_batch():
        for _ in range(n_batch):
            ta.attn_fwd(q, k, v, out=out, lse=lse, scale=fcfg.scale, causal=True, stream=stream)

    sclk = sclk_under_load(fwd_batch)
    torch.cuda.synchronize()
    ceiling_2g = read_ceiling(ta, torch, dev, stream)
    ceiling = read_ceiling(ta, torch, dev, stream, piece=int(d_bytes))
    log(f"plain streaming read: {ceiling:.0f} GB/s at the decode's size ({d_bytes / 1e6:.0f} MB per read, "
        f"rotated over 2 GiB), {ceiling_2g:.0f} GB/s over 2 GiB; shader clock under forward load: {sclk} MHz")
    traffic = None
    if trec is not None and trec.get("workload") == fcfg.name:
        traffic = trec["fetch_bytes"] + trec["write_bytes"]

    result = {
        "metric": METRIC,
        "value": round(f_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "long causal GQA prefill B=1 Hq=32 Hkv=8 L=8192 D=128 bf16 causal, then paged decode "
                        "64 seqs Hq=12 Hkv=2 D=128 bf16 ctx~U[512,4096] block 16",
            "forward_flops_per_launch": f_flops,
            "decode_bytes_per_call": d_bytes,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(f_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(f_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "fwd_kernel<BF16,128>",
            "avg_launch_us": round(f_ms * 1e3, 2),
            "median_launch_us": round(f_med * 1e3, 2),
            "sclk_mhz_under_load": sclk,
            "settle_steps": n_settle,
        },
        "decode": {
            "value": round(d_gbs, 1),
            "unit": "GB/s",
            "bound": "hbm",
            "peak": PEAK_HBM_GBS,
            "frac": round(d_gbs / PEAK_HBM_GBS, 4),
            "avg_call_us": round(d_ms * 1e3, 2),
            "calls_back_to_back": n_dec,
            "in_step_avg_call_us": round(d_step_ms * 1e3, 2),
            "in_step_median_call_us": round(d_step_med * 1e3, 2),
            "kv_replicas": n_rep,
            "read_ceiling_GBs": round(ceiling, 1),
            "read_ceiling_2GiB_GBs": round(ceiling_2g, 1),
            "frac_of_read_ceiling": round(d_gbs / ceiling, 4),
        },
    }

    if not args.no_detail:
        detail = {}

        def settled_ms(launch, n):
            """Average time of n launches between two events on the launch
            stream, after untimed launches for DETAIL_SETTLE_S seconds: each
            detail workload's inputs are generated on the host first, and the
            shader clock drops while the device waits for them."""
            t_s, k = time.perf_counter(), 0
            while True:
                launch(k)
                k += 1
                if k % 4 == 0:
                    torch.cuda.synchronize()
                    if time.perf_counter() - t_s >= DETAIL_SETTLE_S:
                        break
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n):
                launch(k + i)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        def time_fwd(cfg, iters=10):
            """Average launch time over input replicas totalling >= 1 GiB (at
            most 64 replicas), one replica per launch in turn, so that a
            launch whose inputs fit the 256 MB last-level cache does not find
            them there; returns (ms, replicas)."""
            q0, k0, v0 = dense_inputs(cfg)
            per = (2 * q0.numel() * q0.element_size() + (k0.numel() + v0.numel()) * k0.element_size()
                   + cfg.B * cfg.Hq * cfg.Lq * 4)  # q, k, v, out, lse
            n_rep = max(1, min(64, math.ceil(KV_ROTATION_BYTES / per)))
            reps = [tuple(t.to(dev) for t in (q0, k0, v0)) + (torch.empty(q0.shape, dtype=q0.dtype, device=dev),
                    torch.empty((cfg.B, cfg.Hq, cfg.Lq), dtype=torch.float32, device=dev)) for _ in range(n_rep)]
            n = max(iters, n_rep)
            # The launches go straight to the C ABI with arguments marshalled
            # once per replica: the short kernels here take less time than the
            # binding's per-call checks, which would otherwise set the pace.
            code = ta.ATTN_BF16 if q0.dtype == torch.bfloat16 else ta.ATTN_F16
            fargs = [(qq.data_ptr(), kk.data_ptr(), vv.data_ptr(), o.data_ptr(), l.data_ptr(), cfg.B, cfg.Hq,
                      cfg.Hkv, cfg.Lq, cfg.Lk, cfg.D, float(cfg.scale), int(bool(cfg.causal)), int(cfg.window), code,
                      stream.cuda_stream) for (qq, kk, vv, o, l) in reps]
            for i in range(n_rep):
                st_ = lib.attn_fwd(*fargs[i])
                if st_ != 0:
                    raise RuntimeError(f"attn_fwd ({cfg.name}): {ta.attn_status_string(st_)}")
            ms_ = settled_ms(lambda i: lib.attn_fwd(*fargs[i % n_rep]), n)
            del reps
            return ms_, n_rep

        for name in ("gqa8k_window", "std2048", "std2048_causal", "std512", "std512_causal", "vit", "tiny"):
            cfg = CONFIGS[name]
            ms, n_rep_f = time_fwd(cfg)
            if cfg.window >= 0:
                fl = 4.0 * cfg.B * cfg.Hq * cfg.D * window_pairs(cfg.Lq, cfg.Lk, cfg.window, cfg.causal)
            else:
                fl = causal_flops(cfg.B, cfg.Hq, cfg.Lq, cfg.Lk, cfg.D, cfg.causal)
            byts = 2 * (cfg.B * cfg.Lq * cfg.Hq * cfg.D * 2 + cfg.B * cfg.Lk * cfg.Hkv * cfg.D * 2) \
                + cfg.B * cfg.Hq * cfg.Lq * 4
            detail[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(fl / ms / 1e9, 1),
                            "frac_mfma": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                            "GB/s": round(byts / ms / 1e6, 1), "input_replicas": n_rep_f}
            # attainable roofline min(MFMA peak, AI x HBM peak)
            attain = min(PEAK_BF16_TFLOPS, fl / byts * PEAK_HBM_GBS / 1e3)
            detail[name]["frac_attainable"] = round(fl / ms / 1e9 / attain, 4)
            log(f"detail {name}: {detail[name]}")
        # FP8 (e4m3) forward, bf16 output: the skill page's FP8 shape and the long
        # causal GQA workload; fraction of the dense fp8 MFMA peak
        for name in ("gqa8k_causal_fp8", "fp8_causal"):
            cfg = CONFIGS[name]
            fq, fk, fv = (t.to(dev) for t in dense_inputs(cfg))
            fo = torch.empty(fq.shape, dtype=torch.bfloat16, device=dev)
            fl_ = torch.empty((cfg.B, cfg.Hq, cfg.Lq), dtype=torch.float32, device=dev)
            ms = settled_ms(lambda i: ta.attn_fwd_fp8(fq, fk, fv, out=fo, lse=fl_, scale=cfg.scale,
                                                      causal=cfg.causal, stream=stream), 10)
            fl = causal_flops(cfg.B, cfg.Hq, cfg.Lq, cfg.Lk, cfg.D, cfg.causal)
            detail[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(fl / ms / 1e9, 1),
                            "frac_fp8_mfma": round(fl / ms / 1e9 / PEAK_FP8_TFLOPS, 4)}
            log(f"detail {name}: {detail[name]}")
            del fq, fk, fv, fo, fl_

        # forward with dropout (p = 0.1, the skill page's scenario 2 value) on the
        # long causal GQA workload, beside the plain forward on the same inputs,
        # each after its own settling launches
        dcfg = CONFIGS["gqa8k_causal"]
        dq_, dk_, dv_ = (t.to(dev) for t in dense_inputs(dcfg))
        do_ = torch.empty_like(dq_)
        dl_ = torch.empty((dcfg.B, dcfg.Hq, dcfg.Lq), dtype=torch.float32, device=dev)
        ms = settled_ms(lambda it: ta.attn_fwd_dropout(dq_, dk_, dv_, 0.1, 1234, it, out=do_, lse=dl_,
                                                       scale=dcfg.scale, causal=True, stream=stream), 10)
        ms_plain = settled_ms(lambda it: ta.attn_fwd(dq_, dk_, dv_, out=do_, lse=dl_, scale=dcfg.scale, causal=True,
                                                     stream=stream), 10)
        fl = causal_flops(dcfg.B, dcfg.Hq, dcfg.Lq, dcfg.Lk, dcfg.D, True)
        detail["dropout_gqa8k_causal"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(fl / ms / 1e9, 1),
                                          "frac_mfma": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                          "plain_us": round(ms_plain * 1e3, 2),
                                          "time_vs_plain": round(ms / ms_plain, 3)}
        log(f"detail dropout_gqa8k_causal: {detail['dropout_gqa8k_causal']}")
        del dq_, dk_, dv_, do_, dl_

        # backward (dq, dk, dv) on the long causal GQA workload and the L=2048
        # one; algorithmic flops 2.5x the forward's (the recomputed S plus the
        # dV, dP, dK and dQ products)
        for name in ("gqa8k_causal", "std2048"):
            cfg = CONFIGS[name]
            bq, bk, bv = (t.to(dev) for t in dense_inputs(cfg))
            bo, bl = ta.attn_fwd(bq, bk, bv, scale=cfg.scale, causal=cfg.causal, window=cfg.window, stream=stream)
            bdo = torch.randn_like(bo)
            bdq, bdk, bdv = torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv)
            bws = torch.empty(ta.attn_bwd_workspace_size(cfg.B, cfg.Hq, cfg.Lq), dtype=torch.uint8, device=dev)

            def backward():
                ta.attn_bwd(bq, bk, bv, bo, bdo, bl, dq=bdq, dk=bdk, dv=bdv, scale=cfg.scale, causal=cfg.causal,
                            window=cfg.window, workspace=bws, stream=stream)

            ms = settled_ms(lambda i: backward(), 5)
            fl = 2.5 * causal_flops(cfg.B, cfg.Hq, cfg.Lq, cfg.Lk, cfg.D, cfg.causal)
            detail["bwd_" + name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(fl / ms / 1e9, 1),
                                     "frac_mfma": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
            log(f"detail bwd_{name}: {detail['bwd_' + name]}")
            if name == "gqa8k_causal":
                # the same backward with dropout p = 0.1 (decisions recomputed in both kernels)
                bo, bl = ta.attn_fwd_dropout(bq, bk, bv, 0.1, 1234, 0, scale=cfg.scale, causal=cfg.causal,
                                             stream=stream)

                def backward_drop():
                    ta.attn_bwd_dropout(bq, bk, bv, bo, bdo, bl, 0.1, 1234, 0, dq=bdq, dk=bdk, dv=bdv,
                                        scale=cfg.scale, causal=cfg.causal, workspace=bws, stream=stream)

                ms_d = settled_ms(lambda i: backward_drop(), 5)
                detail["bwd_dropout_" + name] = {"us": round(ms_d * 1e3, 2), "TFLOP/s": round(fl / ms_d / 1e9, 1),
                                                 "frac_mfma": round(fl / ms_d / 1e9 / PEAK_BF16_TFLOPS, 4),
                                                 "time_vs_plain": round(ms_d / ms, 3)}
                log(f"detail bwd_dropout_{name}: {detail['bwd_dropout_' + name]}")
            del bq, bk, bv, bo, bl, bdo, bdq, bdk, bdv, bws

        # paged prefill: 512 new tokens per sequence over paged contexts
        pcfg = CONFIGS["paged_prefill"]
        pin = prefill_inputs(pcfg)
        pq, pkc, pvc, pbt, pcl = (t.to(dev) for t in (pin.q, pin.k_cache, pin.v_cache, pin.block_table,
                                                      pin.ctx_lens))
        pout = torch.empty_like(pq)
        plse = torch.empty((pcfg.B, pcfg.Hq, pcfg.Lq), dtype=torch.float32, device=dev)

        def prefill():
            ta.attn_fwd_paged(pq, pkc, pvc, pbt, pcl, out=pout, lse=plse, scale=pcfg.scale, causal=pcfg.causal,
                              stream=stream)

        ms = settled_ms(lambda i: prefill(), 10)
        ctx = pin.ctx_lens.numpy().astype(np.int64)
        i = np.arange(pcfg.Lq)
        pairs = int(sum(np.clip(c - pcfg.Lq + i + 1, 0, c).sum() for c in ctx))
        fl = 4.0 * pcfg.Hq * pcfg.D * pairs
        byts = (2 * pcfg.B * pcfg.Lq * pcfg.Hq * pcfg.D * 2 + pcfg.B * pcfg.Hq * pcfg.Lq * 4
                + int(ctx.sum()) * pcfg.Hkv * pcfg.D * 2 * 2)
        attain = min(PEAK_BF16_TFLOPS, fl / byts * PEAK_HBM_GBS / 1e3)
        detail["paged_prefill"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(fl / ms / 1e9, 1),
                                   "frac_mfma": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                   "GB/s": round(byts / ms / 1e6, 1),
                                   "frac_attainable": round(fl / ms / 1e9 / attain, 4)}
        log(f"detail paged_prefill: {detail['paged_prefill']}")
        result["detail"] = detail

    if not args.no_cpu:
        log("timing the CPU oracle on a sample ...")
        result["cpu_baseline"] = cpu_baseline(fcfg, CONFIGS["paged_decode"])
        log(f"cpu baseline: {result['cpu_baseline']}")
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
