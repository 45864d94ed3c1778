#!/usr/bin/env python3
"""Benchmark of the paged KV-cache decode path on one MI355X.

One step is the whole hot path over one batch: the cache write of the batch's
new tokens, the split-context attention pass and the LSE merge.  By default
the step is paged_decode_step, which fuses the three into one launch; the
three-launch form (kv_cache_append + paged_attention_decode_split +
split_reduce) is timed beside it.  The default workload is the batch x context
sweep point B=32, ctx=4096 (Hq=14, Hkv=2, D=64, block_size=16, fp16).

Timing protocol
  * Kernel gate first: a child process runs 32 fused steps and 32
    three-launch steps under rocprofv3 --kernel-trace, and the line records
    whether the library launched exactly the expected kernels, by name, one
    fused kernel per step (three kernels per three-launch step), and their
    traced average durations.
  * R rotation sets: disjoint block ranges of one large pool, each with its own
    block tables and new tokens, R chosen so the K/V bytes of all sets exceed
    4x the 256 MB Infinity Cache; step i uses set i % R, so every call reads
    its K/V from HBM.
  * W untimed warm-up steps and at least 200 ms of warm-up (clock ramp).
  * Steps are launched from HIP graphs (no host launch cost).  The value of
    record: 15 trials, each of at least max(K, 100) steps (graph replays of
    the R consecutive steps), HIP events on the replay stream around each
    trial; p10 / p50 / p90 of the per-step time, value and % of peak from the
    p50.  Exactly K steps (a graph of K steps, replayed once between two
    synchronizations) are timed too and reported beside it.
  * Two read probes over the same bytes per launch: a contiguous streaming
    read (8-16 loads in flight per lane, best grid) and the decode's own K/V
    access pattern with no arithmetic.
  * The fp64 oracle runs on a bounded sample of the same workload on the
    host, with every core of the process's affinity as BLAS threads and with
    one thread, for the CPU baseline.

Prints one JSON line.  --sweep writes per-point lines for the whole
batch x context sweep (unsplit and split) to a file instead.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) and µs/call vs B×ctx"
PEAK_GBS = 8000.0
LLC_BYTES = 256 * 2**20


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--ctx", type=int, default=4096)
    ap.add_argument("--partition", type=int, default=1024, help="split partition size (tokens)")
    ap.add_argument("--waves", type=int, default=0, help="split pass waves/workgroup (0=default)")
    ap.add_argument("--subtiles", type=int, default=0, help="split pass subtiles/tile (0=default)")
    ap.add_argument("--depth", type=int, default=0, help="split pass tiles in flight (0=default)")
    ap.add_argument("--sets", type=int, default=0, help="rotation sets (0 = auto, >= 4x LLC)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the fused step at the larger B x ctx points")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--sweep", default="", help="write the full sweep as JSON lines to this file")
    ap.add_argument("--path", choices=("step", "split"), default="step",
                    help="step: fused paged_decode_step; split: append + split pass + merge")
    ap.add_argument("--prefill", action="store_true",
                    help="time chunked-prefill attention instead (uses --batch, --ctx, --chunk)")
    ap.add_argument("--chunk", type=int, default=512, help="prefill chunk length (tokens)")
    ap.add_argument("--q8", action="store_true",
                    help="time decode over the 8-bit KV cache (at --batch, --ctx)")
    ap.add_argument("--allocator", action="store_true",
                    help="time the host block allocator (no GPU needed)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 20 plain device copies of MIB MiB (a known-size "
                         "reference for HBM traffic counters)")
    ap.add_argument("--trials", type=int, default=15, help="timed trials (p10/p50/p90)")
    ap.add_argument("--no-gate", action="store_true", help="skip the rocprofv3 kernel gate")
    ap.add_argument("--gate-child", action="store_true", help=argparse.SUPPRESS)
    return ap.parse_args()


def alg_bytes(B, ctx_sum, Hq, Hkv, D):
    """K and V of the attended positions + q read + out written (fp16)."""
    return ctx_sum * Hkv * D * 2 * 2 + B * Hq * D * 2 * 2


def split_kernel_bytes(B, ctx_sum, Hq, Hkv, D):
    """Algorithmic bytes of the split pass alone: K/V of the attended
    positions and q (its partials are workspace, not counted)."""
    return ctx_sum * Hkv * D * 2 * 2 + B * Hq * D * 2


def append_bytes(N, Hkv, D):
    return 2 * (2 * N * Hkv * D * 2) + 8 * N


class Rotation:
    """R disjoint copies of one generated batch inside one large pool."""

    def __init__(self, case, R, device):
        import torch
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        NB = case.num_blocks
        self.R = R
        shape = (R * NB,) + case.k_pool.shape[1:]
        self.k_pool = torch.empty(shape, dtype=torch.float16, device=device)
        self.v_pool = torch.empty(shape, dtype=torch.float16, device=device)
        k0, v0 = t(case.k_pool), t(case.v_pool)
        for r in range(R):
            self.k_pool[r * NB:(r + 1) * NB].copy_(k0)
            self.v_pool[r * NB:(r + 1) * NB].copy_(v0)
        del k0, v0
        bt0 = case.block_tables.astype(np.int64)
        self.bt = [t(np.where(bt0 >= 0, bt0 + r * NB, -1).astype(np.int32)) for r in range(R)]
        s0 = case.slot_mapping
        self.slots = [t(np.where(s0 >= 0, s0 + r * NB * case.block_size, -1)) for r in range(R)]
        self.q = t(case.q)
        self.ctx = t(case.context_lens)
        self.k_new = t(case.k_new)
        self.v_new = t(case.v_new)


def host_info():
    """Cores of this process's affinity, the CPU model and numpy's BLAS."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:  # threadpoolctl missing or unable to inspect
        pass
    return cores, model, blas


def time_cpu_oracle(case, seconds, threads):
    """fp64 oracle on a bounded sample of the batch with `threads` BLAS
    threads; returns (GB/s, description of the sample)."""
    from threadpoolctl import threadpool_limits
    from oracle import paged_ref as ref
    nseq = max(1, min(case.B, 4))
    seqs = list(range(nseq))
    done = 0
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        while True:
            ref.paged_attention_decode(case.q, case.k_pool, case.v_pool, case.block_tables,
                                       case.context_lens, case.scale, seqs=seqs)
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    ctx_sample = int(case.context_lens[:nseq].astype(np.int64).sum())
    sample_bytes = alg_bytes(nseq, ctx_sample, case.Hq, case.Hkv, case.D)
    gbs = sample_bytes * done / dt / 1e9
    sample = (f"oracle paged_attention_decode on {nseq} of {case.B} sequences "
              f"({ctx_sample} positions, all {case.Hkv} KV heads) x {done} repeats in "
              f"{dt:.1f} s, fp64, {threads} BLAS thread(s); rate scaled by algorithmic bytes")
    return gbs, sample


def cpu_baseline(case, seconds):
    cores, model, blas = host_info()
    gbs, sample = time_cpu_oracle(case, seconds, cores)
    gbs1, sample1 = time_cpu_oracle(case, seconds, 1)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": sample, "one_thread": {"value": round(gbs1, 4), "sample": sample1},
            "cpu_model": model, "blas": blas}


def capture(fns):
    """One HIP graph holding the launches of fns, in order."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_trials(g, per_replay, K, trials):
    """µs per captured unit over `trials` trials of >= max(K, 100) units
    each (graph replays), HIP events on the replay stream around each trial.
    Returns the sorted per-trial times."""
    import torch
    reps = max(1, math.ceil(max(K, 100) / per_replay))
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    out = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        e1.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / (reps * per_replay))
    return sorted(out)


def pct(sorted_vals, q):
    """Nearest-rank percentile of sorted values."""
    i = min(len(sorted_vals) - 1, max(0, math.ceil(q / 100 * len(sorted_vals)) - 1))
    return sorted_vals[i]


def time_graph(g, per_replay, K):
    """Average µs per captured unit over >= K units of graph replays."""
    import torch
    reps = max(3, math.ceil(K / per_replay))
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * per_replay)


def _probe_lib():
    import ctypes
    lib_path = os.path.join(ROOT, "paged_kv_decode_cache_amd", "libpkv_probe.so")
    if not os.path.exists(lib_path):
        return None
    lib = ctypes.CDLL(lib_path)
    P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.pkv_probe_stream_read.restype = I
    lib.pkv_probe_stream_read.argtypes = [P, L, P, I, I, P]
    lib.pkv_probe_paged_read.restype = I
    lib.pkv_probe_paged_read.argtypes = [P, P, P, I, I, I, I, I, I, P, P]
    lib.pkv_probe_paged_read_q8.restype = I
    lib.pkv_probe_paged_read_q8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P]
    return lib


def probe_read_gbs(rot, nbytes, R, K):
    """Contiguous streaming read of the same byte count per launch, rotating
    through the K/V pool (cold like the kernel's reads); best grid and loads
    in flight.  Returns (GB/s, grid, loads in flight)."""
    import ctypes
    import torch
    lib = _probe_lib()
    if lib is None:
        return None, None, None
    flat = rot.k_pool.view(-1)
    total = flat.numel() * 2
    per = (min(nbytes, total) // 16) * 16     # never past the end of the pool
    sink = torch.zeros(4, dtype=torch.int32, device=flat.device)
    best = (0.0, None, None)
    for grid in (256, 512, 1024, 4096):
        for u in (8, 16):
            def launch(r, grid=grid, u=u):
                off = (r * per) % (total - per) if total > per else 0
                off -= off % 16
                assert off + per <= total
                st = torch.cuda.current_stream().cuda_stream
                rc = lib.pkv_probe_stream_read(ctypes.c_void_p(flat.data_ptr() + off), per,
                                               ctypes.c_void_p(sink.data_ptr()), grid, u,
                                               ctypes.c_void_p(st))
                if rc != 0:
                    raise RuntimeError(f"probe launch failed: {rc}")
            g = capture([lambda r=r: launch(r) for r in range(R)])
            us = time_graph(g, R, K)
            gbs = per / (us * 1e-6) / 1e9
            if gbs > best[0]:
                best = (gbs, grid, u)
    return best


def probe_paged_gbs(rot, case, P, R, K):
    """The decode's own K/V reads (block tables, one head per workgroup,
    whole-line non-temporal loads, two subtiles in flight per wave) with no
    arithmetic, over the same rotation; GB/s on the K/V bytes."""
    import ctypes
    import torch
    lib = _probe_lib()
    if lib is None or case.D != 64 or case.block_size != 16:
        return None
    ctx = int(case.context_lens.max())
    if int(case.context_lens.min()) != ctx:
        return None
    sink = torch.zeros(4, dtype=torch.int32, device=rot.q.device)

    def launch(r):
        st = torch.cuda.current_stream().cuda_stream
        rc = lib.pkv_probe_paged_read(ctypes.c_void_p(rot.k_pool.data_ptr()),
                                      ctypes.c_void_p(rot.v_pool.data_ptr()),
                                      ctypes.c_void_p(rot.bt[r].data_ptr()), case.B, case.Hkv,
                                      ctx, rot.k_pool.shape[0], rot.bt[r].shape[1], P,
                                      ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st))
        if rc != 0:
            raise RuntimeError(f"paged probe launch failed: {rc}")
    us = time_graph(capture([lambda r=r: launch(r) for r in range(R)]), R, K)
    return case.kv_bytes() / (us * 1e-6) / 1e9


KERNEL_SOURCES = ("paged_kv_decode_cache_amd/csrc/pkv_kernels.hpp",
                  "paged_kv_decode_cache_amd/csrc/pkv_api.hip")
Q8_KERNEL_SOURCES = KERNEL_SOURCES + ("paged_kv_decode_cache_amd/csrc/pkv_q8.hpp",)
TRAFFIC_PROFILES = {"step": "profiles/hbm_traffic_decode_step__sweep_B32_ctx4096.md",
                    "split": "profiles/hbm_traffic_attn_split__sweep_B32_ctx4096.md",
                    "q8": "profiles/hbm_traffic_decode_step_q8__sweep_B32_ctx4096.md"}


def profiled_traffic(kernel_name, profile, sources=KERNEL_SOURCES, partition_size=None):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources for this kernel (and, where the summary
    names one, at this partition size); else None."""
    import hashlib
    path = os.path.join(ROOT, profile)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith(("|", "#", "-", "`")):
            k, v = line.strip().split("=", 1)
            kv[k] = v
    h = hashlib.sha256()
    for rel in sources:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    if kv.get("kernel_sources_sha256") != h.hexdigest():
        return None
    if partition_size is not None and f"kernel_p{partition_size}" in kv:
        # a summary may also give the kernel and bytes at other partition sizes
        if kv[f"kernel_p{partition_size}"] != kernel_name:
            return None
        return int(kv[f"traffic_bytes_p{partition_size}"])
    if kv.get("kernel") != kernel_name:
        return None
    if "partition_size" in kv and partition_size is not None and \
            int(kv["partition_size"]) != partition_size:
        return None
    return int(kv["traffic_bytes"])


def copy_calibration(args, device):
    """With --copy-calibration MIB: 20 plain device copies of MIB MiB, a
    known-size reference for the HBM traffic counters of the same run."""
    import torch
    if not args.copy_calibration:
        return
    n = args.copy_calibration << 20
    src = torch.empty(n, dtype=torch.uint8, device=device).random_()
    dst = torch.empty_like(src)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_headline(args, gate=None):
    import torch
    import paged_kv_decode_cache_amd as pkv
    import workloads

    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    copy_calibration(args, device)
    B, ctx = args.batch, args.ctx
    if B in workloads.SWEEP_B and ctx in workloads.SWEEP_CTX:
        case = workloads.sweep_case(B, ctx)
    else:
        case = workloads.sweep_case(B, ctx, seed=3999)
    P = args.partition
    kv_set = case.kv_bytes()
    R = args.sets or max(2, math.ceil(4 * LLC_BYTES / kv_set))
    rot = Rotation(case, R, device)
    Pm = case.max_partitions(P)
    ws = pkv.StepWorkspace(B, case.Hq, case.Hkv, case.D, Pm, device)
    # the three-launch path has its own partials (the step's workspace must
    # keep its "not written" state between calls)
    po = torch.empty_like(ws.partial_out)
    pl = torch.empty_like(ws.partial_lse)
    out = torch.empty((B, case.Hq, case.D), dtype=torch.float16, device=device)
    launch = (dict(waves=args.waves, subtiles=args.subtiles, depth=args.depth)
              if args.waves or args.subtiles or args.depth else None)
    stream = torch.cuda.current_stream(device)

    def fused_step(i):
        r = i % R
        pkv.paged_decode_step(rot.q, rot.k_pool, rot.v_pool, rot.bt[r], rot.ctx, case.scale, P,
                              k_new=rot.k_new, v_new=rot.v_new, slot_mapping=rot.slots[r],
                              workspace=ws, out=out, launch=launch)

    def split_pass(i):
        pkv.paged_attention_decode_split(rot.q, rot.k_pool, rot.v_pool, rot.bt[i % R], rot.ctx,
                                         case.scale, P, Pm, po, pl, launch=launch)

    def three_launch_step(i, ev=None):
        r = i % R
        pkv.kv_cache_append(rot.k_pool, rot.v_pool, rot.k_new, rot.v_new, rot.slots[r])
        if ev is not None:
            ev[0].record(stream)
        split_pass(i)
        if ev is not None:
            ev[1].record(stream)
        pkv.split_reduce(po, pl, rot.ctx, P, out=out)

    fused = args.path == "step"
    step = fused_step if fused else three_launch_step

    # warm-up: W steps of each path and at least 200 ms
    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t0 < 0.2:
        fused_step(i)
        three_launch_step(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    K = args.steps

    # Graph-launched steps: R consecutive steps (one per rotation set) are
    # captured once and replayed; HIP events on the replay stream bracket each
    # trial.  This is the timing of record (no host launch overhead).
    trials = max(1, args.trials)
    g_fused = capture([lambda r=r: fused_step(r) for r in range(R)])
    g_three = capture([lambda r=r: three_launch_step(r) for r in range(R)])
    g_split = capture([lambda r=r: split_pass(r) for r in range(R)])
    fused_t = time_trials(g_fused, R, K, trials)
    three_t = time_trials(g_three, R, K, trials)
    split_t = time_trials(g_split, R, K, trials)
    fused_us, three_us, split_us = pct(fused_t, 50), pct(three_t, 50), pct(split_t, 50)
    step_t = fused_t if fused else three_t

    # Exactly K steps: one graph of K consecutive steps (rotating through the
    # sets), replayed once between two synchronizations.
    g_k = capture([lambda i=i: (fused_step if fused else three_launch_step)(i)
                   for i in range(K)])
    g_k.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g_k.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    k_region_us = e0.elapsed_time(e1) * 1e3 / K
    del g_k

    # Eager launches (Python binding per call), for context.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    eager_step_us = (time.perf_counter() - t0) * 1e6 / K

    # Unsplit decode on the same rotation, graph-launched.
    g_uns = capture([lambda r=r: pkv.paged_attention_decode(
        rot.q, rot.k_pool, rot.v_pool, rot.bt[r], rot.ctx, case.scale, out=out)
        for r in range(R)])
    unsplit_us = time_graph(g_uns, R, K)
    probe, probe_grid, probe_loads = probe_read_gbs(rot, case.kv_bytes(), R, K)
    paged_probe = probe_paged_gbs(rot, case, P, R, K)

    ctx_sum = int(case.context_lens.astype(np.int64).sum())
    step_bytes = alg_bytes(B, ctx_sum, case.Hq, case.Hkv, case.D)
    app_bytes = append_bytes(B, case.Hkv, case.D)
    # the library's default tile: 1 subtile for the fused step, 2 for the split
    # pass at head_dim 64 (an explicit --subtiles applies to both)
    ns_step = args.subtiles or 1
    ns = args.subtiles or (2 if case.D == 64 else 1)
    nw = args.waves or 4
    depth = args.depth or 2
    dual = "true" if case.Hq // case.Hkv <= 8 else "false"
    if fused:
        ms_per_step = fused_us * 1e-3
        kern_us = fused_us
        kbytes = step_bytes + app_bytes
        Pm_s = case.max_partitions(P)
        nw_step = args.waves or step_waves(case.D, B, case.Hkv, Pm_s)
        kname = (f"void pkv::attn_kernel<{case.D}, {ns_step}, {nw_step}, {depth}, "
                 f"{step_mode(Pm_s)}, {dual}>(pkv::AttnParams)")
        step_desc = "paged_decode_step (append + split pass + merge in one launch)"
    else:
        ms_per_step = three_us * 1e-3
        kern_us = split_us
        kbytes = split_kernel_bytes(B, ctx_sum, case.Hq, case.Hkv, case.D)
        kname = f"void pkv::attn_kernel<{case.D}, {ns}, {nw}, {depth}, 1, {dual}>(pkv::AttnParams)"
        step_desc = "kv_cache_append + paged_attention_decode_split + split_reduce"
    tprof = TRAFFIC_PROFILES[args.path]
    traffic = profiled_traffic(kname, tprof) if (B, ctx, P) == (32, 4096, 1024) else None
    achieved = kbytes / (kern_us * 1e-6) / 1e9
    value = (step_bytes + app_bytes) / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"batch x context sweep point B={B} ctx={ctx} (Hq={case.Hq}, "
                        f"Hkv={case.Hkv}, D={case.D}, block_size={case.block_size})",
            "B": B, "ctx": ctx, "Hq": case.Hq, "Hkv": case.Hkv, "D": case.D,
            "block_size": case.block_size, "partition_size": P, "max_partitions": Pm,
            "step": step_desc,
            "rotation_sets": R, "kv_bytes_all_sets": kv_set * R,
            "launch": "HIP graph of R consecutive steps, replayed",
            "algorithmic_bytes_per_step": step_bytes + app_bytes,
            "attention_bytes_per_step": step_bytes,
            "append_bytes_per_step": app_bytes,
            "accumulate": "fp32",
        },
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "roofline": {
            "bound": "hbm",
            "kernel": kname,
            "achieved": round(achieved, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": tprof if traffic else None,
            "kernel_us": round(kern_us, 3),
            "kernel_timing": (f"p50 of {trials} trials, each >= max(K, 100) launches as graph "
                              "replays of R back-to-back launches, HIP events on the replay "
                              "stream"),
            "algorithmic_bytes_per_launch": kbytes,
            "probe_read_gbs": round(probe, 1) if probe else None,
            "probe_read_shape": (f"contiguous grid-stride read, {probe_grid} workgroups x 256 "
                                 f"lanes, {probe_loads} non-temporal 16-byte loads in flight "
                                 "per lane") if probe else None,
            "frac_of_probe": round(achieved / probe, 4) if probe else None,
            "probe_paged_gbs": round(paged_probe, 1) if paged_probe else None,
            "frac_of_paged_probe": round(achieved / paged_probe, 4) if paged_probe else None,
        },
        "timing": {
            "trials": trials,
            "steps_per_trial": R * max(1, math.ceil(max(K, 100) / R)),
            "us_per_step_p10": round(pct(step_t, 10), 3),
            "us_per_step_p50": round(pct(step_t, 50), 3),
            "us_per_step_p90": round(pct(step_t, 90), 3),
            "exactly_K_steps_us_per_step": round(k_region_us, 3),
            "exactly_K_steps": "one graph of K consecutive steps, replayed once between two "
                               "synchronizations, HIP events around the replay",
        },
        "eager_us_per_step": round(eager_step_us, 3),
        "three_launch_step_us": round(three_us, 3),
        "split_pass_us": round(split_us, 3),
        "split_pass_gbs": round(split_kernel_bytes(B, ctx_sum, case.Hq, case.Hkv, case.D)
                                / (split_us * 1e-6) / 1e9, 1),
        "fused_step_us": round(fused_us, 3),
        "unsplit_decode_us": round(unsplit_us, 3),
        "unsplit_decode_gbs": round(step_bytes / (unsplit_us * 1e-6) / 1e9, 1),
    }
    if gate is not None:
        res["kernel_gate"] = gate
        if fused and gate.get("fused_kernel_traced_avg_us"):
            res["roofline"]["kernel_traced_avg_us"] = gate["fused_kernel_traced_avg_us"]
    if not args.no_large and (B, ctx, P) == (32, 4096, 1024):
        del g_fused, g_three, g_split, g_uns, rot, ws, po, pl
        torch.cuda.empty_cache()
        res["large_points"] = time_large_points(trials, K, device)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    return res


# Larger points of the sweep's shapes inside B >= 32, ctx >= 4096, each with the
# fused step's best partition size in the sweep.
LARGE_POINTS = ((64, 8192, 4096), (128, 8192, 4096), (256, 8192, 4096))


def time_large_points(trials, K, device):
    """The fused step at LARGE_POINTS, timed as the headline (rotation over
    >= 4x the Infinity Cache, graph replays, p50 of the trials)."""
    import torch
    import paged_kv_decode_cache_amd as pkv
    import workloads
    out_lines = []
    for B, ctx, P in LARGE_POINTS:
        case = workloads.extra_case(B, ctx)
        R = max(2, math.ceil(4 * LLC_BYTES / case.kv_bytes()))
        rot = Rotation(case, R, device)
        ws = pkv.StepWorkspace(B, case.Hq, case.Hkv, case.D, case.max_partitions(P), device)
        out = torch.empty((B, case.Hq, case.D), dtype=torch.float16, device=device)

        def step(i, rot=rot, ws=ws, out=out, case=case, P=P, R=R):
            r = i % R
            pkv.paged_decode_step(rot.q, rot.k_pool, rot.v_pool, rot.bt[r], rot.ctx, case.scale,
                                  P, k_new=rot.k_new, v_new=rot.v_new, slot_mapping=rot.slots[r],
                                  workspace=ws, out=out)
        for i in range(2 * R):
            step(i)
        torch.cuda.synchronize()
        g = capture([lambda r=r: step(r) for r in range(R)])
        t = time_trials(g, R, K, trials)
        ctx_sum = int(case.context_lens.astype(np.int64).sum())
        nbytes = alg_bytes(B, ctx_sum, case.Hq, case.Hkv, case.D) + append_bytes(B, case.Hkv,
                                                                                 case.D)
        us = pct(t, 50)
        out_lines.append({"B": B, "ctx": ctx, "partition_size": P, "rotation_sets": R,
                          "algorithmic_bytes_per_step": nbytes,
                          "us_per_step_p10": round(pct(t, 10), 3),
                          "us_per_step_p50": round(us, 3),
                          "us_per_step_p90": round(pct(t, 90), 3),
                          "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "pct_of_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / PEAK_GBS, 2)})
        del g, rot, ws, out
        torch.cuda.empty_cache()
    return out_lines


PREFILL_METRIC = "chunked prefill attention: achieved TFLOP/s (% of fp16 MFMA peak) and µs/call"
PEAK_FP16_TFLOPS = 2500.0


def prefill_flops(case):
    """Useful flops of a chunked-prefill call: q.K and p.V over each row's
    causal prefix (2 flops per multiply-add, 2 products per position)."""
    total = 0
    for b in range(case.B):
        n = int(case.chunk_lens[b])
        ctx = int(case.context_lens[b])
        first = max(0, ctx - n)          # positions of the chunk rows, +1 each
        seen = sum(p + 1 for p in range(first, ctx))
        total += seen
    return 4 * case.Hq * case.D * total


def run_prefill(args):
    """Chunked prefill: B sequences, each a `--chunk`-token chunk ending at
    position ctx - 1 (Hq=14, Hkv=2, D=64, bs=16).  The kernel is bound by
    MFMA/VALU issue, not HBM (~3000 flop per K/V byte at 512-row chunks), so
    the K/V set (16.8 MB at B=8, ctx=4096) is not rotated."""
    import torch
    import paged_kv_decode_cache_amd as pkv
    import workloads

    device = torch.device("cuda:0")
    B, ctx, n = args.batch, args.ctx, args.chunk
    case = workloads.prefill_case(f"prefill_B{B}_ctx{ctx}_chunk{n}", Hq=14, Hkv=2, D=64,
                                  block_size=16, ctx=[ctx] * B, chunk=[n] * B, seed=6000)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    q, kp, vp = t(case.q), t(case.k_pool), t(case.v_pool)
    bt, cl, qs = t(case.block_tables), t(case.context_lens), t(case.query_start)
    out = torch.empty_like(q)

    def call(_i):
        pkv.paged_attention_prefill(q, kp, vp, bt, cl, qs, case.scale, case.max_q, out=out)

    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t0 < 0.2:
        call(i)
        i += 1
    torch.cuda.synchronize()
    R = 16
    us_whole = time_graph(capture([lambda r=r: call(r) for r in range(R)]), R, args.steps)

    # the split over context partitions: split pass + split_reduce (two
    # launches), and the split pass alone, at the best partition size
    maxb = case.block_tables.shape[1]
    T = case.total_q
    split = None
    for P in (256, 512, 1024, 2048):
        if P > ctx:
            continue
        Pm = pkv.max_partitions_for(maxb, case.block_size, P)
        po = torch.empty((T, case.Hq, Pm, case.D), dtype=torch.float32, device=device)
        pl = torch.empty((T, case.Hq, Pm), dtype=torch.float32, device=device)
        rl = torch.zeros((T,), dtype=torch.int32, device=device)

        def split_pass(_i, P=P, Pm=Pm, po=po, pl=pl, rl=rl):
            pkv.paged_attention_prefill_split(q, kp, vp, bt, cl, qs, case.scale, case.max_q, P,
                                              Pm, partial_out=po, partial_lse=pl,
                                              row_context_lens=rl)

        def split_merged(i, P=P, po=po, pl=pl, rl=rl, split_pass=split_pass):
            split_pass(i)
            pkv.split_reduce(po, pl, rl, P, out=out)

        us_sm = time_graph(capture([lambda r=r: split_merged(r) for r in range(R)]), R,
                           args.steps)
        us_sp = time_graph(capture([lambda r=r: split_pass(r) for r in range(R)]), R,
                           args.steps)
        if split is None or us_sm < split[1]:
            split = (P, us_sm, us_sp, Pm)
    flops = prefill_flops(case)
    # the library gives launches with fewer workgroups than CUs 8 waves each
    rows_per_wg = 16 * 4 // (case.Hq // case.Hkv)
    q_tiles = -(-case.max_q // rows_per_wg)
    grid = case.B * case.Hkv * q_tiles
    use_split = split is not None and split[1] < us_whole
    if use_split:
        grid *= split[3]
    nw = 8 if grid < 256 else 4
    kname = f"void pkv::prefill_kernel<64, 4, {nw}, 2, {'true' if use_split else 'false'}>" \
            "(pkv::PrefillParams)"
    us = split[1] if use_split else us_whole
    kernel_us = split[2] if use_split else us_whole
    kv = case.B * ctx * case.Hkv * case.D * 4
    qo = case.total_q * case.Hq * case.D * 4
    tflops = flops / (us * 1e-6) / 1e12
    kernel_tflops = flops / (kernel_us * 1e-6) / 1e12
    res = {
        "metric": PREFILL_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us * 1e-3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"chunked prefill: {B} sequences x {n}-token chunk ending at "
                               f"position {ctx - 1} (Hq=14, Hkv=2, D=64, block_size=16)",
                   "B": B, "ctx": ctx, "chunk": n, "useful_flops_per_call": flops,
                   "kv_bytes_per_call": kv, "q_out_bytes_per_call": qo,
                   "path": (f"paged_attention_prefill_split (partition {split[0]}) + "
                            "split_reduce" if use_split else "paged_attention_prefill"),
                   "launch": "HIP graph of 16 calls, replayed", "accumulate": "fp32"},
        "us_per_call": round(us, 3),
        "roofline": {"bound": "mfma", "kernel": kname,
                     "achieved": round(kernel_tflops, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kernel_tflops / PEAK_FP16_TFLOPS, 4),
                     "traffic": None, "kernel_us": round(kernel_us, 3),
                     "hbm_gbs_on_kv_and_q_out": round((kv + qo) / (kernel_us * 1e-6) / 1e9, 1)},
        "whole_context_us": round(us_whole, 3),
        "split_merged_us": round(split[1], 3) if split else None,
        "split_pass_us": round(split[2], 3) if split else None,
        "split_best_partition": split[0] if split else None,
    }
    if not args.no_cpu:
        from threadpoolctl import threadpool_limits
        from oracle import paged_ref as ref
        rows = min(n, 32)
        sub_qs = np.array([0, rows], dtype=np.int32)
        q1 = case.q[int(case.query_start[0]):int(case.query_start[0]) + rows]
        ctx1 = np.array([ctx - n + rows], dtype=np.int32)   # the chunk's first rows
        sub = workloads.PrefillCase(case.name, 1, case.Hq, case.Hkv, case.D, case.block_size,
                                    case.num_blocks, case.scale, ctx1, sub_qs,
                                    case.block_tables[:1], case.k_pool, case.v_pool, q1,
                                    case.k_chunk[:rows], case.v_chunk[:rows],
                                    case.chunk_slots[:rows])
        done = 0
        t0 = time.perf_counter()
        with threadpool_limits(limits=1):
            while True:
                ref.paged_attention_prefill(q1, case.k_pool, case.v_pool, case.block_tables[:1],
                                            ctx1, sub_qs, case.scale)
                done += 1
                if time.perf_counter() - t0 >= args.cpu_seconds:
                    break
        dt = time.perf_counter() - t0
        cpu = prefill_flops(sub) * done / dt / 1e12
        res["cpu_baseline"] = {
            "value": round(cpu, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle paged_attention_prefill on the first {rows} rows of one "
                      f"sequence's chunk x {done} repeats in {dt:.1f} s, fp64, one thread"}
    return res


Q8_METRIC = ("paged decode attention over an 8-bit KV cache: achieved HBM GB/s "
             "(% of peak) and µs/call")


def q8_bytes(B, ctx_sum, Hq, Hkv, D):
    """Algorithmic bytes of decode over the 8-bit cache: int8 codes and fp32
    scales of the attended K/V rows, q read and out written (fp16)."""
    return ctx_sum * Hkv * (D + 4) * 2 + B * Hq * D * 2 * 2


def run_q8(args):
    """Decode over the 8-bit cache at the sweep point B x ctx (Hq=14, Hkv=2,
    D=64, bs=16): the step (quantising append + split pass + merge, three
    launches), the split pass alone and the unsplit kernel, rotated over
    >= 4x the Infinity Cache and graph-timed."""
    import torch
    import paged_kv_decode_cache_amd as pkv
    import workloads

    device = torch.device("cuda:0")
    copy_calibration(args, device)
    B, ctx = args.batch, args.ctx
    case = (workloads.sweep_case(B, ctx) if B in workloads.SWEEP_B and ctx in workloads.SWEEP_CTX
            else workloads.sweep_case(B, ctx, seed=3999))
    kc, vc, ks, vs = workloads.q8_pools(case)
    NB = case.num_blocks
    ctx_sum = int(case.context_lens.astype(np.int64).sum())
    set_bytes = ctx_sum * case.Hkv * (case.D + 4) * 2
    R = args.sets or min(64, max(2, math.ceil(4 * LLC_BYTES / set_bytes)))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    # codes in the library's head-major layout [NB, Hkv, bs, D]
    codes_k = torch.empty((R * NB, case.Hkv, case.block_size, case.D), dtype=torch.int8,
                          device=device)
    codes_v = torch.empty_like(codes_k)
    sc_k = torch.empty((R * NB, case.Hkv, case.block_size), dtype=torch.float32, device=device)
    sc_v = torch.empty_like(sc_k)
    k0, v0 = t(kc.transpose(0, 2, 1, 3)), t(vc.transpose(0, 2, 1, 3))
    ks0, vs0 = t(ks.transpose(0, 2, 1)), t(vs.transpose(0, 2, 1))
    for r in range(R):
        codes_k[r * NB:(r + 1) * NB].copy_(k0)
        codes_v[r * NB:(r + 1) * NB].copy_(v0)
        sc_k[r * NB:(r + 1) * NB].copy_(ks0)
        sc_v[r * NB:(r + 1) * NB].copy_(vs0)
    del k0, v0, ks0, vs0
    bt0 = case.block_tables.astype(np.int64)
    bt = [t(np.where(bt0 >= 0, bt0 + r * NB, -1).astype(np.int32)) for r in range(R)]
    s0 = case.slot_mapping
    slots = [t(np.where(s0 >= 0, s0 + r * NB * case.block_size, -1)) for r in range(R)]
    q, k_new, v_new, cl = t(case.q), t(case.k_new), t(case.v_new), t(case.context_lens)
    out = torch.empty((B, case.Hq, case.D), dtype=torch.float16, device=device)
    pools = (codes_k, codes_v, sc_k, sc_v)

    def split_pass(i, P, Pm, po, pl):
        pkv.paged_attention_decode_split_q8(q, *pools, bt[i % R], cl, case.scale, P, Pm, po, pl)

    def step(i, P, Pm, po, pl):
        pkv.kv_cache_append_q8(*pools, k_new, v_new, slots[i % R])
        split_pass(i, P, Pm, po, pl)
        pkv.split_reduce(po, pl, cl, P, out=out)

    def unsplit(i):
        pkv.paged_attention_decode_q8(q, *pools, bt[i % R], cl, case.scale, out=out)

    def fused_step(i, P, ws):
        pkv.paged_decode_step_q8(q, *pools, bt[i % R], cl, case.scale, P, k_new=k_new,
                                 v_new=v_new, slot_mapping=slots[i % R], workspace=ws, out=out)

    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t0 < 0.2:
        unsplit(i)
        i += 1
    torch.cuda.synchronize()
    K = args.steps
    time_it = lambda fn: time_graph(capture([lambda r=r: fn(r) for r in range(R)]), R, K)
    # each path at its best partition size: the fused step (the step of
    # record), the three-launch step and the split pass alone
    best, best3, best_split = None, None, None
    for P in [P for P in (256, 512, 1024, 2048, 4096) if P == 256 or P <= int(case.context_lens.max())]:
        Pm = case.max_partitions(P)
        po = torch.empty((B, case.Hq, Pm, case.D), dtype=torch.float32, device=device)
        pl = torch.empty((B, case.Hq, Pm), dtype=torch.float32, device=device)
        ws = pkv.StepWorkspace(B, case.Hq, case.Hkv, case.D, Pm, device)
        us_fused = time_it(lambda r: fused_step(r, P, ws))
        us_three = time_it(lambda r: step(r, P, Pm, po, pl))
        us_split = time_it(lambda r: split_pass(r, P, Pm, po, pl))
        if best is None or us_fused < best[1]:
            best = (P, us_fused)
        if best3 is None or us_three < best3[1]:
            best3 = (P, us_three)
        if best_split is None or us_split < best_split[1]:
            best_split = (P, us_split)
    us_unsplit = time_it(unsplit)
    # the split pass's code and scale reads through the tables with no
    # arithmetic (a 4-wave read per partition), at its fastest partition size
    probe_us, probe_P = None, None
    plib = _probe_lib()
    if plib is not None and case.D == 64 and case.block_size == 16 and \
            int(case.context_lens.min()) == int(case.context_lens.max()):
        import ctypes
        sink = torch.zeros(4, dtype=torch.int32, device=device)
        vp = lambda x: ctypes.c_void_p(x.data_ptr())

        def probe(r, P):
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            rc = plib.pkv_probe_paged_read_q8(vp(codes_k), vp(codes_v), vp(sc_k), vp(sc_v),
                                              vp(bt[r]), B, case.Hkv, ctx, R * NB,
                                              bt[r].shape[1], P, vp(sink), st)
            if rc != 0:
                raise RuntimeError(f"8-bit paged probe launch failed: {rc}")
        for Pp in (256, 512, 1024):
            us = time_it(lambda r, Pp=Pp: probe(r, Pp))
            if probe_us is None or us < probe_us:
                probe_us, probe_P = us, Pp
    P, us_step = best
    step_bytes = q8_bytes(B, ctx_sum, case.Hq, case.Hkv, case.D)
    app = 2 * B * case.Hkv * (case.D * 2 + case.D + 4) + 8 * B   # fp16 in, codes + scale out
    value = (step_bytes + app) / (us_step * 1e-6) / 1e9
    fp16_bytes = alg_bytes(B, ctx_sum, case.Hq, case.Hkv, case.D)
    G = case.Hq // case.Hkv
    nw8 = 8 if case.D == 64 and step_mode(case.max_partitions(P)) == 4 else \
        step_waves(case.D, B, case.Hkv, case.max_partitions(P))
    q8_kernel = (f"void pkv::attn_q8_kernel<{case.D}, {2 if case.D == 64 and nw8 == 4 else 1}, "
                 f"{nw8}, 2, {step_mode(case.max_partitions(P))}, "
                 f"{'true' if G <= 8 else 'false'}>(pkv::Q8Params)")
    traffic = (profiled_traffic(q8_kernel, TRAFFIC_PROFILES["q8"], Q8_KERNEL_SOURCES, P)
               if (B, ctx) == (32, 4096) and case.D == 64 else None)
    res = {
        "metric": Q8_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(us_step * 1e-3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8/f16",
        "data": "synthetic",
        "config": {"workload": f"batch x context sweep point B={B} ctx={ctx} (Hq={case.Hq}, "
                               f"Hkv={case.Hkv}, D={case.D}, block_size={case.block_size}), "
                               "8-bit cache (int8 codes, fp32 scale per token and head)",
                   "partition_size": P, "rotation_sets": R,
                   "step": "paged_decode_step_q8 (quantising append + split pass + merge in "
                           "one launch)",
                   "algorithmic_bytes_per_step": step_bytes + app,
                   "fp16_cache_bytes_for_comparison": fp16_bytes,
                   "launch": "HIP graph of R consecutive steps, replayed"},
        "us_per_step": round(us_step, 3),
        "roofline": {"bound": "hbm", "kernel": q8_kernel,
                     "achieved": round(value, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / PEAK_GBS, 4), "traffic": traffic,
                     "kernel_us": round(us_step, 3),
                     "kernel_timing": "HIP events around graph replays of R back-to-back "
                                      "launches",
                     "algorithmic_bytes_per_launch": step_bytes + app},
        "three_launch_step_us": round(best3[1], 3),
        "three_launch_best_partition": best3[0],
        "split_pass_us": round(best_split[1], 3),
        "split_pass_best_partition": best_split[0],
        "unsplit_decode_us": round(us_unsplit, 3),
        "unsplit_decode_gbs": round(step_bytes / (us_unsplit * 1e-6) / 1e9, 1),
        "probe_paged_q8_us": None if probe_us is None else round(probe_us, 3),
        "probe_paged_q8_partition": probe_P,
        "probe_paged_q8_gbs": (None if probe_us is None else
                               round(ctx_sum * case.Hkv * (case.D + 4) * 2 /
                                     (probe_us * 1e-6) / 1e9, 1)),
        "probe_paged_q8_shape": "the split pass's code and scale reads through the block "
                                "tables (4 waves per workgroup, two subtiles in flight, "
                                "one 16-byte load per lane per 1 KiB of codes), no arithmetic",
    }
    return res


def run_allocator(args):
    """Host block allocator (C ABI, host memory): µs per decode-step build for
    256 sequences (each grows by one token; slots, tables of width 256 and
    lengths written out) and per prefill build (256 chunks of 16 tokens),
    with the plain-Python reference model timed on the same operations."""
    import paged_kv_decode_cache_amd as pkv
    from oracle.block_alloc_ref import BlockAllocatorRef

    B, W, bs = 256, 256, 16
    NB = B * W
    seqs = list(range(B))

    def drive(alloc, decode, prefill, free, steps):
        t_dec = t_pre = 0.0
        n_dec = n_pre = 0
        for i in range(steps):
            if i % 200 == 0:                 # restart every sequence with a chunk
                for s in seqs:
                    free(s)
                t0 = time.perf_counter()
                prefill(seqs, [16] * B, W)
                t_pre += time.perf_counter() - t0
                n_pre += 1
            t0 = time.perf_counter()
            decode(seqs, W)
            t_dec += time.perf_counter() - t0
            n_dec += 1
        return t_dec / n_dec * 1e6, t_pre / n_pre * 1e6

    lib = pkv.BlockAllocator(NB, bs, B, W)
    lib_dec, lib_pre = drive(lib, lib.decode_batch, lib.prefill_batch, lib.free, args.steps * 4)
    m = BlockAllocatorRef(NB, bs, B, W)
    ref_dec, ref_pre = drive(m, m.decode_batch, m.prefill_batch, m.free_seq, 400)
    return {
        "metric": "host block allocator: µs per decode-step build", "value": round(lib_dec, 3),
        "unit": "µs", "n_gpus": 0, "steps": args.steps * 4, "warmup": 0,
        "ms_per_step": round(lib_dec * 1e-3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32/int64", "data": "synthetic",
        "config": {"workload": f"{B} sequences grown one token per step, tables of width {W} "
                               f"(block_size {bs}); every 200 steps all restart with a "
                               f"16-token chunk", "B": B, "width": W, "block_size": bs},
        "prefill_build_us": round(lib_pre, 3),
        "roofline": None,
        "cpu_baseline": {"value": round(ref_dec, 3), "unit": "µs", "cores": 1,
                         "kind": "oracle",
                         "sample": f"plain-Python reference model, 400 decode builds; "
                                   f"prefill build {ref_pre:.1f} µs"},
    }


def run_sweep(args):
    """Every batch x context point plus the other workloads: unsplit and split
    timings (rotated over >= 4x LLC of K/V), one JSON line per point."""
    import torch
    import paged_kv_decode_cache_amd as pkv
    import workloads

    device = torch.device("cuda:0")
    stream = torch.cuda.current_stream(device)
    points = [("sweep", B, c) for B in workloads.SWEEP_B for c in workloads.SWEEP_CTX]
    points += [("qwen", 8, 0), ("skewed", 256, 0)]
    points += [("long", B, c) for B, c in workloads.LONG_POINTS]
    points += [("extra", B, c) for B, c in workloads.EXTRA_POINTS]
    lines = []
    for kind, B, c in points:
        case = (workloads.sweep_case(B, c) if kind == "sweep" else workloads.qwen_case()
                if kind == "qwen" else workloads.skewed_case() if kind == "skewed"
                else workloads.extra_case(B, c) if kind == "extra"
                else workloads.long_case(B, c))
        kv = case.kv_bytes()
        R = max(2, math.ceil(4 * LLC_BYTES / kv))
        if kv * R > 24e9:
            R = max(1, int(24e9 // kv))
        R = min(R, 64)
        rot = Rotation(case, R, device)
        ctx_sum = int(case.context_lens.astype(np.int64).sum())
        nbytes = alg_bytes(case.B, ctx_sum, case.Hq, case.Hkv, case.D)
        K = int(min(400, max(20, 2e9 / nbytes)))
        out = torch.empty((case.B, case.Hq, case.D), dtype=torch.float16, device=device)

        def time_it(fn):
            return time_graph(capture([lambda r=r: fn(r) for r in range(R)]), R, K)

        us_unsplit = time_it(lambda i: pkv.paged_attention_decode(
            rot.q, rot.k_pool, rot.v_pool, rot.bt[i % R], rot.ctx, case.scale, out=out))

        def append_unsplit(i):
            pkv.kv_cache_append(rot.k_pool, rot.v_pool, rot.k_new, rot.v_new, rot.slots[i % R])
            pkv.paged_attention_decode(rot.q, rot.k_pool, rot.v_pool, rot.bt[i % R], rot.ctx,
                                       case.scale, out=out)
        us_append_unsplit = time_it(append_unsplit)
        best = None
        best_step = None
        for P in (128, 256, 512, 1024, 2048, 4096):
            if P % case.block_size:
                continue
            Pm = case.max_partitions(P)
            ws = pkv.StepWorkspace(case.B, case.Hq, case.Hkv, case.D, Pm, device)
            po = torch.empty_like(ws.partial_out)
            pl = torch.empty_like(ws.partial_lse)

            def split(i):
                pkv.paged_attention_decode_split(rot.q, rot.k_pool, rot.v_pool, rot.bt[i % R],
                                                 rot.ctx, case.scale, P, Pm, po, pl)
                pkv.split_reduce(po, pl, rot.ctx, P, out=out)

            def fused(i):
                pkv.paged_decode_step(rot.q, rot.k_pool, rot.v_pool, rot.bt[i % R], rot.ctx,
                                      case.scale, P, workspace=ws, out=out)
            def three(i, split=split):
                pkv.kv_cache_append(rot.k_pool, rot.v_pool, rot.k_new, rot.v_new, rot.slots[i % R])
                split(i)

            us = time_it(split)
            if best is None or us < best[1]:
                best = (P, us, time_it(three))
            us = time_it(fused)
            if best_step is None or us < best_step[1]:
                best_step = (P, us)
            del po, pl, ws
        line = {"point": case.name, "kind": kind, "B": case.B, "sum_ctx": ctx_sum,
                "alg_bytes": nbytes, "rotation_sets": R,
                "unsplit_us": round(us_unsplit, 3),
                "unsplit_gbs": round(nbytes / us_unsplit / 1e3, 1),
                "split_best_partition": best[0], "split_us": round(best[1], 3),
                "split_gbs": round(nbytes / best[1] / 1e3, 1),
                "append_split_merge_us": round(best[2], 3),
                "append_unsplit_us": round(us_append_unsplit, 3),
                "fused_best_partition": best_step[0], "fused_us": round(best_step[1], 3),
                "fused_gbs": round(nbytes / best_step[1] / 1e3, 1)}
        print(json.dumps(line), flush=True)
        lines.append(line)
        del rot
        torch.cuda.empty_cache()
    with open(args.sweep, "w") as f:
        for ln in lines:
            f.write(json.dumps(ln) + "\n")


GATE_STEPS = 32


def step_mode(max_partitions):
    """The fused step's kernel instantiation as the library picks it by
    partitions per pair: the two-level merge past 32 (MODE 3), the direct
    merge at 4 or fewer (MODE 4), else the merge through LDS (MODE 2)."""
    return 3 if max_partitions > 32 else (4 if max_partitions <= 4 else 2)


def step_waves(D, B, Hkv, Pm):
    """Waves per workgroup of the fused step at the library's default shape:
    8 at head_dim 64 when the grid is at most 256 workgroups and a pair has
    at least 8 partitions, else 4."""
    return 8 if D == 64 and B * Hkv * Pm <= 256 and Pm >= 8 else 4


def gate_expected(D, G, Pm, args, B=32, Hkv=2):
    """Kernel names one fused step and one three-launch step must launch, at
    the library's default shapes (or the explicit ones)."""
    dual = "true" if G <= 8 else "false"
    ns_step = args.subtiles or 1
    ns = args.subtiles or (2 if D == 64 else 1)
    nw, depth = args.waves or 4, args.depth or 2
    nw_step = args.waves or step_waves(D, B, Hkv, Pm)
    return {
        "fused": [f"void pkv::attn_kernel<{D}, {ns_step}, {nw_step}, {depth}, {step_mode(Pm)}, {dual}>"
                  "(pkv::AttnParams)"],
        "three_launch": ["pkv::append_kernel(pkv::AppendParams)",
                         f"void pkv::attn_kernel<{D}, {ns}, {nw}, {depth}, 1, {dual}>"
                         "(pkv::AttnParams)",
                         f"void pkv::split_reduce_kernel<{D}>(pkv::ReduceParams)|"
                         f"void pkv::split_reduce_rows_kernel<{D}>(pkv::ReduceParams)"],
    }


def run_gate_child(args):
    """Under rocprofv3: GATE_STEPS fused steps, then GATE_STEPS three-launch
    steps, eager, rotating over the headline's sets (so the traced durations
    are of cold reads, as in the timed run)."""
    import torch
    import paged_kv_decode_cache_amd as pkv
    import workloads
    device = torch.device("cuda:0")
    B, ctx, P = args.batch, args.ctx, args.partition
    case = (workloads.sweep_case(B, ctx) if B in workloads.SWEEP_B and ctx in workloads.SWEEP_CTX
            else workloads.sweep_case(B, ctx, seed=3999))
    R = args.sets or max(2, math.ceil(4 * LLC_BYTES / case.kv_bytes()))
    rot = Rotation(case, R, device)
    q, kp, vp, cl, kn, vn = rot.q, rot.k_pool, rot.v_pool, rot.ctx, rot.k_new, rot.v_new
    Pm = case.max_partitions(P)
    ws = pkv.StepWorkspace(B, case.Hq, case.Hkv, case.D, Pm, device)
    po = torch.empty_like(ws.partial_out)
    pl = torch.empty_like(ws.partial_lse)
    out = torch.empty((B, case.Hq, case.D), dtype=torch.float16, device=device)
    launch = (dict(waves=args.waves, subtiles=args.subtiles, depth=args.depth)
              if args.waves or args.subtiles or args.depth else None)
    torch.cuda.synchronize()
    for i in range(GATE_STEPS):
        pkv.paged_decode_step(q, kp, vp, rot.bt[i % R], cl, case.scale, P, k_new=kn, v_new=vn,
                              slot_mapping=rot.slots[i % R], workspace=ws, out=out,
                              launch=launch)
    for i in range(GATE_STEPS):
        pkv.kv_cache_append(kp, vp, kn, vn, rot.slots[i % R])
        pkv.paged_attention_decode_split(q, kp, vp, rot.bt[i % R], cl, case.scale, P, Pm, po, pl,
                                         launch=launch)
        pkv.split_reduce(po, pl, cl, P, out=out)
    torch.cuda.synchronize()


def run_kernel_gate(args):
    """Run the gate child under rocprofv3 --kernel-trace --stats (before this
    process touches the GPU) and check the library's kernels by name and
    count: exactly GATE_STEPS launches of the fused kernel, GATE_STEPS of
    each three-launch kernel, and no other kernel of the library."""
    import csv
    import shutil
    import subprocess
    import tempfile
    prof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    if args.no_gate or not os.path.exists(prof):
        return {"status": "skipped", "reason": "--no-gate" if args.no_gate else
                "rocprofv3 not found"}
    base = os.path.join(ROOT, "gpurun_out")
    out_dir = tempfile.mkdtemp(prefix="gate_", dir=base if os.path.isdir(base) else None)
    cmd = [prof, "--kernel-trace", "--stats", "--output-format", "csv", "-d", out_dir, "-o",
           "gate", "--", sys.executable, os.path.abspath(__file__), "--gate-child",
           "--batch", str(args.batch), "--ctx", str(args.ctx), "--partition",
           str(args.partition), "--waves", str(args.waves), "--subtiles", str(args.subtiles),
           "--depth", str(args.depth), "--sets", str(args.sets)]
    env = dict(os.environ, TMPDIR="/tmp")
    try:
        r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True,
                           timeout=240)
        rc = r.returncode
    except subprocess.TimeoutExpired:
        return {"status": "fail", "reason": "rocprofv3 run timed out", "command": " ".join(cmd)}
    stats = os.path.join(out_dir, "gate_kernel_stats.csv")
    # rocprofv3 itself can end with a segmentation fault after the traced
    # program has finished and its results are whole
    if not os.path.exists(stats) or rc not in (0, -11, 139):
        return {"status": "fail", "reason": f"rocprofv3 exit {rc}, stats present: "
                                            f"{os.path.exists(stats)}",
                "stderr_tail": (r.stderr or "")[-400:]}
    observed = {}
    for row in csv.DictReader(open(stats)):
        observed[row["Name"]] = {"calls": int(row["Calls"]),
                                 "average_us": round(float(row["AverageNs"]) / 1e3, 3)}
    import workloads
    case = workloads.sweep_case(args.batch, args.ctx) if (
        args.batch in workloads.SWEEP_B and args.ctx in workloads.SWEEP_CTX) else None
    Hq, Hkv, D = (case.Hq, case.Hkv, case.D) if case else (14, 2, 64)
    Pm = case.max_partitions(args.partition) if case else -(-args.ctx // args.partition)
    want = gate_expected(D, Hq // Hkv, Pm, args, args.batch, Hkv)
    problems = []
    matched = set()
    for path, names in want.items():
        for alts in names:
            hit = [n for n in alts.split("|") if n in observed]
            calls = sum(observed[n]["calls"] for n in hit)
            matched.update(hit)
            if calls != GATE_STEPS:
                problems.append(f"{path}: {alts} launched {calls} times, expected {GATE_STEPS}")
    extra = [n for n in observed if n not in matched and ("pkv::" in n)]
    if extra:
        problems.append(f"unexpected library kernels: {extra}")
    fused_name = want["fused"][0]
    three = [n for alts in want["three_launch"] for n in alts.split("|") if n in observed]
    return {
        "status": "pass" if not problems else "fail",
        "problems": problems,
        "steps": GATE_STEPS,
        "expected_per_step": {"fused": want["fused"], "three_launch": want["three_launch"]},
        "observed": {n: v for n, v in observed.items() if "pkv::" in n},
        "fused_kernel_traced_avg_us": observed.get(fused_name, {}).get("average_us"),
        "three_launch_kernels_traced_sum_us": round(sum(observed[n]["average_us"]
                                                        for n in three), 3),
        "trace": "rocprofv3 --kernel-trace --stats of a child process, eager launches rotating "
                 "over the same sets as the timed run",
    }


def main():
    args = parse()
    if args.gate_child:
        run_gate_child(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the decode path "
                                   "shards with no collective, by sequence or KV head, one process per GPU",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.allocator:
        print(json.dumps(run_allocator(args)), flush=True)
        return
    # the gate runs its child before this process initialises the GPU
    headline = not (args.sweep or args.q8 or args.prefill)
    gate = run_kernel_gate(args) if headline else None
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.sweep:
        run_sweep(args)
        return
    if args.q8:
        print(json.dumps(run_q8(args)), flush=True)
        return
    if args.prefill:
        if args.batch == 32 and args.ctx == 4096 and "--batch" not in sys.argv:
            args.batch = 8
        print(json.dumps(run_prefill(args)), flush=True)
        return
    print(json.dumps(run_headline(args, gate)), flush=True)


if __name__ == "__main__":
    main()
