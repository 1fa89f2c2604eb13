#!/usr/bin/env python3
"""Benchmark of the SDM forward hot path on one MI355X.

One step = the whole hot path over one batch: Phase 1 of every chunk of the workload (sort, scans,
records, tile bounds, A / QK) followed by every DW step of the workload, all enqueued on one stream
with the inputs already in HBM, launched eagerly (--graph: replayed from a HIP graph). Before the W warmup
steps, untimed steps run for about --settle seconds so that the GPU clocks leave idle. `value` is
the step's throughput in Phase-1 K+Q entries per second. Kernel durations for the roofline come
from a second, eager pass of the same steps with HIP events bound to each kernel's own start and
end.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I] [--no-cpu-baseline] [--graph]
                    [--settle S]
    python bench.py --copy-calibration MIB   # a plain device copy, for scaling HBM byte counters

The default workload is the largest one-GPU configuration, the large bank with a ragged tail
(index 4: P=16, T=16384, C=256, W=R=32, S=4194304 per stream, hd=128, bf16 bank); the others are
parity cases that can also be timed with --workload. Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_BYTES = 8.0e12
METRIC = "Phase-1 K+Q entries/sec and DW bank GB/s (fraction of HBM roofline), 1 GPU"
KERNEL_SOURCES = {   # the files each kernel's code comes from (traffic counters are keyed on them)
    "p1_main_kernel": ["phase1.hip", "p1_scan.hpp", "sdm_device.hpp"],
    "p1_pairs_kernel": ["phase1.hip", "p1_scan.hpp", "sdm_device.hpp"],
    "dw_kernel": ["dw.hip", "sdm_device.hpp"],
    "read_gather_kernel": ["read.hip", "sdm_device.hpp"],
    "read_solve_kernel": ["read.hip", "sdm_device.hpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def p1_main_bytes(C, W, R):
    """Algorithmic bytes of the sort/scan kernel per chunk: per K entry id 4 + value 4 read and
    log_k, rex, cpe, k_eff, pos_k, spay_k 4 each + is_last, is_only 1 each + krec 16 written
    (50 B); per Q entry 8 read and log_q, q_w, pos_q, spay_q 4 each + 2 flag bytes (26 B); 4 B of
    gate per token."""
    return C * W * 50 + C * R * 26 + 4 * C


def p1_pairs_bytes(C):
    """The dense [C, C] float32 A and QK written per chunk."""
    return 8 * C * C


def dw_bytes(groups, C, W, hd, bank_es, dv_es):
    """One DW launch (P chunks): base row read + new row written per valid group, each token row
    read once, 16 B of record per K entry. Returns (total, bank part)."""
    bank = 2 * groups * hd * bank_es
    return bank + C * hd * dv_es + 16 * C * W, bank


def read_gather_bytes(P, C, W, R, hd, bank_es):
    """One read-side gather launch: per entry its id and weight (8 B) and its bank row slice; p0 and
    q0 written as float32 rows per token."""
    return P * C * (W + R) * (hd * bank_es + 8) + 2 * P * C * hd * 4


def read_solve_bytes(P, C, hd):
    """One substitution launch: the A and QK triangles (dense float32), v, p0 and q0 read, dv, pred
    and read written (float32 rows), beta."""
    return 2 * P * C * C * 4 + 6 * P * C * hd * 4 + P * C * 4


def source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_delta_memory_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload_name, kernel):
    """HBM bytes per launch of `kernel` from profiles/traffic_<workload>.txt (rocprofv3 FETCH_SIZE and
    WRITE_SIZE, each scaled by what the counter reads for a plain copy of known size), or None when
    missing or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload_name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("src_sha." + kernel) != source_digest(kernel):
        return None
    key = "bytes_per_launch." + kernel
    return float(vals[key]) if key in vals else None


def host_threads():
    """Threads for the oracle: OMP_NUM_THREADS when set (the host's share of cores), else the CPUs
    this process may run on, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(wl, bank0, target_s=12.0, target_1core_s=5.0):
    """The oracle, as it stands, on a bounded sample of the same workload: Phase 1 of a sample of
    chunks plus the DW of the same chunks from the initial bank, on `host_threads()` threads
    (chunks spread over them), and a smaller sample on one thread."""
    import torch

    import oracle

    sh = wl.shape
    threads = host_threads()
    n = sh.C * (sh.W + sh.R)
    dv = wl.dv.reshape(-1, sh.hd)
    okw = dict(P=wl.P, stream_offset=sh.S, first_partial=wl.first_partial, valid_last=wl.valid_last)

    def jobs_for(chunks):   # DW inputs gathered outside the timed region
        jobs = []
        for c in chunks:
            slots = oracle.dw_slots(wl.k_idx, wl.q_idx, wl.k_val, wl.q_val, wl.g, c, **okw)
            base = bank0.index_select(0, torch.as_tensor(slots, device=bank0.device)).float().cpu().numpy()
            jobs.append((c, base.astype(np.float64), dv[c * sh.C:(c + 1) * sh.C].astype(np.float64)))
        return jobs

    def run_dw(job):
        c, base, rows = job
        oracle.dw_apply(wl.k_idx, wl.q_idx, wl.k_val, wl.q_val, wl.g, c, rows, base, **okw)

    def timed(chunks, jobs, nthreads):
        from concurrent.futures import ThreadPoolExecutor

        t0 = time.perf_counter()
        oracle.phase1(wl.k_idx, wl.q_idx, wl.k_val, wl.q_val, wl.g, chunks=chunks, threads=nthreads, **okw)
        t_p1 = time.perf_counter() - t0
        t0 = time.perf_counter()
        if nthreads == 1:
            for j in jobs:
                run_dw(j)
        else:
            with ThreadPoolExecutor(max_workers=nthreads) as ex:
                list(ex.map(run_dw, jobs))
        return t_p1, time.perf_counter() - t0

    # Calibrate on one chunk, then size each sample for its target time.
    one_p1, one_dw = timed([0], jobs_for([0]), 1)
    one = max(one_p1 + one_dw, 1e-4)
    m1 = int(min(wl.N, max(1, target_1core_s / one)))
    t1_p1, t1_dw = timed(list(range(m1)), jobs_for(range(m1)), 1)
    m = int(min(wl.N, max(threads, target_s * threads / one)))
    chunks = list(range(m))
    jobs = jobs_for(chunks)
    t_p1, t_dw = timed(chunks, jobs, threads)
    # A short sample (a small workload can finish in well under a second) is repeated, whole
    # passes only, until about 10 s of oracle work have been timed (at most 30 s).
    passes = 1
    once = t_p1 + t_dw
    while t_p1 + t_dw < 10.0 and t_p1 + t_dw + once <= 30.0:
        a, b = timed(chunks, jobs, threads)
        t_p1 += a
        t_dw += b
        passes += 1
    return {
        "value": passes * m * n / (t_p1 + t_dw), "unit": "entries/s", "cores": threads, "kind": "oracle",
        "sample": "%d of %d chunks (Phase 1 + the DW of the same chunks from the initial bank), %d passes on %d "
                  "threads: phase1 %.2f s, dw %.2f s" % (m, wl.N, passes, threads, t_p1, t_dw),
        "value_1core": m1 * n / (t1_p1 + t1_dw),
        "sample_1core": "%d chunks on 1 thread: phase1 %.2f s, dw %.2f s" % (m1, t1_p1, t1_dw),
        "cpu_model": cpu_model(),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the step from a HIP graph in the timed region")
    ap.add_argument("--pair-stream", action="store_true",
                    help="the pair sums on a second stream beside the DW launches (default: one stream)")
    ap.add_argument("--settle", type=float, default=0.25, metavar="S",
                    help="untimed steps for about S seconds before the warmup steps (clocks settle)")
    ap.add_argument("--no-gds", action="store_true", help="skip the GDS (backward of the read gather) measurement")
    ap.add_argument("--no-read-side", action="store_true",
                    help="skip the separate measurement of the read side (gather + substitution) and the forward loop")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 3 times (a known-traffic kernel for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the hot path has no multi-GPU part); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_delta_memory_amd as sdm
    from sparse_delta_memory_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d MiB 3 times" % args.copy_calibration)
        return
    wl = W.make(args.workload)
    sh = wl.shape
    log("workload %d %s: N=%d chunks, n=%d entries/chunk" % (args.workload, sh.name, wl.N, sh.C * (sh.W + sh.R)))
    shape = sdm.make_shape(wl.N, sh.C, sh.W, sh.R, P=sh.P, key_bits=sh.key_bits, stream_offset=sh.S,
                           first_partial=wl.first_partial, valid_last=wl.valid_last, tile_len=128)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    ins = dict(k_idx=t(wl.k_idx), q_idx=t(wl.q_idx), k_val=t(wl.k_val), q_val=t(wl.q_val), g=t(wl.g))
    dv = t(wl.dv.reshape(-1, sh.hd))
    if sh.dv_dtype == "bf16":
        dv = dv.to(torch.bfloat16)
    out = sdm.alloc_phase1_outputs(shape, device=dev)
    ws = torch.empty(sdm.phase1_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    dw_ws = sdm.alloc_dw_workspace(shape, sh.hd, device=dev)
    bank = W.make_bank(wl, dev)
    bank0 = bank.clone() if not args.no_cpu_baseline else None
    stream = torch.cuda.current_stream(dev)
    P, C = sh.P, sh.C
    plan = sdm.DwPlan(bank, dv, out["krec"], shape, dv_step_rows=P * C, workspace=dw_ws)
    n_ev = 4 + 2 * wl.steps   # start / end of the sort-scan kernel, the pair kernel, every DW launch

    # --pair-stream: the pair sums (A, QK) feed nothing in the step and DW needs only the sort/scan
    # kernel's records, so the pair kernel may run on a second stream (default priority, like every
    # stream here) beside the DW launches; the launch stream waits for it at the end of the step.
    # Measured: Zipf 0.81 -> 0.77 ms per step, but uniform 0.186 -> 0.217, wide rows 0.408 -> 0.424
    # and large_ragged 2.004 -> 2.006 (the pair kernel then competes with DW for the compute units),
    # so one stream stays the default.
    side = torch.cuda.Stream(device=dev)
    p1_done = torch.cuda.Event()
    pairs_done = torch.cuda.Event()

    def step(ev=None):
        evp = None if ev is None else ev[0:4]
        if not args.pair_stream:
            sdm.phase1(shape, out=out, workspace=ws, events=evp, **ins)
        else:
            sdm.phase1(shape, out=out, workspace=ws, events=evp, defer_pairs=True, **ins)
            p1_done.record(stream)
            side.wait_event(p1_done)
            sdm.phase1_pairs(shape, out, ws, stream=side, events=evp)
            pairs_done.record(side)
        for ti in range(wl.steps):
            plan.step(ti, events=None if ev is None else ev[4 + 2 * ti:6 + 2 * ti])
        if args.pair_stream:
            stream.wait_event(pairs_done)

    # Untimed settling: steps for about --settle seconds (the GPU leaves its idle clocks; a cold
    # first timed region measured up to 20 % slow), then the W warmup steps proper.
    t_settle = time.perf_counter()
    for _ in range(100000):
        step()
        torch.cuda.synchronize()
        if time.perf_counter() - t_settle >= args.settle:
            break
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        # The whole step (2 Phase-1 kernels and every DW launch) captured once and replayed: the
        # launches then cost no host time. Captured launches take no timing events.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    # Timed region: exactly `steps` steps.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Kernel durations: the same steps again, launched eagerly with events bound to each kernel's
    # own start and end (binding them costs host time per launch, so they stay out of the timed
    # region above).
    evs = [sdm.timing_events(n_ev, stream) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    ms_main = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_pairs = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    ms_dw = float(np.mean([e[4 + 2 * ti].elapsed_time(e[5 + 2 * ti]) for e in evs for ti in range(wl.steps)]))

    # Valid groups per step (for the DW's algorithmic bytes), from the records' FIRST flags.
    first = (out["krec"][..., 0] & (W_FIRST | W_INVALID)) == W_FIRST
    groups_per_chunk = first.sum(dim=1).cpu().numpy().astype(np.int64)
    groups_per_step = groups_per_chunk.reshape(wl.steps, P).sum(axis=1)
    bank_es = 2 if sh.bank_dtype == "bf16" else 4
    dv_es = 2 if sh.dv_dtype == "bf16" else 4
    dw_tot = [dw_bytes(int(gs), C * P, sh.W, sh.hd, bank_es, dv_es) for gs in groups_per_step]
    dw_launch_bytes = float(np.mean([d[0] for d in dw_tot]))
    dw_bank_bytes = float(np.mean([d[1] for d in dw_tot]))
    main_bytes = wl.N * p1_main_bytes(sh.C, sh.W, sh.R)
    pairs_bytes = wl.N * p1_pairs_bytes(sh.C)
    kernels = {
        "p1_main_kernel": (main_bytes, ms_main),
        "p1_pairs_kernel": (pairs_bytes, ms_pairs),
        "dw_kernel": (dw_launch_bytes, ms_dw),
    }
    per = {}
    for name, (b, ms) in kernels.items():
        ach = b / (ms * 1e-3)
        per[name] = {"bytes_per_launch": b, "ms_per_launch": ms, "GBps": ach / 1e9, "frac": ach / HBM_PEAK_BYTES,
                     "launches_per_step": wl.steps if name == "dw_kernel" else 1}
    dom = max(per, key=lambda k: per[k]["ms_per_launch"] * per[k]["launches_per_step"])
    traffic = read_traffic(sh.name, dom)
    entries = wl.N * sh.C * (sh.W + sh.R)
    ms_step = wall / args.steps * 1e3
    res = {
        "metric": METRIC,
        "value": entries / (ms_step * 1e-3),
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generators; no dataset)",
        "config": {
            "workload": "%s: P=%d T=%d C=%d W=%d R=%d S=%d hd=%d bank %s dv %s slots %s" % (
                sh.name, sh.P, sh.T, sh.C, sh.W, sh.R, sh.S, sh.hd, sh.bank_dtype, sh.dv_dtype, sh.slots),
            "chunks": wl.N, "dw_steps": wl.steps, "global_batch": wl.N * sh.C, "seq_len": sh.T,
            "parallelism": "single GPU", "launch": ("hipGraph replay" if args.graph else "eager") +
            (", pair sums on a second stream" if args.pair_stream else ""),
        },
        "phase1_entries_per_s": entries / ((ms_main + ms_pairs) * 1e-3),
        "phase1_hbm_frac": (main_bytes + pairs_bytes) / ((ms_main + ms_pairs) * 1e-3) / HBM_PEAK_BYTES,
        "dw_bank_GBps": dw_bank_bytes / (ms_dw * 1e-3) / 1e9,
        "dw_hbm_frac": dw_launch_bytes / (ms_dw * 1e-3) / HBM_PEAK_BYTES,
        "kernels": per,
        "roofline": {
            "kernel": dom, "bound": "hbm", "achieved": per[dom]["GBps"], "peak": HBM_PEAK_BYTES / 1e9, "unit": "GB/s",
            "frac": per[dom]["frac"], "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if not args.no_read_side:
        res["read_side"] = measure_read_side(args, wl, shape, out, ins, bank, plan, stream, W, sdm, torch)
    if not args.no_gds:
        res["gds"] = measure_gds(wl, shape, out, ins, bank, stream, sdm, torch)
        res["gwr_pa"] = measure_gwr_pa(wl, shape, out, ins, bank, stream, sdm, torch, W)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores)...")
        res["cpu_baseline"] = cpu_baseline(wl, bank0)
    print(json.dumps(res), flush=True)


def measure_read_side(args, wl, shape, out, ins, bank, dw_plan, stream, W, sdm, torch):
    """The read side of every step (gather + substitution kernels) timed by events bound to each
    kernel, and the wall time of a forward loop: for each step the read side, then its DW step (the
    DW then consumes the read side's token rows). Not part of the headline step."""
    sh = wl.shape
    P, C, hd = sh.P, sh.C, sh.hd
    dev = bank.device
    v_host, beta_host = W.make_read_inputs(wl)
    v = torch.from_numpy(v_host).to(dev)
    beta = torch.from_numpy(beta_host).to(dev)
    dv = torch.zeros((v.shape[0], hd), dtype=torch.float32, device=dev)
    pred, read = torch.zeros_like(dv), torch.zeros_like(dv)
    rplan = sdm.ReadPlan(bank, out, ins["k_idx"], ins["q_idx"], v, beta, dv, pred, read, shape, step_rows=P * C)
    fplan = sdm.DwPlan(bank, dv, out["krec"], shape, dv_step_rows=P * C)

    def forward():
        for ti in range(wl.steps):
            rplan.step(ti)
            fplan.step(ti)

    for _ in range(2):
        forward()
    torch.cuda.synchronize()
    reps = max(1, min(args.steps, 5))
    t0 = time.perf_counter()
    for _ in range(reps):
        forward()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    evs = [sdm.timing_events(4, stream) for _ in range(wl.steps)]
    torch.cuda.synchronize()
    for ti in range(wl.steps):
        rplan.step(ti, events=evs[ti])
    torch.cuda.synchronize()
    ms_g = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_s = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    bank_es = 2 if sh.bank_dtype == "bf16" else 4
    gb = read_gather_bytes(P, C, sh.W, sh.R, hd, bank_es)
    sb = read_solve_bytes(P, C, hd)
    return {
        "gather_kernel": {"bytes_per_launch": gb, "ms_per_launch": ms_g, "GBps": gb / (ms_g * 1e-3) / 1e9,
                          "frac": gb / (ms_g * 1e-3) / HBM_PEAK_BYTES},
        "solve_kernel": {"bytes_per_launch": sb, "ms_per_launch": ms_s, "GBps": sb / (ms_s * 1e-3) / 1e9,
                         "frac": sb / (ms_s * 1e-3) / HBM_PEAK_BYTES},
        "forward_loop_ms": wall * 1e3,
        "forward_loop": "every step: read side (2 kernels) then DW; %d steps, eager" % wl.steps,
    }


def gds_bytes(P, C, R, hd, bank_es, groups_q, grad_es):
    """Algorithmic bytes of one GDS step: the dots read per read its id (8 with the q_w/element
    words counted in the scatter), its bank row, and write its dot; the scatter reads per Q-row
    position its element, id and q_w, and reads and writes each group's grad row once; each token's
    gradient row is read once for the step."""
    dots = P * C * R * (hd * bank_es + 8 + 4)
    scatter = P * C * R * (4 + 8) + 2 * groups_q * hd * grad_es
    return dots + scatter + P * C * hd * 4


def gwr_bytes(P, C, W, hd, grad_es):
    """One GWR step: per write its id and weight (8 B), its gradient row and its dot (4 B); each
    token row read and its d_dv row written once (float32)."""
    return P * C * W * (hd * grad_es + 12) + 2 * P * C * hd * 4


def pa_bytes(P, C, W, hd, groups, grad_es, bank_es):
    """One PA step: per K-row position its record (16 B), k_eff and beta (8 B) and its two
    gradient outputs (4 B + 8 B of element bookkeeping); per write group its grad row read and
    written, its snapshot row read and its bank row restored; each token's d_dva row read once."""
    return P * C * W * 36 + groups * hd * (2 * grad_es + 2 * bank_es) + P * C * hd * 4


def measure_gds(wl, shape, out, ins, bank, stream, sdm, torch):
    """GDS of every step (dots + scatter kernels), timed by events on the launch stream around each
    call; gradient rows seeded. Not part of the headline step."""
    sh = wl.shape
    P, C, R, hd = sh.P, sh.C, sh.R, sh.hd
    dev = bank.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.bank_seed + 23)
    gr = torch.randn((wl.steps * P * C, hd), generator=gen, device=dev)
    d = torch.zeros((wl.N, C, R), device=dev)
    grad = torch.zeros_like(bank)
    sp = out["spay_q"]
    heads = ((sp & W_FIRST) != 0) & ((sp & W_INVALID) == 0)
    groups_q = float(heads.view(wl.steps, P * C * R).sum(dim=1).float().mean())
    ws = sdm.alloc_gds_workspace(shape, hd, device=dev)   # long read groups split across waves
    for ti in range(min(2, wl.steps)):
        sdm.gds_step(bank, out, ins["q_idx"], gr, shape, ti, step_rows=P * C, d_q_w=d, grad=grad, stream=stream,
                     workspace=ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(wl.steps)]
    for ti in range(wl.steps):
        ev[ti][0].record(stream)
        sdm.gds_step(bank, out, ins["q_idx"], gr, shape, ti, step_rows=P * C, d_q_w=d, grad=grad, stream=stream,
                     workspace=ws)
        ev[ti][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    b = gds_bytes(P, C, R, hd, 2 if sh.bank_dtype == "bf16" else 4, groups_q, 2 if sh.bank_dtype == "bf16" else 4)
    return {"bytes_per_step": b, "ms_per_step": ms, "GBps": b / (ms * 1e-3) / 1e9, "frac": b / (ms * 1e-3) / HBM_PEAK_BYTES,
            "note": "dots + scatter kernels per step, events around the call; grad in the bank dtype"}


def measure_gwr_pa(wl, shape, out, ins, bank, stream, sdm, torch, W):
    """GWR and PA of every step, each timed by events on the launch stream around its call (PA after
    the step's DW has written its snapshot); seeded gradient inputs. Not part of the headline step.
    Algorithmic bytes: gwr_bytes and pa_bytes (each token row counted once)."""
    sh = wl.shape
    P, C, Wn, hd = sh.P, sh.C, sh.W, sh.hd
    dev = bank.device
    es = 2 if sh.bank_dtype == "bf16" else 4
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.bank_seed + 43)
    rows = wl.steps * P * C
    dv = torch.randn((rows, hd), generator=gen, device=dev)
    d_dva = torch.randn((rows, hd), generator=gen, device=dev)
    w = torch.randn((wl.N, C, Wn), generator=gen, device=dev)
    beta = torch.rand((wl.N, C), generator=gen, device=dev)
    grad = (torch.randn(bank.shape, generator=gen, device=dev) * 0.01).to(bank.dtype)
    d_dv = torch.zeros_like(dv)
    d_k_pd = torch.zeros((wl.N, C, Wn), device=dev)
    g_decay = torch.zeros((wl.N, C, Wn), device=dev)
    d_k_eff = torch.zeros((wl.N, C, Wn), device=dev)
    snap = torch.zeros((P * C * Wn, hd), dtype=bank.dtype, device=dev)
    work = bank.clone()
    plan = sdm.DwPlan(work, dv, out["krec"], shape, dv_step_rows=P * C, snapshot=snap, snap_step_rows=0)
    pa_ws = sdm.alloc_pa_workspace(shape, hd, device=dev)   # long write groups split across waves
    kr = out["krec"][..., 0]
    groups = float((((kr & W_FIRST) != 0) & ((kr & W_INVALID) == 0)).view(wl.steps, -1).sum(dim=1).float().mean())
    ev_g, ev_p = [], []
    for ti in range(wl.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sdm.gwr_step(grad, ins["k_idx"], w, dv, shape, ti, step_rows=P * C, d_dv=d_dv, d_k_pd=d_k_pd, stream=stream)
        b.record(stream)
        ev_g.append((a, b))
        plan.step(ti, stream=stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sdm.pa_step(grad, snap, out, beta, d_dva, shape, ti, step_rows=P * C, snap_step_rows=0, bank=work,
                    g_decay=g_decay, d_k_eff=d_k_eff, stream=stream, workspace=pa_ws)
        b.record(stream)
        ev_p.append((a, b))
    torch.cuda.synchronize()
    skip = 1 if wl.steps > 1 else 0   # the first calls include their one-time costs
    ms_g = float(np.mean([a.elapsed_time(b) for a, b in ev_g[skip:]]))
    ms_p = float(np.mean([a.elapsed_time(b) for a, b in ev_p[skip:]]))
    bg = gwr_bytes(P, C, Wn, hd, es)
    bp = pa_bytes(P, C, Wn, hd, groups, es, es)
    return {"gwr": {"bytes_per_step": bg, "ms_per_step": ms_g, "frac": bg / (ms_g * 1e-3) / HBM_PEAK_BYTES},
            "pa": {"bytes_per_step": bp, "ms_per_step": ms_p, "frac": bp / (ms_p * 1e-3) / HBM_PEAK_BYTES},
            "note": "events around each call on the launch stream; grad and bank in the bank dtype"}


W_FIRST = -(1 << 31)      # bit 31 of the int32 record element
W_INVALID = 1 << 17

if __name__ == "__main__":
    main()
