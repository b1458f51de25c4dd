#!/usr/bin/env python3
"""Throughput of the chunked SSD scan forward on one MI355X.

Workload: the Mamba-2 2.7B layer shape, b=8, T=8192, H=80, P=64, N=128, G=1,
chunk_len=256, x/B/C in bf16, da/D fp32, y and final_state fp32, seeded
synthetic inputs (ssd_inputs.CONFIGS[2]) resident in HBM before timing.
A step is one full forward scan (every stage) over the batch.

Prints one JSON line with tokens/s, the HBM roofline of the dominant kernel
(algorithmic bytes / kernel time measured with HIP events on the launch
stream) and the float64 CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3
# VALU issue of unpacked fp32: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane
# slots per second; a full-rate op takes one slot per lane, exp2 two (half rate)
VALU_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9
SEL_SLOTS_PER_UPDATE = 6       # dl*A, exp2 (2 slots), (dl*u)*B, state fma, C.h fma


def algorithmic_bytes(s) -> int:
    """Compulsory I/O: every input read once at its dtype, outputs written once."""
    esz = 2 if s.dtype == "bf16" else 4
    b, T, H, P, N, G, R = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.mimo_rank
    n = b * T * R * H * P * esz            # x
    n += b * T * H * 4                      # da
    n += 2 * b * T * R * G * N * esz        # B, C
    n += H * 4 if s.skip != "none" else 0   # D
    n += b * H * P * N * 4 if s.init_state else 0
    n += b * T * H * (N // 2) * 4 if s.rotation else 0
    n += b * T * R * H * P * 4              # y
    n += b * H * P * N * 4                  # final_state
    return n


KERNEL_TILE_ROWS = 32            # fused rows (t, r) per tile the walks run, for any chunk_len


def algorithmic_flops(s, tile_rows: int = KERNEL_TILE_ROWS) -> int:
    """Causal (block-)lower-triangular K2 + K3 + K5 flops at the tile the kernels walk.

    The walks run 32-row tiles of fused (step, rank) rows whatever chunk_len is
    (the chunked form is exact for any chunk length), so the intra-tile terms,
    K2 and the K5 diagonal block, are counted at that tile: per tile the
    (row, column) pairs with step(row) >= step(column).
    """
    b, T, H, P, N, G, R = (s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups,
                           s.mimo_rank)
    ntiles = -(-(T * R) // tile_rows)
    q = tile_rows // R                       # steps per tile
    pairs = R * R * q * (q + 1) // 2         # causal (row, column) pairs per tile
    k3 = 2 * b * H * T * R * P * N
    k5_off = 2 * b * H * T * R * P * N
    k5_diag = 2 * b * H * ntiles * pairs * P
    k2 = 2 * b * ntiles * pairs * N * (H if s.rotation else G)
    return k3 + k5_off + k5_diag + k2


# kernel sources behind each workload's counter summary
SSD_SOURCES = ("ssd_scan.hip", "ssd_kernels.h", "ssd_select.h", "ssd_common.h",
               "ssd_cols_bf16.hip", "ssd_cols_f32.hip", "ssd_walk_bf16.hip", "ssd_walk_f32.hip")
KERNEL_SOURCES = {
    "ssd": SSD_SOURCES,
    "selective_scan": ("sel_scan.hip", "ssd_common.h"),
    "trapezoid": SSD_SOURCES + ("trap_scan.hip",),
    "backward": SSD_SOURCES + ("ssd_backward.hip", "ssd_step.h"),
}


def source_digest(workload: str = "ssd") -> str:
    """First 16 hex digits of the SHA-256 over the workload's kernel sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[workload]:
        h.update(open(os.path.join(ROOT, "chunked_ssd_scan_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def profiled_traffic(workload_tag: str, workload: str = "ssd"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None.

    The summary carries a fenced json block with the calibrated bytes and the
    digest of the kernel sources it was measured on; a stale digest gives None.
    """
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_tag}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\s*(\{.*?\})\s*```", open(path).read(), flags=re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_sha256_16") != source_digest(workload):
        return None
    return int(d["hbm_bytes_per_launch"])


def _hip():
    import ctypes
    return ctypes.CDLL("libamdhip64.so")


def _timing_event(hip):
    """A HIP event created without the system-scope fence (timing only: no
    cache writeback between the kernels of a call)."""
    import ctypes
    e = ctypes.c_void_p()
    if hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(0x20000000)) != 0:
        raise RuntimeError("hipEventCreateWithFlags failed")
    return e.value


def _elapsed_ms(hip, a, b) -> float:
    import ctypes
    ms = ctypes.c_float()
    if hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return float(ms.value)


def prewarm(step, seconds: float) -> int:
    """Run whole calls back to back for at least ``seconds`` of wall time, so
    that the shader clock has left its idle state before anything is timed.
    Returns the number of calls."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def time_calls(step, calls: int, flush_bytes: int) -> dict:
    """Per-call HIP event timing of the whole call and of its output walk.

    Before each call a plain fill overwrites ``flush_bytes`` of device memory
    (outside both event pairs), so that no call finds its inputs in the L2 or
    the MALL left there by the previous one. The call is bracketed by one pair
    of events on the launch stream, and the library records a second pair just
    before and after the output walk. Returns the median and min of each.
    """
    import torch
    hip = _hip()
    flush = torch.empty(max(flush_bytes // 4, 1), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    ev = [(_timing_event(hip), _timing_event(hip), _timing_event(hip), _timing_event(hip))
          for _ in range(calls)]
    vp = __import__("ctypes").c_void_p
    for i, (c0, c1, w0, w1) in enumerate(ev):
        flush.fill_(float(i))
        if hip.hipEventRecord(vp(c0), vp(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")
        step(walk_events=(w0, w1))
        if hip.hipEventRecord(vp(c1), vp(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")
    if hip.hipDeviceSynchronize() != 0:
        raise RuntimeError("hipDeviceSynchronize failed")
    call = [_elapsed_ms(hip, c0, c1) for c0, c1, _, _ in ev]
    walk = [_elapsed_ms(hip, w0, w1) for _, _, w0, w1 in ev]
    for e in ev:
        for h in e:
            hip.hipEventDestroy(vp(h))
    del flush
    return {"call_ms_median": statistics.median(call), "call_ms_min": min(call),
            "walk_ms_median": statistics.median(walk), "walk_ms_min": min(walk),
            "calls": calls, "flush_bytes": flush_bytes}


def flushed_block(tc: dict, walk_bytes: int, call_bytes: int) -> dict:
    """The flushed per-call timings of a workload and their HBM fractions."""
    frac = lambda nb, ms: nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    return {"kernel_ms_median": tc["walk_ms_median"], "kernel_ms_min": tc["walk_ms_min"],
            "forward_ms_median": tc["call_ms_median"], "forward_ms_min": tc["call_ms_min"],
            "frac_median": frac(walk_bytes, tc["walk_ms_median"]),
            "forward_frac_median": frac(call_bytes, tc["call_ms_median"])}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, shape, nslices: int):
    import oracle
    nbh = shape.batch * shape.nheads
    nslices = max(1, min(nslices, nbh))
    step = nbh / nslices
    sel = [int(i * step) for i in range(nslices)]
    threads = len(os.sched_getaffinity(0))
    secs = oracle.time_oracle(inp, sel, nthreads=threads)
    tokens = shape.batch * shape.seqlen * (nslices / nbh)
    return {
        "value": tokens / secs,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{nslices} of the {nbh} (batch, head) slices over the full T={shape.seqlen}; "
                   f"{secs:.2f} s wall; tokens/s scaled by the slice fraction"),
    }


def selective_bench(args) -> dict:
    """The diagonal selective scan (b4 T4096 D512 N16, fp32) as its own line."""
    import torch
    import chunked_ssd_scan_amd as ssd
    import ssd_inputs as si

    shape = si.SCAN_CONFIGS[1]
    dev = torch.device("cuda:0")
    inp = si.make_scan_inputs(shape, seed=0)
    g = inp.to(dev)
    y = torch.empty_like(g.u)
    stream = torch.cuda.current_stream(dev)

    def step(walk_events=None):
        ssd.selective_scan(g.u, g.delta, g.A, g.B, g.C, g.skip, y=y, stream=stream.cuda_stream,
                           chunks=args.segments, walk_events=walk_events)

    nwarm = prewarm(step, args.prewarm)
    wall, walks = timed_region_walks(step, args)
    tc = time_calls(step, args.calls, FLUSH_BYTES)
    # the timed region's averages (the output pass, the whole call); the
    # flushed per-call medians and minima beside them
    call_ms, out_ms = wall * 1e3 / args.steps, statistics.fmean(walks)
    if not torch.isfinite(y).all():
        raise RuntimeError("non-finite output")
    b, T, D, N = shape.batch, shape.seqlen, shape.d_model, shape.d_state
    updates = b * T * D * N
    slots = updates * SEL_SLOTS_PER_UPDATE
    achieved = slots / (out_ms * 1e-3) / 1e12
    peak = VALU_SLOTS_PER_S / 1e12
    nbytes = (3 * b * T * D + 2 * b * T * N + D * N + D) * 4
    out = {
        "metric": "selective scan fwd tokens/s + % of VALU issue (b4,T4096,D512,N16)",
        "value": b * T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; see ssd_inputs.make_scan_inputs)",
        "config": {"workload": shape.name, "batch": b, "seqlen": T, "d_model": D, "d_state": N,
                   "chunks": args.segments or "auto"},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TOP/s",
                     "frac": achieved / peak,
                     "traffic": profiled_traffic("selective_scan", "selective_scan"),
                     "algorithmic_slots": slots, "kernel_ms": out_ms, "forward_ms": call_ms,
                     "forward_frac": slots / (call_ms * 1e-3) / 1e12 / peak,
                     "hbm_frac_forward": nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "flushed": {"kernel_ms_median": tc["walk_ms_median"], "kernel_ms_min": tc["walk_ms_min"],
                                 "forward_ms_median": tc["call_ms_median"],
                                 "forward_ms_min": tc["call_ms_min"]}},
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        reps = 3
        t1 = time.perf_counter()
        for _ in range(reps):
            oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.skip, nthreads=threads)
        secs = (time.perf_counter() - t1) / reps
        out["cpu_baseline"] = {"value": b * T / secs, "unit": "tokens/s", "cores": threads,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"the whole workload, {reps} runs, {secs:.3f} s each"}
    return out


def trapezoid_bench(args) -> dict:
    """The Mamba-3 trapezoid forward on the Mamba-3 MIMO layer shape as its own line."""
    import dataclasses
    import torch
    import chunked_ssd_scan_amd as ssd
    import ssd_inputs as si

    shape = si.CONFIGS[3]
    dev = torch.device("cuda:0")
    ti = si.make_trapezoid_inputs(shape, seed=0)
    g = ti.to(dev)
    bi = g.base
    b, T, R, H, P = bi.x.shape
    N = shape.dstate
    y = torch.empty((b, T, R, H, P), device=dev, dtype=torch.float32)
    fin = torch.empty((b, H, P, N), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)

    def step(walk_events=None):
        ssd.trapezoid(bi.x, bi.da, bi.B, bi.C, g.beta, g.gamma, g.prev_x, g.prev_B, bi.init_state,
                      shape.chunk_len, bi.theta, y=y, final_state=fin, segments=args.segments,
                      stream=stream.cuda_stream, walk_events=walk_events)

    nwarm = prewarm(step, args.prewarm)
    wall, walks = timed_region_walks(step, args)
    tc = time_calls(step, args.calls, FLUSH_BYTES)
    # the timed region's averages (the roofline figure); the flushed per-call
    # medians and minima beside them
    walk_ms, call_ms = statistics.fmean(walks), wall * 1e3 / args.steps
    if not (torch.isfinite(y).all() and torch.isfinite(fin).all()):
        raise RuntimeError("non-finite output")
    # the dominant kernel is the rotating walk over 2T sub-steps, which on this
    # shape stages its sub-steps from the original arrays: its compulsory bytes
    # are x, B, C and theta read once, the sub-steps' decay and scale (2T per
    # head, written by a small kernel before it) instead of da, the previous
    # token's x and B, init, and the odd sub-steps' y and the final state
    esz = 2 if shape.dtype == "bf16" else 4
    one = algorithmic_bytes(dataclasses.replace(shape, skip="none"))
    prev = b * R * (H * P + shape.ngroups * N) * esz
    walk_bytes = one - b * T * H * 4 + 2 * b * 2 * T * H * 4 + prev
    trap_bytes = one + 2 * b * T * H * 4 + prev
    achieved = walk_bytes / (walk_ms * 1e-3) / 1e9
    out = {
        "metric": "trapezoid fwd tokens/s + % of HBM roofline (b4,T4096,H32,P64,N128,R4)",
        "value": b * T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded; see ssd_inputs.make_trapezoid_inputs)",
        "config": {"workload": "mamba3 MIMO layer, trapezoid " + shape.name, "batch": b,
                   "seqlen": T, "nheads": H, "headdim": P, "dstate": N, "mimo_rank": R,
                   "rotation": True, "init_state": True, "prev_token": True,
                   "segments": args.segments or "auto"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": profiled_traffic("trapezoid", "trapezoid"),
                     "algorithmic_bytes": walk_bytes, "kernel_ms": walk_ms, "forward_ms": call_ms,
                     "forward_bytes": trap_bytes,
                     "forward_frac": trap_bytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "flushed": flushed_block(tc, walk_bytes, trap_bytes)},
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        nbh = b * H
        nsl = max(1, min(args.cpu_slices // 8, nbh))
        sel = [int(i * nbh / nsl) for i in range(nsl)]
        t1 = time.perf_counter()
        oracle.trapezoid(ti.base.x, ti.base.da, ti.base.B, ti.base.C, ti.beta, ti.gamma, ti.prev_x,
                         ti.prev_B, ti.base.init_state, ti.base.theta, bh=sel, nthreads=threads)
        secs = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": b * T * (nsl / nbh) / secs, "unit": "tokens/s",
                               "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": (f"{nsl} of the {nbh} (batch, head) slices over the full "
                                          f"T={T}; {secs:.2f} s wall; tokens/s scaled by the "
                                          f"slice fraction")}
    return out


FLUSH_BYTES = 1 << 30           # overwritten before each per-call timing: beyond L2 and MALL


def timed_region(step, args) -> float:
    """The contract's timed loop: W warm-up steps, then exactly K steps
    bracketed by device synchronisation. Returns the wall time of the K steps."""
    return timed_region_walks(step, args, False)[0]


def timed_region_walks(step, args, walks: bool = True):
    """The contract's timed loop, with the output walk of every timed step
    bracketed by a pair of HIP events that the library records on the launch
    stream (created beforehand, without the system-scope fence). Returns the
    wall time of the K steps and the K walk durations in ms (None without)."""
    import torch
    hip = _hip() if walks else None
    ev = [(_timing_event(hip), _timing_event(hip)) for _ in range(args.steps)] if walks else None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if ev:
            step(walk_events=ev[i])
        else:
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not ev:
        return wall, None
    vp = __import__("ctypes").c_void_p
    ms = [_elapsed_ms(hip, w0, w1) for w0, w1 in ev]
    for pair in ev:
        for h in pair:
            hip.hipEventDestroy(vp(h))
    return wall, ms


def ssd_step_fn(ssd, g, shape, y, fin, stream, segments=0, block_slices=0):
    def step(walk_events=None):
        ssd.forward(g.x, g.da, g.B, g.C, g.D, g.init_state, shape.chunk_len, g.theta,
                    y=y, final_state=fin, segments=segments, block_slices=block_slices,
                    stream=stream, walk_events=walk_events)
    return step


def ssd_workload(cfg: int, args, with_timed_region: bool):
    """Inputs of workload ``cfg`` resident in HBM, pre-warm, then the flushed
    per-call timing (and the contract's timed loop when asked)."""
    import torch
    import chunked_ssd_scan_amd as ssd
    import ssd_inputs as si

    shape = si.CONFIGS[cfg]
    dev = torch.device("cuda:0")
    inp = si.make_inputs(shape, seed=0)
    g = inp.to(dev)
    b, T, R, H, P = g.x.shape
    y = torch.empty(g.x.shape, device=dev, dtype=torch.float32)
    fin = torch.empty((b, H, P, shape.dstate), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev).cuda_stream
    step = ssd_step_fn(ssd, g, shape, y, fin, stream, args.segments, args.block_slices)
    nwarm = prewarm(step, args.prewarm)
    wall, walks = timed_region_walks(step, args) if with_timed_region else (None, None)
    tc = time_calls(step, args.calls, FLUSH_BYTES)
    tc["walks_timed"] = walks
    if not (torch.isfinite(y).all() and torch.isfinite(fin).all()):
        raise RuntimeError(f"workload {cfg}: non-finite output")
    nbytes = algorithmic_bytes(shape)
    flops = algorithmic_flops(shape)
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if shape.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    gbs = lambda ms: nbytes / (ms * 1e-3) / 1e9
    summary = {
        "workload": shape.name, "tokens": shape.tokens,
        "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
        "walk_ms_median": tc["walk_ms_median"], "walk_ms_min": tc["walk_ms_min"],
        "forward_ms_median": tc["call_ms_median"], "forward_ms_min": tc["call_ms_min"],
        "walk_hbm_frac": gbs(tc["walk_ms_median"]) / HBM_PEAK_GBS,
        "forward_hbm_frac": gbs(tc["call_ms_median"]) / HBM_PEAK_GBS,
        "forward_tokens_per_s": shape.tokens / (tc["call_ms_median"] * 1e-3),
        "mfma_frac_walk": flops / (tc["walk_ms_median"] * 1e-3) / 1e12 / mfma_peak,
        "traffic": profiled_traffic(f"cfg{cfg}"),
        "prewarm_calls": nwarm,
    }
    return shape, inp, wall, tc, summary


def moments_flops(shape, trap: bool, valid_len: int) -> int:
    """Algorithmic flops of the state moments: per counted step and (batch,
    head) the unique entries of the Gram sum_p h[p,n] h[p,n'] (P N (N + 1) / 2
    multiply-adds) and the m1 sum (P N adds), plus the state writes of every
    step (2 P N R, twice for the two-write trapezoid)."""
    b, T, H, P, N, R = shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate, \
        shape.mimo_rank
    gram = P * N * (N + 1) + P * N
    writes = 2 * P * N * R * (2 if trap else 1)
    return b * H * (valid_len * gram + T * writes)


def moments_bench(args) -> dict:
    """Physical-frame state moments of the Mamba-3 trapezoid on the MIMO layer shape."""
    import torch
    import chunked_ssd_scan_amd as ssd
    import ssd_inputs as si

    shape = si.CONFIGS[3]
    dev = torch.device("cuda:0")
    ti = si.make_trapezoid_inputs(shape, seed=0)
    g = ti.to(dev)
    bi = g.base
    b, T, R, H, P = bi.x.shape
    N = shape.dstate
    vl = T
    m2 = torch.empty((b, H, N, N), device=dev)
    m1 = torch.empty((b, H, N), device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(walk_events=None):
        ssd.state_moments(bi.x, bi.da, bi.B, g.beta, g.gamma, g.prev_x, g.prev_B, bi.init_state,
                          bi.theta, valid_len=vl, m2=m2, m1=m1, stream=stream.cuda_stream)

    nwarm = prewarm(step, args.prewarm)
    wall = timed_region(step, args)
    # per-call event timing after the same flush as the other lines (the
    # moments entry point has no walk events: the call is the unit)
    flush = torch.empty(FLUSH_BYTES // 4, device=dev)
    ts = []
    for i in range(args.calls):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del flush
    # the timed region's average call is the roofline figure; the flushed
    # per-call median and minimum beside it
    call_ms = wall * 1e3 / args.steps
    if not (torch.isfinite(m2).all() and torch.isfinite(m1).all()):
        raise RuntimeError("non-finite output")
    flops = moments_flops(shape, True, vl)
    achieved = flops / (call_ms * 1e-3) / 1e12
    out = {
        "metric": "state moments tokens/s + % of MFMA roofline (b4,T4096,H32,P64,N128,R4 trapezoid)",
        "value": b * T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded; see ssd_inputs.make_trapezoid_inputs)",
        "config": {"workload": "mamba3 MIMO layer, trapezoid state moments " + shape.name,
                   "batch": b, "seqlen": T, "nheads": H, "headdim": P, "dstate": N,
                   "mimo_rank": R, "valid_len": vl, "rotation": True, "init_state": True,
                   "prev_token": True},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": None, "algorithmic_flops": flops, "kernel_ms": call_ms,
                     "forward_ms": call_ms,
                     "flushed": {"kernel_ms_median": statistics.median(ts), "kernel_ms_min": min(ts)}},
        "timing": {"prewarm_s": args.prewarm, "prewarm_calls": nwarm},
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        nbh = b * H
        nsl = max(1, min(args.cpu_slices // 40, nbh))
        sel = [int(i * nbh / nsl) for i in range(nsl)]
        t1 = time.perf_counter()
        oracle.state_moments(ti.base.x, ti.base.da, ti.base.B, ti.beta, ti.gamma, ti.prev_x,
                             ti.prev_B, ti.base.init_state, ti.base.theta, valid_len=vl, bh=sel,
                             nthreads=threads)
        secs = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": b * T * (nsl / nbh) / secs, "unit": "tokens/s",
                               "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": (f"{nsl} of the {nbh} (batch, head) slices over the full "
                                          f"T={T}; {secs:.2f} s wall; tokens/s scaled by the "
                                          f"slice fraction")}
    return out


def backward_bytes(shape) -> int:
    """Compulsory HBM bytes of the backward: x, B, C (input dtype), da, dy,
    theta, D, init and dfinal read once; dx, dda, dB, dC, dtheta, dinit and
    dD (fp32) written once."""
    b, T, H, P, N, G, R = shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate, \
        shape.ngroups, shape.mimo_rank
    esz = 2 if shape.dtype == "bf16" else 4
    xs, bs = b * T * R * H * P, b * T * R * G * N
    rd = xs * esz + 2 * bs * esz + b * T * H * 4 + xs * 4 + b * H * P * N * 4
    wr = xs * 4 + 2 * bs * 4 + b * T * H * 4 + b * H * P * N * 4
    if shape.rotation:
        rd += b * T * H * (N // 2) * 4
        wr += b * T * H * (N // 2) * 4
    if shape.init_state:
        rd += b * H * P * N * 4
    if shape.skip != "none":
        rd += H * 4
        wr += H * 4
    return rd + wr


def backward_flops(shape) -> int:
    """Algorithmic flops of the backward: per (batch, step, head) five rank-R
    contractions of a P x N state, 2 P N R each (the recomputed write
    x B^T, dC = dy^T h, the state-gradient read dy C^T, dx = H B, dB = H^T x)."""
    b, T, H, P, N, R = shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate, \
        shape.mimo_rank
    return 10 * b * T * H * P * N * R


def backward_bench(args) -> dict:
    """Gradients of the scan (dx, dda, dB, dC, dinit, dtheta, dD) on one layer shape."""
    import torch
    import chunked_ssd_scan_amd as ssd
    import ssd_inputs as si

    shape = si.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    inp = si.make_inputs(shape, seed=0)
    dy, df = si.make_cotangents(shape, seed=0)
    g = inp.to(dev)
    dyg, dfg = dy.to(dev), df.to(dev)
    b, T, R, H, P = g.x.shape
    N = shape.dstate
    stream = torch.cuda.current_stream(dev)
    out_t = {"dx": torch.empty(g.x.shape, device=dev), "dda": torch.empty((b, T, H), device=dev),
             "dB": torch.empty(g.B.shape, device=dev), "dC": torch.empty(g.B.shape, device=dev),
             "dinit": torch.empty((b, H, P, N), device=dev)}
    if g.theta is not None:
        out_t["dtheta"] = torch.empty((b, T, H, N // 2), device=dev)
    if g.D is not None:
        out_t["dD"] = torch.empty((H,), device=dev)

    def step(walk_events=None):
        ssd.backward(g.x, g.da, g.B, g.C, dyg, D=g.D, init_state=g.init_state, theta=g.theta,
                     dfinal=dfg, out=out_t, stream=stream.cuda_stream)

    nwarm = prewarm(step, args.prewarm)
    wall = timed_region(step, args)
    flush = torch.empty(FLUSH_BYTES // 4, device=dev)
    ts = []
    for i in range(args.calls):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del flush
    # the timed region's average call is the roofline figure; the flushed
    # per-call median and minimum beside it
    call_ms = wall * 1e3 / args.steps
    for k, v in out_t.items():
        if not torch.isfinite(v).all():
            raise RuntimeError(f"non-finite {k}")
    nbytes, flops = backward_bytes(shape), backward_flops(shape)
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if shape.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    out = {
        "metric": f"backward tokens/s + % of HBM roofline ({shape.name})",
        "value": b * T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded; see ssd_inputs.make_inputs and make_cotangents)",
        "config": {"workload": "backward " + shape.name, "batch": b, "seqlen": T, "nheads": H,
                   "headdim": P, "dstate": N, "mimo_rank": R, "rotation": shape.rotation,
                   "init_state": shape.init_state, "skip": shape.skip, "dfinal": True},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": profiled_traffic(f"backward_cfg{args.config}", "backward"),
                     "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                     "mfma_frac": flops / (call_ms * 1e-3) / 1e12 / mfma_peak,
                     "kernel_ms": call_ms, "unit_timed": "whole call",
                     "flushed": {"kernel_ms_median": statistics.median(ts), "kernel_ms_min": min(ts)}},
        "timing": {"prewarm_s": args.prewarm, "prewarm_calls": nwarm},
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        bs = max(1, min(b, threads))
        ts_tok = max(64, min(T, args.cpu_slices * 1024 // max(1, H * R)))
        cut = lambda t: None if t is None else t[:bs, :ts_tok].contiguous()
        x, da, Bm, Cm, th, dys = map(cut, (inp.x, inp.da, inp.B, inp.C, inp.theta, dy))
        h0 = None if inp.init_state is None else inp.init_state[:bs].contiguous()
        t1 = time.perf_counter()
        oracle.ssd_backward(x, da, Bm, Cm, dys, inp.D, h0, th, df[:bs].contiguous(),
                            nthreads=threads)
        secs = time.perf_counter() - t1
        used = min(threads, bs * shape.ngroups)
        out["cpu_baseline"] = {"value": bs * ts_tok / secs, "unit": "tokens/s", "cores": used,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": (f"batches 0..{bs - 1}, the first {ts_tok} of T={T} "
                                          f"tokens, all {H} heads; {secs:.2f} s wall (the "
                                          f"oracle runs one thread per (batch, group))")}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prewarm", type=float, default=2.0, metavar="SECONDS",
                    help="whole calls run back to back for this long before anything is timed, "
                         "whatever --warmup is (the shader clock ramps up from idle)")
    ap.add_argument("--calls", type=int, default=40,
                    help="per-call event timings (each after a 1 GiB flush) for median and min")
    ap.add_argument("--config", type=int, default=2,
                    help="workload id in ssd_inputs.CONFIGS (the reported line uses 2)")
    ap.add_argument("--other-workloads", default="1,3,4",
                    help="further workload ids timed the same way and reported under "
                         "'workloads' (empty: none)")
    ap.add_argument("--cpu-slices", type=int, default=320)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--segments", type=int, default=0)
    ap.add_argument("--block-slices", type=int, default=0)
    ap.add_argument("--workload", choices=("ssd", "selective_scan", "trapezoid", "moments",
                                           "backward"),
                    default="ssd",
                    help="ssd: the chunked SSD scan (the reported line); selective_scan: "
                         "the diagonal selective scan, b4 T4096 D512 N16 (--segments = chunks); "
                         "trapezoid: the Mamba-3 two-write forward on the MIMO layer shape; "
                         "moments: its physical-frame state moments; backward: the gradients "
                         "of the scan on workload --config")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 launches) for counter calibration")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: there is no multi-GPU path "
              "(the scan shards over (batch, head) without communication)",
              file=sys.stderr)
        return 2

    import torch
    import chunked_ssd_scan_amd as ssd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, device="cuda:0", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
        return 0
    ssd.load_library()
    if args.workload == "selective_scan":
        print(json.dumps(selective_bench(args)), flush=True)
        return 0
    if args.workload == "trapezoid":
        print(json.dumps(trapezoid_bench(args)), flush=True)
        return 0
    if args.workload == "moments":
        print(json.dumps(moments_bench(args)), flush=True)
        return 0
    if args.workload == "backward":
        print(json.dumps(backward_bench(args)), flush=True)
        return 0

    shape, inp, wall, tc, main_summary = ssd_workload(args.config, args, with_timed_region=True)
    print(f"# workload {args.config}: walk median {tc['walk_ms_median']:.4f} ms, call median "
          f"{tc['call_ms_median']:.4f} ms", file=sys.stderr, flush=True)
    others = {}
    for w in [int(v) for v in args.other_workloads.split(",") if v.strip()]:
        if w == args.config:
            continue
        _, _, _, otc, osum = ssd_workload(w, args, with_timed_region=False)
        print(f"# workload {w}: walk median {otc['walk_ms_median']:.4f} ms, call median "
              f"{otc['call_ms_median']:.4f} ms", file=sys.stderr, flush=True)
        others[str(w)] = osum
        torch.cuda.empty_cache()

    tokens = shape.batch * shape.seqlen
    ms_per_step = wall * 1e3 / args.steps
    nbytes = algorithmic_bytes(shape)
    flops = algorithmic_flops(shape)
    # the roofline figure: the output walk's average duration over the timed
    # region (HIP events around every timed walk); the whole call's is the
    # timed region's time per step. The flushed per-call medians and minima
    # are reported beside them.
    walk_ms = statistics.fmean(tc["walks_timed"])
    call_ms = ms_per_step
    achieved = nbytes / (walk_ms * 1e-3) / 1e9
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if shape.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    out = {
        "metric": "SSD scan fwd tokens/s + % of HBM/MFMA roofline (b8,T8192,H80,P64,N128)",
        "value": tokens * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded, layer-shaped; see ssd_inputs.py)",
        "config": {"workload": shape.name, "batch": shape.batch, "seqlen": shape.seqlen,
                   "nheads": shape.nheads, "headdim": shape.headdim, "dstate": shape.dstate,
                   "ngroups": shape.ngroups, "mimo_rank": shape.mimo_rank,
                   "chunk_len": shape.chunk_len, "kernel_tile_rows": KERNEL_TILE_ROWS,
                   "rotation": shape.rotation,
                   "segments": args.segments or "auto",
                   "block_slices": args.block_slices or "auto"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": main_summary["traffic"],
                     "algorithmic_bytes": nbytes, "kernel_ms": walk_ms,
                     "kernel_ms_timed_min": min(tc["walks_timed"]),
                     "kernel_ms_timed_max": max(tc["walks_timed"]),
                     "forward_ms": call_ms,
                     "forward_frac": nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "flushed": flushed_block(tc, nbytes, nbytes)},
        "mfma": {"algorithmic_tflop": flops / 1e12,
                 "tile_rows": KERNEL_TILE_ROWS,
                 "achieved_tflops": flops / (walk_ms * 1e-3) / 1e12,
                 "peak_tflops": mfma_peak,
                 "frac": flops / (walk_ms * 1e-3) / 1e12 / mfma_peak},
        "timing": {"prewarm_s": args.prewarm, "prewarm_calls": main_summary["prewarm_calls"],
                   "timed_region": "the K steps back to back, wall clock between two device "
                                   "synchronisations; the roofline's kernel_ms is the mean of "
                                   "HIP events around each timed step's output walk",
                   "flushed": f"{args.calls} calls, each after a {FLUSH_BYTES >> 20} MiB fill "
                              "that evicts L2 and MALL; medians and minima",
                   "workloads": "other workloads: flushed per-call medians"},
        "workloads": others,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, shape, args.cpu_slices)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
