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


def algorithmic_flops(s) -> int:
    """Causal (block-)lower-triangular K2 + K3 + K5 flops at the given chunk length."""
    b, T, H, P, N, G, R, l = (s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups,
                              s.mimo_rank, s.chunk_len)
    nc = -(-T // l)
    L = l * R
    tri = L * (L + 1) // 2
    k3 = 2 * b * H * T * R * P * N
    k5_off = 2 * b * H * T * R * P * N
    k5_diag = 2 * b * H * nc * tri * P
    k2 = 2 * b * nc * tri * N * (H if s.rotation else G)
    return k3 + k5_off + k5_diag + k2


# kernel sources behind each workload's counter summary
KERNEL_SOURCES = {
    "ssd": ("ssd_scan.hip", "ssd_common.h"),
    "selective_scan": ("sel_scan.hip", "ssd_common.h"),
    "trapezoid": ("ssd_scan.hip", "ssd_common.h", "trap_scan.hip"),
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


def time_walk(step, steps: int) -> float:
    """Mean duration (ms) of the output walk kernel over `steps` calls.

    Each call gets its own pair of HIP events, created without the system-scope
    fence (a timing-only event: no cache writeback between the two kernels of
    a call), which the library records just before and after the walk launch.
    """
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    no_fence = 0x20000000                      # hipEventDisableSystemFence

    def event():
        e = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(no_fence)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e.value

    pairs = [(event(), event()) for _ in range(steps)]
    for pr in pairs:
        step(walk_events=pr)
    if hip.hipDeviceSynchronize() != 0:
        raise RuntimeError("hipDeviceSynchronize failed")
    total = 0.0
    for a, b in pairs:
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        total += ms.value
        hip.hipEventDestroy(ctypes.c_void_p(a))
        hip.hipEventDestroy(ctypes.c_void_p(b))
    return total / steps


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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = start.elapsed_time(end) / args.steps
    out_ms = time_walk(step, args.steps)
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
                     "hbm_frac_forward": nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
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
                               "kind": "oracle",
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = start.elapsed_time(end) / args.steps
    walk_ms = time_walk(step, args.steps)
    if not (torch.isfinite(y).all() and torch.isfinite(fin).all()):
        raise RuntimeError("non-finite output")
    # the dominant kernel is the rotating walk over 2T sub-steps: its own
    # compulsory bytes are those of that single-write problem (no D), less
    # the y of the even sub-steps, which it does not write
    sub = dataclasses.replace(shape, seqlen=2 * T, skip="none")
    walk_bytes = algorithmic_bytes(sub) - b * T * R * H * P * 4
    esz = 2 if shape.dtype == "bf16" else 4
    trap_bytes = (algorithmic_bytes(dataclasses.replace(shape, skip="none"))
                  + 2 * b * T * H * 4 + b * R * (H * P + shape.ngroups * N) * esz)
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
                     "forward_frac": trap_bytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
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
                               "cores": threads, "kind": "oracle",
                               "sample": (f"{nsl} of the {nbh} (batch, head) slices over the full "
                                          f"T={T}; {secs:.2f} s wall; tokens/s scaled by the "
                                          f"slice fraction")}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=2,
                    help="workload id in ssd_inputs.CONFIGS (the reported line uses 2)")
    ap.add_argument("--cpu-slices", type=int, default=320)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--segments", type=int, default=0)
    ap.add_argument("--block-slices", type=int, default=0)
    ap.add_argument("--workload", choices=("ssd", "selective_scan", "trapezoid"), default="ssd",
                    help="ssd: the chunked SSD scan (the reported line); selective_scan: "
                         "the diagonal selective scan, b4 T4096 D512 N16 (--segments = chunks); "
                         "trapezoid: the Mamba-3 two-write forward on the MIMO layer shape")
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
    import ssd_inputs as si

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
    shape = si.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    inp = si.make_inputs(shape, seed=0)
    g = inp.to(dev)
    b, T, R, H, P = g.x.shape
    y = torch.empty(g.x.shape, device=dev, dtype=torch.float32)
    fin = torch.empty((b, H, P, shape.dstate), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)

    def step(walk_events=None):
        ssd.forward(g.x, g.da, g.B, g.C, g.D, g.init_state, shape.chunk_len, g.theta,
                    y=y, final_state=fin, segments=args.segments,
                    block_slices=args.block_slices, stream=stream.cuda_stream,
                    walk_events=walk_events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # one event pair on the launch stream around the whole timed region: the
    # average forward (both kernels, back to back) without per-step markers
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = start.elapsed_time(end) / args.steps
    # the dominant kernel alone: the library records a HIP event pair just
    # before and after the output walk of each call (same number of calls)
    walk_ms = time_walk(step, args.steps)
    if not (torch.isfinite(y).all() and torch.isfinite(fin).all()):
        print("non-finite output", file=sys.stderr)
        return 1

    tokens = shape.batch * shape.seqlen
    ms_per_step = wall * 1e3 / args.steps
    nbytes = algorithmic_bytes(shape)
    flops = algorithmic_flops(shape)
    achieved = nbytes / (walk_ms * 1e-3) / 1e9
    tag = f"cfg{args.config}"
    traffic = profiled_traffic(tag)
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
                   "chunk_len": shape.chunk_len, "rotation": shape.rotation,
                   "segments": args.segments or "auto",
                   "block_slices": args.block_slices or "auto"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": nbytes, "kernel_ms": walk_ms,
                     "forward_ms": launch_ms,
                     "forward_frac": nbytes / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "mfma": {"algorithmic_tflop": flops / 1e12,
                 "achieved_tflops": flops / (walk_ms * 1e-3) / 1e12,
                 "peak_tflops": mfma_peak,
                 "frac": flops / (walk_ms * 1e-3) / 1e12 / mfma_peak},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, shape, args.cpu_slices)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
