"""Gradients of the scan on the GPU vs the float64 oracle (needs a gfx950 GPU).

Bar: normwise max relative error ||out - ref||_inf / ||ref||_inf per output
(dx, dda, dB, dC, dinit, dtheta, dD) within 1e-4 for fp32 inputs and 2e-2 for
bf16 inputs (the contractions take dy and the state gradient in bf16 there).
dda and dtheta are sums of per-step inner products that can cancel to zero
(exactly so at T = 1 from a zero state), so their denominator is at least the
size of those products, max over (b, t) of sum |C dC| + |B dB|.
"""
from __future__ import annotations

import types

import numpy as np
import pytest
import torch

import oracle
import ssd_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _ssd():
    import chunked_ssd_scan_amd as ssd
    ssd.load_library()
    return ssd


def normwise(got, ref):
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


def run(inp, dy, df):
    ssd = _ssd()
    dev = _dev()
    g = inp.to(dev)
    out = ssd.backward(g.x, g.da, g.B, g.C, dy.to(dev), D=g.D, init_state=g.init_state,
                       theta=g.theta, dfinal=None if df is None else df.to(dev))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def ref(inp, dy, df):
    return oracle.ssd_backward(inp.x, inp.da, inp.B, inp.C, dy, inp.D, inp.init_state, inp.theta,
                               df)


def step_scale(inp, want):
    C, B = inp.C.double().numpy(), inp.B.double().numpy()
    per_step = (np.abs(C * want["dC"]) + np.abs(B * want["dB"])).sum(axis=(2, 3, 4))
    return float(per_step.max())


def compare(got, want, tol, label, inp):
    assert set(got) == set(want), (sorted(got), sorted(want))
    floor = step_scale(inp, want)
    errs = {}
    for k in want:
        g, w = np.asarray(got[k], np.float64), np.asarray(want[k], np.float64)
        den = max(np.abs(w).max(), floor if k in ("dda", "dtheta") else 0.0, 1e-300)
        errs[k] = float(np.abs(g - w).max() / den)
    print(f"{label}: " + " ".join(f"{k} {e:.2e}" for k, e in errs.items()) + f" (tol {tol:g})",
          flush=True)
    for k, e in errs.items():
        assert e <= tol, (k, e)
    return errs


# (T, P, N, R, H, G, dtype, rotation, init, skip, dfinal)
CASES = [
    (1, 16, 16, 1, 2, 1, "f32", False, False, "none", False),
    (1, 16, 16, 1, 2, 1, "f32", True, True, "randn", True),
    (100, 16, 32, 2, 3, 1, "f32", True, True, "randn", True),
    (97, 128, 64, 8, 2, 1, "f32", True, False, "randn", True),
    (45, 64, 128, 1, 2, 2, "f32", True, True, "none", True),
    (200, 32, 16, 16, 4, 2, "f32", False, True, "randn", False),
    (333, 64, 128, 4, 2, 1, "bf16", True, True, "none", True),
    (257, 32, 64, 1, 4, 2, "bf16", False, True, "randn", True),
    (64, 64, 128, 16, 2, 1, "bf16", True, True, "randn", False),
    (130, 128, 128, 2, 2, 1, "bf16", True, False, "none", True),
    # bf16 without rotation, headdim <= 64: the chunked walks
    (300, 64, 128, 1, 2, 1, "bf16", False, True, "randn", True),
    (77, 16, 16, 2, 3, 1, "bf16", False, False, "none", True),
    (129, 32, 32, 4, 4, 2, "bf16", False, True, "randn", False),
    (64, 64, 64, 16, 2, 1, "bf16", False, True, "none", True),
    (1, 64, 128, 1, 2, 1, "bf16", False, True, "randn", True),
    (500, 64, 128, 8, 2, 2, "bf16", False, False, "randn", True),
    (45, 32, 128, 2, 2, 1, "bf16", False, True, "randn", True),
    # bf16 with rotation, headdim <= 64: the chunked walks in the folded frame
    (210, 32, 64, 8, 4, 2, "bf16", True, True, "randn", True),
    (1, 16, 32, 4, 2, 1, "bf16", True, True, "none", True),
    # the partials' reduction in several rank passes with odd head counts,
    # and nine heads a group at rank 1 (heads four at a time)
    (90, 32, 64, 8, 5, 1, "bf16", True, True, "randn", True),
    (70, 16, 32, 16, 3, 1, "f32", True, True, "none", True),
    (110, 64, 128, 1, 18, 2, "bf16", True, False, "randn", True),
]


@pytest.mark.parametrize("T,P,N,R,H,G,dtype,rot,init,skip,dfin", CASES)
def test_backward_cases(T, P, N, R, H, G, dtype, rot, init, skip, dfin):
    shape = si.small_shape(seqlen=T, headdim=P, dstate=N, mimo_rank=R, nheads=H, ngroups=G,
                           dtype=dtype, rotation=rot, init_state=init, skip=skip, dt_shift=3.0)
    seed = T + 7 * R + N
    inp = si.make_inputs(shape, seed=seed)
    dy, df = si.make_cotangents(shape, seed=seed, dfinal=dfin)
    compare(run(inp, dy, df), ref(inp, dy, df), TOL[dtype],
            f"T{T} P{P} N{N} R{R} H{H} G{G} {dtype} rot={rot} init={init} D={skip} dfinal={dfin}",
            inp)


@pytest.mark.parametrize("dtype,rot", [("f32", True), ("bf16", True), ("bf16", False)])
def test_backward_long_sequence_segments(dtype, rot):
    # few (batch, head) pairs and a long sequence: the plan splits it into
    # segments, so both walks start from carried states (forward: the state
    # passes; backward: the reverse state pass and its carry)
    shape = si.small_shape(batch=1, seqlen=3000, nheads=2, headdim=64, dstate=128, mimo_rank=4,
                           dtype=dtype, rotation=rot, init_state=True, skip="randn", dt_shift=5.0)
    inp = si.make_inputs(shape, seed=91)
    dy, df = si.make_cotangents(shape, seed=91)
    compare(run(inp, dy, df), ref(inp, dy, df), TOL[dtype], f"segments {dtype} rot={rot}", inp)


def test_backward_in_place_and_deterministic():
    ssd = _ssd()
    dev = _dev()
    shape = si.small_shape(seqlen=150, headdim=64, dstate=64, mimo_rank=2, nheads=2,
                           rotation=True, init_state=True, skip="randn", dtype="bf16")
    inp = si.make_inputs(shape, seed=92)
    dy, df = si.make_cotangents(shape, seed=92)
    first = run(inp, dy, df)
    g = inp.to(dev)
    out = {k: torch.full(v.shape, float("nan"), device=dev) for k, v in first.items()}
    res = ssd.backward(g.x, g.da, g.B, g.C, dy.to(dev), D=g.D, init_state=g.init_state,
                       theta=g.theta, dfinal=df.to(dev), out=out)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert res[k].data_ptr() == out[k].data_ptr()
        assert np.array_equal(res[k].cpu().numpy(), v), k


@pytest.mark.parametrize("segments_shape", [False, True])
def test_backward_on_a_caller_stream(segments_shape):
    # the call runs its forward-direction chain on a stream of its own and
    # joins it back into the caller's stream: on a non-default caller stream
    # the outputs match the default stream's bit for bit, and a copy queued on
    # that stream right after the call (before any host synchronisation) sees
    # them complete. The long shape has segments (state passes on both chains)
    ssd = _ssd()
    dev = _dev()
    if segments_shape:
        shape = si.small_shape(batch=1, seqlen=3000, nheads=2, headdim=64, dstate=128, mimo_rank=4,
                               dtype="bf16", rotation=True, init_state=True, skip="randn", dt_shift=5.0)
    else:
        shape = si.small_shape(seqlen=300, headdim=64, dstate=128, mimo_rank=1, nheads=4,
                               dtype="bf16", skip="randn")
    inp = si.make_inputs(shape, seed=93)
    dy, df = si.make_cotangents(shape, seed=93)
    first = run(inp, dy, df)
    g = inp.to(dev)
    dyg, dfg = dy.to(dev), df.to(dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        res = ssd.backward(g.x, g.da, g.B, g.C, dyg, D=g.D, init_state=g.init_state, theta=g.theta,
                           dfinal=dfg, stream=side.cuda_stream)
        copies = {k: v.clone() for k, v in res.items()}
    side.synchronize()
    for k, v in first.items():
        assert np.array_equal(copies[k].cpu().numpy(), v), k


@pytest.mark.parametrize("cfg", [1, 3])
def test_backward_full_layer_every_element(cfg):
    # full layer shapes, every output element compared: the Mamba-2 130M
    # layer (b4 T4096 H24 P64 N128, D) and the Mamba-3 MIMO layer (b4 T4096
    # H32 P64 N128 R4, rotation, init state), bf16
    shape = si.CONFIGS[cfg]
    inp = si.make_inputs(shape, seed=cfg)
    dy, df = si.make_cotangents(shape, seed=cfg)
    got = run(inp, dy, df)
    want = ref(inp, dy, df)
    errs = compare(got, want, TOL[shape.dtype], shape.name, inp)
    # worst (batch, head) slice of the per-head outputs
    worst = 0.0
    for k in ("dx", "dinit"):
        g, w = got[k], want[k]
        for bi in range(shape.batch):
            for h in range(shape.nheads):
                sl = (bi, slice(None), slice(None), h) if k == "dx" else (bi, h)
                worst = max(worst, normwise(g[sl], w[sl]))
    print(f"{shape.name}: worst (batch, head) slice of dx/dinit {worst:.2e}", flush=True)
    assert worst <= TOL[shape.dtype]
    assert max(errs.values()) <= TOL[shape.dtype]


def test_backward_bench_layer_sampled_batches():
    # the backward bench's layer at full size (Mamba-2 2.7B: b8 T8192 H80 P64
    # N128, D, dfinal), one call as bench.py times it; the oracle runs on two
    # whole batches (batches are independent; every head of a batch, so dB and
    # dC are complete), and dx, dda, dB, dC and dinit of those batches are
    # compared element by element. dD sums over the batches and is left out
    shape = si.CONFIGS[2]
    inp = si.make_inputs(shape, seed=0)
    dy, df = si.make_cotangents(shape, seed=0)
    got = run(inp, dy, df)
    for bi in (0, shape.batch - 1):
        sl = lambda t: None if t is None else t[bi:bi + 1]
        want = oracle.ssd_backward(sl(inp.x), sl(inp.da), sl(inp.B), sl(inp.C), sl(dy), inp.D,
                                   sl(inp.init_state), sl(inp.theta), sl(df))
        want = {k: v for k, v in want.items() if k in ("dx", "dda", "dB", "dC", "dinit")}
        g = {k: got[k][bi:bi + 1] for k in want}
        compare(g, want, TOL[shape.dtype], f"{shape.name} batch {bi}",
                types.SimpleNamespace(B=inp.B[bi:bi + 1], C=inp.C[bi:bi + 1]))

