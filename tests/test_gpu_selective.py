"""Diagonal selective scan on the GPU vs the float64 oracle (needs a gfx950 GPU).

Bar: normwise max relative error ||y - ref||_inf / ||ref||_inf within 1e-4
(fp32 inputs, fp32 arithmetic). At the full b4 T4096 D512 N16 size every
(batch, channel) sequence is compared; each is also held to the bar against
its own norm.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ssd_inputs as si

pytestmark = pytest.mark.gpu

TOL = 1e-4


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


def run(inp, y=None):
    ssd = _ssd()
    g = inp.to(_dev())
    y = ssd.selective_scan(g.u, g.delta, g.A, g.B, g.C, g.skip, y=y)
    torch.cuda.synchronize()
    return y


def check(inp, label):
    y = run(inp)
    ref = oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.skip)
    err = normwise(y.cpu().double().numpy(), ref)
    print(f"{label} y err {err:.3e} (tol {TOL:g})", flush=True)
    assert err <= TOL, (label, err)


def test_tiny_config():
    check(si.make_scan_inputs(si.SCAN_CONFIGS[0], seed=0), "tiny")


# (batch, T, D, N, dt_shift): ragged channel groups (D not a multiple of 64),
# odd state sizes in each kernel width, sequences shorter than a chunk, and
# long sequences on few channels (many chunks joined by the carry pass)
SHAPES = [
    (1, 1, 8, 4, 2.0), (1, 15, 64, 16, 2.0), (1, 16, 65, 16, 2.0), (1, 17, 1, 1, 2.0),
    (2, 100, 63, 17, 2.0), (3, 333, 130, 32, 2.0), (1, 257, 64, 33, 2.0),
    (2, 1000, 200, 64, 2.0), (1, 2000, 64, 16, 2.0), (1, 3001, 7, 5, 2.0),
    (1, 4096, 64, 16, 6.0), (2, 1500, 96, 48, 0.0), (1, 20001, 3, 2, 2.0),
]


@pytest.mark.parametrize("b,T,D,N,shift", SHAPES)
def test_shapes(b, T, D, N, shift):
    shape = si.ScanShape(b, T, D, N, shift, f"b{b} T{T} D{D} N{N}")
    check(si.make_scan_inputs(shape, seed=b * 7 + T), shape.name)


def test_full_size_every_channel():
    # b4 T4096 D512 N16: every one of the 2048 (batch, channel) sequences
    inp = si.make_scan_inputs(si.SCAN_CONFIGS[1], seed=0)
    b, T, Dm = inp.u.shape
    y = run(inp).cpu().double().numpy()
    ref = oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.skip)
    err = normwise(y, ref)
    per = np.abs(y - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-300)
    print(f"full size: all {b * Dm} channels, tensor y err {err:.3e}, worst channel "
          f"{float(per.max()):.3e}", flush=True)
    assert err <= TOL
    assert float(per.max()) <= TOL


def test_deterministic_and_in_place():
    inp = si.make_scan_inputs(si.ScanShape(2, 777, 100, 16, 2.0, ""), seed=3)
    y1 = run(inp)
    y2 = torch.full_like(y1, float("nan"))
    y2 = run(inp, y=y2)
    assert torch.equal(y1, y2)


def test_nan_stays_in_its_channel():
    # B and C are shared by every channel; a NaN in one channel's input must
    # not reach another channel, nor the same channel before it appears
    inp = si.make_scan_inputs(si.ScanShape(1, 600, 70, 16, 2.0, ""), seed=5)
    inp.u[0, 400, 9] = float("nan")
    y = run(inp).cpu()
    assert torch.isnan(y[0, 400:, 9]).all()
    assert torch.isfinite(y[0, :400, 9]).all()
    others = torch.cat([y[0, :, :9], y[0, :, 10:]], dim=1)
    assert torch.isfinite(others).all()


@pytest.mark.parametrize("chunks", [1, 2, 7, 100, 999, 5000])
def test_chunk_count_does_not_change_result(chunks):
    # explicit chunk counts, including more chunks than blocks of steps and
    # counts clamped to the sequence length (chunks of one step or empty)
    inp = si.make_scan_inputs(si.ScanShape(2, 999, 70, 16, 2.0, ""), seed=11)
    ssd = _ssd()
    g = inp.to(_dev())
    y = ssd.selective_scan(g.u, g.delta, g.A, g.B, g.C, g.skip, chunks=chunks)
    torch.cuda.synchronize()
    ref = oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.skip)
    err = normwise(y.cpu().double().numpy(), ref)
    print(f"chunks {chunks}: y err {err:.3e}", flush=True)
    assert err <= TOL, (chunks, err)


def test_walk_events_time_the_output_pass():
    ssd = _ssd()
    inp = si.make_scan_inputs(si.ScanShape(2, 2048, 256, 16, 2.0, ""), seed=2)
    g = inp.to(_dev())
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    call = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    call[0].record()
    y = ssd.selective_scan(g.u, g.delta, g.A, g.B, g.C, g.skip, walk_events=ev)
    call[1].record()
    torch.cuda.synchronize()
    t_out, t_call = ev[0].elapsed_time(ev[1]), call[0].elapsed_time(call[1])
    assert 0.0 < t_out <= t_call, (t_out, t_call)
    ref = oracle.selective_scan(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.skip)
    assert normwise(y.cpu().double().numpy(), ref) <= TOL
