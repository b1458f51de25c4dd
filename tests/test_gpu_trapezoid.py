"""Mamba-3 trapezoid forward on the GPU vs the float64 oracle (needs a gfx950 GPU).

Bar: normwise max relative error per output tensor (y and final_state) within
1e-4 for fp32 inputs and 2e-2 for bf16 inputs. At the Mamba-3 MIMO layer
shape every (batch, head) slice is compared, in groups of slices.
"""
from __future__ import annotations

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


def run(ti, **kw):
    ssd = _ssd()
    g = ti.to(_dev())
    bi = g.base
    y, f = ssd.trapezoid(bi.x, bi.da, bi.B, bi.C, g.beta, g.gamma, g.prev_x, g.prev_B,
                         bi.init_state, ti.base.shape.chunk_len, bi.theta, **kw)
    torch.cuda.synchronize()
    return y, f


def ref(ti, bh=None):
    bi = ti.base
    return oracle.trapezoid(bi.x, bi.da, bi.B, bi.C, ti.beta, ti.gamma, ti.prev_x, ti.prev_B,
                            bi.init_state, bi.theta, bh=bh)


def check(ti, label):
    y, f = run(ti)
    yr, fr = ref(ti)
    tol = TOL[ti.base.shape.dtype]
    ey, ef = normwise(y.cpu().numpy(), yr), normwise(f.cpu().numpy(), fr)
    print(f"{label}: y err {ey:.3e} final err {ef:.3e} (tol {tol:g})", flush=True)
    assert ey <= tol and ef <= tol, (label, ey, ef)


# (T, P, N, R, H, G, dtype, rotation, init, prev)
CASES = [
    (1, 16, 16, 1, 2, 1, "f32", False, False, True),
    (37, 16, 32, 1, 3, 3, "f32", False, True, True),
    (100, 64, 64, 2, 4, 2, "f32", True, True, True),
    (33, 32, 128, 4, 2, 1, "f32", True, False, False),
    (257, 64, 128, 1, 4, 1, "bf16", False, True, True),
    (300, 64, 128, 4, 4, 1, "bf16", True, True, True),
    (129, 128, 64, 8, 2, 2, "bf16", True, False, True),
    (65, 64, 256, 2, 2, 1, "bf16", False, False, False),
]


@pytest.mark.parametrize("T,P,N,R,H,G,dtype,rot,init,prev", CASES)
def test_trapezoid_cases(T, P, N, R, H, G, dtype, rot, init, prev):
    shape = si.small_shape(seqlen=T, headdim=P, dstate=N, mimo_rank=R, nheads=H, ngroups=G,
                           dtype=dtype, rotation=rot, init_state=init, skip="none")
    ti = si.make_trapezoid_inputs(shape, seed=T + 3 * R, prev=prev)
    check(ti, f"T{T} P{P} N{N} R{R} H{H} G{G} {dtype} rot={rot} init={init} prev={prev}")


def test_trapezoid_mimo_layer_every_slice():
    # the Mamba-3 MIMO layer shape: b4 T4096 H32 P64 N128 R4, bf16, rotation,
    # init state, previous token; every (batch, head) slice is compared
    ti = si.make_trapezoid_inputs(si.CONFIGS[3], seed=0)
    y, f = run(ti)
    b, T, R, H, P = ti.base.x.shape
    yc, fc = y.cpu(), f.cpu()
    worst = (0.0, 0.0)
    num_y = num_f = den_y = den_f = 0.0
    for s0 in range(0, b * H, 32):
        sel = list(range(s0, min(b * H, s0 + 32)))
        ys, fs = ref(ti, bh=sel)
        for i, bh in enumerate(sel):
            bb, h = divmod(bh, H)
            gy, gf = yc[bb, :, :, h].double().numpy(), fc[bb, h].double().numpy()
            ey, ef = normwise(gy, ys[i]), normwise(gf, fs[i])
            worst = (max(worst[0], ey), max(worst[1], ef))
            num_y = max(num_y, float(np.abs(gy - ys[i]).max()))
            den_y = max(den_y, float(np.abs(ys[i]).max()))
            num_f = max(num_f, float(np.abs(gf - fs[i]).max()))
            den_f = max(den_f, float(np.abs(fs[i]).max()))
            assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (bh, ey, ef)
    ty, tf = num_y / den_y, num_f / den_f
    print(f"MIMO layer all {b * H} slices: tensor y err {ty:.3e} final err {tf:.3e}; worst "
          f"slice y {worst[0]:.3e} final {worst[1]:.3e}", flush=True)
    assert ty <= TOL["bf16"] and tf <= TOL["bf16"]


@pytest.mark.parametrize("split", [1, 50, 99])
def test_trapezoid_split_calls(split):
    # the second call starts from the first's final state with its last token
    # as the previous-token entries
    shape = si.small_shape(seqlen=100, headdim=64, dstate=64, mimo_rank=2, nheads=2,
                           rotation=True, init_state=True, skip="none")
    ti = si.make_trapezoid_inputs(shape, seed=9)
    y, f = run(ti)
    ssd = _ssd()
    g = ti.to(_dev())
    bi = g.base
    s = lambda t, a, b_: t[:, a:b_].contiguous()
    y1, f1 = ssd.trapezoid(s(bi.x, 0, split), s(bi.da, 0, split), s(bi.B, 0, split),
                           s(bi.C, 0, split), s(g.beta, 0, split), s(g.gamma, 0, split), g.prev_x,
                           g.prev_B, bi.init_state, 64, s(bi.theta, 0, split))
    y2, f2 = ssd.trapezoid(s(bi.x, split, 100), s(bi.da, split, 100), s(bi.B, split, 100),
                           s(bi.C, split, 100), s(g.beta, split, 100), s(g.gamma, split, 100),
                           bi.x[:, split - 1].contiguous(), bi.B[:, split - 1].contiguous(), f1, 64,
                           s(bi.theta, split, 100))
    torch.cuda.synchronize()
    yy = torch.cat([y1, y2], dim=1)
    assert normwise(yy.cpu().numpy(), y.cpu().numpy()) <= 1e-5
    assert normwise(f2.cpu().numpy(), f.cpu().numpy()) <= 1e-5


def test_trapezoid_final_state_in_place():
    shape = si.small_shape(seqlen=77, headdim=64, dstate=128, mimo_rank=1, nheads=2,
                           rotation=True, init_state=True, skip="none")
    ti = si.make_trapezoid_inputs(shape, seed=10)
    y, f = run(ti)
    ssd = _ssd()
    g = ti.to(_dev())
    bi = g.base
    h = bi.init_state.clone()
    y2, f2 = ssd.trapezoid(bi.x, bi.da, bi.B, bi.C, g.beta, g.gamma, g.prev_x, g.prev_B, h, 64,
                           bi.theta, final_state=h)
    torch.cuda.synchronize()
    assert f2.data_ptr() == h.data_ptr()
    assert torch.equal(y2, y) and torch.equal(f2, f)


@pytest.mark.parametrize("segments", [1, 3])
def test_trapezoid_launch_options(segments):
    # explicit segment counts for the scan over the 2T sub-steps, and walk
    # events around its output walk, leave the result within the bar
    shape = si.small_shape(seqlen=400, headdim=64, dstate=128, mimo_rank=4, nheads=2,
                           dtype="bf16", rotation=True, init_state=True, skip="none")
    ti = si.make_trapezoid_inputs(shape, seed=12)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    call = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    _dev()
    call[0].record()
    y, f = run(ti, segments=segments, walk_events=ev)
    call[1].record()
    torch.cuda.synchronize()
    assert 0.0 < ev[0].elapsed_time(ev[1]) <= call[0].elapsed_time(call[1])
    yr, fr = ref(ti)
    ey, ef = normwise(y.cpu().numpy(), yr), normwise(f.cpu().numpy(), fr)
    print(f"segments {segments}: y err {ey:.3e} final err {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (segments, ey, ef)
