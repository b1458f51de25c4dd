"""Physical-frame state moments on the GPU vs the float64 oracle (needs a gfx950 GPU).

Bar: normwise max relative error ||out - ref||_inf / ||ref||_inf per output
(m2 and m1) within 1e-4 for fp32 inputs and 2e-2 for bf16 inputs. At the
Mamba-3 MIMO layer shape every (batch, head) slice is compared.
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


def run(ti, trap, valid_len=None):
    ssd = _ssd()
    g = ti.to(_dev())
    bi = g.base
    kw = dict(beta=g.beta, gamma=g.gamma, prev_x=g.prev_x, prev_B=g.prev_B) if trap else {}
    m2, m1 = ssd.state_moments(bi.x, bi.da, bi.B, init_state=bi.init_state, theta=bi.theta,
                               valid_len=valid_len, **kw)
    torch.cuda.synchronize()
    return m2, m1


def ref(ti, trap, valid_len=None, bh=None):
    bi = ti.base
    kw = dict(beta=ti.beta, gamma=ti.gamma, prev_x=ti.prev_x, prev_B=ti.prev_B) if trap else {}
    return oracle.state_moments(bi.x, bi.da, bi.B, init_state=bi.init_state, theta=bi.theta,
                                valid_len=valid_len, bh=bh, **kw)


# (trap, T, valid_len, P, N, R, H, G, dtype, rotation, init)
CASES = [
    (False, 1, 1, 16, 16, 1, 2, 1, "f32", False, False),
    (False, 100, 77, 16, 32, 2, 3, 1, "f32", True, True),
    (False, 333, 333, 64, 128, 4, 2, 1, "bf16", True, True),
    (False, 257, 200, 32, 64, 1, 4, 2, "bf16", False, True),
    (False, 97, 97, 128, 64, 8, 2, 1, "f32", True, False),
    (False, 64, 60, 64, 128, 16, 2, 1, "bf16", True, True),
    (True, 1, 1, 16, 16, 1, 2, 1, "f32", True, True),
    (True, 150, 150, 64, 128, 4, 3, 1, "bf16", True, True),
    (True, 301, 123, 32, 64, 2, 2, 2, "f32", True, True),
    (True, 77, 77, 128, 128, 1, 2, 1, "bf16", False, True),
    (True, 500, 499, 64, 32, 4, 4, 1, "bf16", True, False),
]


@pytest.mark.parametrize("trap,T,vl,P,N,R,H,G,dtype,rot,init", CASES)
def test_moments_cases(trap, T, vl, P, N, R, H, G, dtype, rot, init):
    shape = si.small_shape(seqlen=T, headdim=P, dstate=N, mimo_rank=R, nheads=H, ngroups=G,
                           dtype=dtype, rotation=rot, init_state=init, skip="none", dt_shift=4.0)
    ti = si.make_trapezoid_inputs(shape, seed=T + 7 * R + N)
    m2, m1 = run(ti, trap, vl)
    r2, r1 = ref(ti, trap, vl)
    e2, e1 = normwise(m2.cpu().numpy(), r2), normwise(m1.cpu().numpy(), r1)
    print(f"trap={trap} T{T} vl{vl} P{P} N{N} R{R} {dtype} rot={rot}: m2 err {e2:.3e} "
          f"m1 err {e1:.3e} (tol {TOL[dtype]:g})", flush=True)
    assert e2 <= TOL[dtype] and e1 <= TOL[dtype], (e2, e1)
    assert torch.equal(m2, m2.transpose(-1, -2))


@pytest.mark.parametrize("trap", [False, True])
def test_moments_long_sequence_segments(trap):
    # few (batch, head) pairs and a long sequence: the plan splits it into
    # segments whose entering states come from the forward's state passes
    shape = si.small_shape(batch=1, seqlen=3000, nheads=2, headdim=64, dstate=128, mimo_rank=4,
                           dtype="bf16", rotation=True, init_state=True, skip="none", dt_shift=5.0)
    ti = si.make_trapezoid_inputs(shape, seed=81)
    m2, m1 = run(ti, trap, 2900)
    r2, r1 = ref(ti, trap, 2900)
    e2, e1 = normwise(m2.cpu().numpy(), r2), normwise(m1.cpu().numpy(), r1)
    print(f"segments trap={trap}: m2 err {e2:.3e} m1 err {e1:.3e}", flush=True)
    assert e2 <= TOL["bf16"] and e1 <= TOL["bf16"]


def test_moments_mimo_layer_every_slice():
    # the Mamba-3 MIMO layer shape, trapezoid: b4 T4096 H32 P64 N128 R4, bf16,
    # rotation, init state, previous token; valid_len short of T
    ti = si.make_trapezoid_inputs(si.CONFIGS[3], seed=0)
    vl = 4000
    m2, m1 = run(ti, True, vl)
    r2, r1 = ref(ti, True, vl)
    b, H = m2.shape[:2]
    g2, g1 = m2.cpu().numpy(), m1.cpu().numpy()
    e2, e1 = normwise(g2, r2), normwise(g1, r1)
    per = [normwise(g2[i, j], r2[i, j]) for i in range(b) for j in range(H)]
    print(f"MIMO layer all {b * H} slices: m2 err {e2:.3e} m1 err {e1:.3e}; worst slice m2 "
          f"{max(per):.3e}", flush=True)
    assert e2 <= TOL["bf16"] and e1 <= TOL["bf16"] and max(per) <= TOL["bf16"]


def test_moments_in_place_and_deterministic():
    ssd = _ssd()
    shape = si.small_shape(seqlen=200, headdim=64, dstate=64, mimo_rank=2, nheads=2,
                           rotation=True, init_state=True, skip="none")
    ti = si.make_trapezoid_inputs(shape, seed=82)
    a2, a1 = run(ti, True)
    g = ti.to(_dev())
    m2 = torch.full_like(a2, float("nan"))
    m1 = torch.full_like(a1, float("nan"))
    bi = g.base
    o2, o1 = ssd.state_moments(bi.x, bi.da, bi.B, g.beta, g.gamma, g.prev_x, g.prev_B,
                               bi.init_state, bi.theta, m2=m2, m1=m1)
    torch.cuda.synchronize()
    assert o2.data_ptr() == m2.data_ptr() and torch.equal(o2, a2) and torch.equal(o1, a1)
