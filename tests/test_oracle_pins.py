"""Pins that tie the float64 oracle to the pages and to mathematics (CPU only).

Each test computes the expected value another way than the oracle's token
recurrence: closed forms, the one-chunk quadratic (segsum) form, the K1..K5
chunk algorithm, explicit decay products, the Mamba-1 selective-scan statement,
exact invariants (linearity, causality, split calls), and the decay factors
printed in the LeetGPU worked example. The last test plants mistakes in copies
of the oracle source and checks that the pins catch every one of them.
"""
from __future__ import annotations

import json
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import forms
import oracle
import ssd_inputs as si

HERE = os.path.dirname(os.path.abspath(__file__))
TOL = 1e-10   # float64 formulations that differ only in summation order


def relerr(a, ref):
    a, ref = np.asarray(a), np.asarray(ref)
    return float(np.abs(a - ref).max() / max(np.abs(ref).max(), 1e-300))


def ora(inp, **kw):
    return oracle.ssd_oracle_inputs(inp, **kw)


def args(inp):
    return (inp.x, inp.da, inp.B, inp.C, inp.D, inp.init_state, inp.theta)


CASES = {
    "siso": dict(),
    "siso_init": dict(init_state=True),
    "mimo3": dict(mimo_rank=3),
    "rot": dict(rotation=True),
    "rot_init_mimo2": dict(rotation=True, init_state=True, mimo_rank=2),
    "groups2": dict(nheads=4, ngroups=2, init_state=True),
    "bf16": dict(dtype="bf16", mimo_rank=2, rotation=True),
    "noskip": dict(skip="none", seqlen=20),
    "t1": dict(seqlen=1, init_state=True, rotation=True, mimo_rank=2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_quadratic_form(name):
    inp = si.make_inputs(si.small_shape(**CASES[name]), seed=1)
    y, f = ora(inp)
    yq, fq = forms.quadratic_form(*args(inp))
    assert relerr(y, yq) < TOL and relerr(f, fq) < TOL


@pytest.mark.parametrize("chunk_len", [1, 3, 8, 16, 37, 64])
def test_chunk_length_independence(chunk_len):
    # "mamba3/scan.py" verify(): chunk sizes 8/16/64 and a ragged length 37
    inp = si.make_inputs(si.small_shape(seqlen=37, mimo_rank=2, rotation=True,
                                        init_state=True), seed=2)
    y, f = ora(inp)
    yc, fc = forms.chunked_form(*args(inp), chunk_len=chunk_len)
    assert relerr(y, yc) < TOL and relerr(f, fc) < TOL


def test_product_form_tiny():
    inp = si.make_inputs(si.small_shape(batch=1, seqlen=9, nheads=2, headdim=4, dstate=6,
                                        mimo_rank=2, rotation=True, init_state=True), seed=3)
    y, f = ora(inp)
    yp, fp = forms.product_form(*args(inp))
    assert relerr(y, yp) < TOL and relerr(f, fp) < TOL


def test_da_zero_is_pure_cumsum():
    inp = si.make_inputs(si.small_shape(mimo_rank=2, init_state=True), seed=4)
    inp.da.zero_()
    y, f = ora(inp)
    x, B, C, D, h0 = map(forms.f64, (inp.x, inp.B, inp.C, inp.D, inp.init_state))
    # S_t = h0 + sum_{s<=t} sum_r x_{s,r} (outer) B_{s,r}
    W = np.einsum("btrhp,btrhn->bthpn", x, np.repeat(B, x.shape[3] // B.shape[3], axis=3))
    S = np.cumsum(W, axis=1) + h0[:, None]
    Cx = np.repeat(C, x.shape[3] // C.shape[3], axis=3)
    yc = np.einsum("btrhn,bthpn->btrhp", Cx, S) + D[None, None, None, :, None] * x
    assert relerr(y, yc) < TOL and relerr(f, S[:, -1]) < TOL


@pytest.mark.parametrize("a", [-0.3, -1.7])
def test_constant_decay_geometric_series(a):
    T = 50
    x = torch.ones(1, T, 1, 1, 1)
    B = torch.ones(1, T, 1, 1, 1)
    y, f = oracle.ssd_oracle(x, torch.full((1, T, 1), a), B, B.clone())
    a = float(np.float32(a))                                 # da is stored in fp32
    t = np.arange(T)
    expect = (1 - np.exp(a * (t + 1))) / (1 - np.exp(a))   # the write at t is read at t
    assert relerr(y[0, :, 0, 0, 0], expect) < 1e-13
    assert abs(f[0, 0, 0, 0] - expect[-1]) < 1e-13


def test_constant_theta_closed_form():
    # one write at t=0 of (1, 0), no decay: the state turns by theta each later step
    T, th = 40, 0.37
    x = torch.zeros(1, T, 1, 1, 1)
    x[0, 0] = 1.0
    B = torch.zeros(1, T, 1, 1, 2)
    B[0, 0, 0, 0, 0] = 1.0
    C = torch.zeros(1, T, 2, 1, 2)   # rank 0 reads cos, rank 1 reads sin
    C[..., 0, 0, 0] = 1.0
    C[..., 1, 0, 1] = 1.0
    x2 = torch.cat([x, x * 0], dim=2)
    B2 = torch.cat([B, B * 0], dim=2)
    theta = torch.full((1, T, 1, 1), th)
    y, f = oracle.ssd_oracle(x2, torch.zeros(1, T, 1), B2, C, theta=theta)
    th = float(np.float32(th))                               # theta is stored in fp32
    t = np.arange(T)
    assert relerr(y[0, :, 0, 0, 0], np.cos(t * th)) < 1e-12
    assert relerr(y[0, :, 1, 0, 0], np.sin(t * th)) < 1e-12
    # an initial state is turned by the inclusive cumulative angle (t+1)*theta
    h0 = torch.zeros(1, 1, 1, 2)
    h0[0, 0, 0, 0] = 1.0
    y, f = oracle.ssd_oracle(x2 * 0, torch.zeros(1, T, 1), B2, C, init_state=h0, theta=theta)
    assert relerr(y[0, :, 0, 0, 0], np.cos((t + 1) * th)) < 1e-12
    assert relerr(y[0, :, 1, 0, 0], np.sin((t + 1) * th)) < 1e-12
    assert relerr(f[0, 0, 0], [math.cos(T * th), math.sin(T * th)]) < 1e-12


def test_theta_zero_is_no_rotation():
    inp = si.make_inputs(si.small_shape(rotation=True, init_state=True), seed=5)
    inp.theta.zero_()
    y, f = ora(inp)
    y0, f0 = oracle.ssd_oracle(inp.x, inp.da, inp.B, inp.C, inp.D, inp.init_state)
    assert np.array_equal(y, y0) and np.array_equal(f, f0)


def test_rotation_identity_folded_frame():
    # h_t = R(Phi_t) g_t: the physical recurrence equals the un-rotated recurrence
    # on B~ = R(-Phi) B, C~ = R(-Phi) C, and the final states differ by R(Phi_{T-1})
    inp = si.make_inputs(si.small_shape(rotation=True, init_state=True, mimo_rank=2,
                                        nheads=2), seed=6)
    y, f = ora(inp)
    b, T, R, G, N = inp.B.shape
    H = inp.x.shape[3]
    assert G == 1
    Phi = np.cumsum(forms.f64(inp.theta), axis=1)          # [b,T,H,N/2]
    for h in range(H):
        Bt = forms.rotate_pairs(forms.f64(inp.B)[:, :, :, 0, :], -Phi[:, :, None, h, :])
        Ct = forms.rotate_pairs(forms.f64(inp.C)[:, :, :, 0, :], -Phi[:, :, None, h, :])
        tt = lambda a: torch.from_numpy(np.ascontiguousarray(a[:, :, :, None, :]))
        yg, fg = oracle.ssd_oracle(inp.x[:, :, :, h:h + 1].double().contiguous(), inp.da[:, :, h:h + 1].contiguous(),
                                   tt(Bt), tt(Ct), inp.D[h:h + 1].contiguous(),
                                   inp.init_state[:, h:h + 1].contiguous())
        assert relerr(y[:, :, :, h], yg[:, :, :, 0]) < TOL
        fphys = forms.rotate_pairs(fg[:, 0], Phi[:, -1, h][:, None, :])
        assert relerr(f[:, h], fphys) < TOL


def _slice_t(inp, t0, t1, init):
    sl = lambda a: None if a is None else a[:, t0:t1].contiguous()
    return oracle.ssd_oracle(sl(inp.x), sl(inp.da), sl(inp.B), sl(inp.C), inp.D,
                             init, sl(inp.theta))


@pytest.mark.parametrize("split", [1, 13, 36])
def test_split_call_composition(split):
    inp = si.make_inputs(si.small_shape(seqlen=37, rotation=True, init_state=True,
                                        mimo_rank=2), seed=7)
    y, f = ora(inp)
    y1, f1 = _slice_t(inp, 0, split, inp.init_state)
    y2, f2 = _slice_t(inp, split, 37, torch.from_numpy(f1).float())
    # the hand-over rounds the carried state to fp32 (init_state is fp32)
    assert relerr(np.concatenate([y1, y2], axis=1), y) < 1e-6
    assert relerr(f2, f) < 1e-6


def test_mimo_extra_ranks_zero_is_siso():
    inp = si.make_inputs(si.small_shape(mimo_rank=3, skip="none", init_state=True), seed=8)
    inp.x[:, :, 1:] = 0
    y, f = ora(inp)
    for r in range(3):
        yr, fr = oracle.ssd_oracle(inp.x[:, :, :1].contiguous(), inp.da,
                                   inp.B[:, :, :1].contiguous(), inp.C[:, :, r:r + 1].contiguous(),
                                   None, inp.init_state)
        assert relerr(y[:, :, r], yr[:, :, 0]) < TOL
        assert relerr(f, fr) < TOL


def test_linearity_in_x_and_initial_state():
    inp = si.make_inputs(si.small_shape(mimo_rank=2, rotation=True, init_state=True,
                                        skip="none"), seed=9)
    y, f = ora(inp)
    yx, fx = oracle.ssd_oracle(inp.x, inp.da, inp.B, inp.C, None, None, inp.theta)
    yh, fh = oracle.ssd_oracle(inp.x * 0, inp.da, inp.B, inp.C, None, inp.init_state, inp.theta)
    assert relerr(yx + yh, y) < TOL and relerr(fx + fh, f) < TOL


def test_skip_term():
    inp = si.make_inputs(si.small_shape(mimo_rank=2), seed=10)
    y, _ = ora(inp)
    y0, _ = oracle.ssd_oracle(inp.x, inp.da, inp.B, inp.C, None)
    Dx = forms.f64(inp.D)[None, None, None, :, None] * forms.f64(inp.x)
    assert relerr(y - y0, Dx) < TOL


def test_causality():
    # "mamba3/scan.py" verify(): appending large future tokens leaves the past unchanged
    inp = si.make_inputs(si.small_shape(seqlen=30, mimo_rank=2, rotation=True,
                                        init_state=True), seed=11)
    y, _ = ora(inp)
    t0 = 17
    for t in (inp.x, inp.B, inp.C, inp.theta):
        t[:, t0:] *= 50
    inp.da[:, t0:] = -5.0
    y2, _ = ora(inp)
    assert np.array_equal(y[:, :t0], y2[:, :t0])
    assert not np.allclose(y[:, t0:], y2[:, t0:])


def test_mamba1_selective_scan_special_case():
    # The LeetGPU statement with a decay row constant over n (A[d, n] = a_d) is this
    # scan with one head per channel, P = 1, G = 1, x = delta*u, da = delta*a_d.
    # Its skip term multiplies u (not x = delta*u), so it is added outside.
    g = torch.Generator().manual_seed(12)
    b, T, Dm, N = 2, 23, 5, 7
    u = torch.randn(b, T, Dm, generator=g)
    delta = torch.nn.functional.softplus(torch.randn(b, T, Dm, generator=g))
    a = -torch.rand(Dm, generator=g) * 2 - 0.1
    A = a[:, None].expand(Dm, N).contiguous()
    Bm = torch.randn(b, T, N, generator=g)
    Cm = torch.randn(b, T, N, generator=g)
    skip = torch.randn(Dm, generator=g)
    ref = forms.mamba1_scan(u, delta, A, Bm, Cm, skip)
    x = (delta * u)[:, :, None, :, None].contiguous()        # [b,T,1,H=D,P=1]
    da = (delta * a).contiguous()                             # [b,T,H]
    y, _ = oracle.ssd_oracle(x, da, Bm[:, :, None, None, :].contiguous(),
                             Cm[:, :, None, None, :].contiguous())
    got = y[:, :, 0, :, 0] + forms.f64(skip) * forms.f64(u)
    assert relerr(got, ref) < 1e-6                            # x, da rounded to fp32


def test_single_step():
    inp = si.make_inputs(si.small_shape(seqlen=1, init_state=True, mimo_rank=2), seed=13)
    y, f = ora(inp)
    x, da, B, C, D, h0 = map(forms.f64, (inp.x, inp.da, inp.B, inp.C, inp.D, inp.init_state))
    for bi in range(x.shape[0]):
        for h in range(x.shape[3]):
            S = math.exp(da[bi, 0, h]) * h0[bi, h] + x[bi, 0, :, h].T @ B[bi, 0, :, 0]
            assert relerr(f[bi, h], S) < TOL
            yy = C[bi, 0, :, 0] @ S.T + D[h] * x[bi, 0, :, h]
            assert relerr(y[bi, 0, :, h], yy) < TOL


def test_golden_selective_scan_decay_factors():
    gold = json.load(open(os.path.join(HERE, "golden", "selective_scan_abar.json")))
    T = 4
    for a, printed in zip(gold["A_row"], gold["Abar_printed"]):
        x = torch.zeros(1, T, 1, 1, 1)
        x[0, 0] = 1.0
        ones = torch.ones(1, T, 1, 1, 1)
        da = torch.full((1, T, 1), gold["delta"] * a)
        y, _ = oracle.ssd_oracle(x, da, ones, ones.clone())
        ratio = y[0, 1:, 0, 0, 0] / y[0, :-1, 0, 0, 0]           # one step of decay
        assert np.allclose(np.round(ratio, gold["decimals"]), printed)


def test_bf16_inputs_are_decoded_exactly():
    inp = si.make_inputs(si.small_shape(dtype="bf16", rotation=True, mimo_rank=2), seed=14)
    y, f = ora(inp)
    y32, f32 = oracle.ssd_oracle(inp.x.float(), inp.da, inp.B.float(), inp.C.float(),
                                 inp.D, None, inp.theta)
    assert np.array_equal(y, y32) and np.array_equal(f, f32)


def test_slice_selection_matches_full_run():
    inp = si.make_inputs(si.small_shape(mimo_rank=2, rotation=True), seed=15)
    y, f = ora(inp)
    H = inp.x.shape[3]
    sel = [4, 0, 3]
    ys, fs = ora(inp, bh=sel)
    for i, bh in enumerate(sel):
        assert np.array_equal(ys[i], y[bh // H, :, :, bh % H])
        assert np.array_equal(fs[i], f[bh // H, bh % H])


# ----------------------------------------------------------------------------
# Planted mistakes: each mutant copy of the oracle must fail some pin.
# ----------------------------------------------------------------------------
MUTANTS = {
    "rotation_sign": ("S[p * N + 2 * k] = c * a0 - s * a1;", "S[p * N + 2 * k] = c * a0 + s * a1;"),
    "dropped_skip": ("acc += dh * load_elem", "acc += 0.0 * dh * load_elem"),
    "decay_sign": ("double a = exp((double)pr->da", "double a = exp(-(double)pr->da"),
    "decay_one_step_late": ("pr->da[(b * T + t) * H + h]", "pr->da[(b * T + (t > 0 ? t - 1 : 0)) * H + h]"),
    "rank_zero_only_written": ("int64_t xrow = (((b * T + t) * R + r) * H + h) * P;\n            int64_t brow",
                               "int64_t xrow = (((b * T + t) * R + 0) * H + h) * P;\n            int64_t brow"),
    "group_index": ("const int64_t g = h / (H / G);", "const int64_t g = h % G;"),
    "write_uses_C": ("load_elem(pr->B, brow + n", "load_elem(pr->C, brow + n"),
    "init_ignored": ("S[i] = (double)h0[i];", "S[i] = 0.0 * h0[i];"),
    "theta_wrong_head": ("((b * T + t) * H + h) * (N / 2)", "((b * T + t) * H + (H - 1 - h)) * (N / 2)"),
}


def _pin_battery(lib_path):
    """Quadratic-form and closed-form checks against a given oracle build."""
    worst = 0.0
    for kw in (dict(mimo_rank=2, rotation=True, init_state=True, nheads=4, ngroups=2),
               dict(seqlen=12, skip="randn")):
        inp = si.make_inputs(si.small_shape(**kw), seed=16)
        y, f = oracle.ssd_oracle(*args(inp), lib_path=lib_path)
        yq, fq = forms.quadratic_form(*args(inp))
        worst = max(worst, relerr(y, yq), relerr(f, fq))
    return worst


def test_pins_catch_planted_mistakes(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")).read()
    assert _pin_battery(None) < TOL
    # each mistake is planted in the SSD recurrence's slice function only
    a, b = src.index("static void run_slice("), src.index("int ssd_oracle_f64(")
    body = src[a:b]
    for name, (old, new) in MUTANTS.items():
        assert body.count(old) == 1, name
        path = tmp_path / f"{name}.c"
        path.write_text(src[:a] + body.replace(old, new) + src[b:])
        so = str(tmp_path / f"{name}.so")
        subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", so, str(path), "-lm"], check=True)
        assert _pin_battery(so) > 1e-6, f"planted mistake {name!r} was not caught"


# --------------------------------------------------------------------------
# Mamba-1 selective scan oracle ("SSM Selective Scan", problem statement)
# --------------------------------------------------------------------------

def _scan_inputs(b=2, T=29, Dm=5, N=3, seed=31):
    return si.make_scan_inputs(si.ScanShape(b, T, Dm, N), seed=seed)


def test_selective_scan_matches_the_statement_form():
    # forms.mamba1_scan writes the page's four equations per (b, d) with NumPy;
    # D != N and b > 1 catch transposed A or swapped B/C indices.
    s = _scan_inputs()
    y = oracle.selective_scan(s.u, s.delta, s.A, s.B, s.C, s.skip)
    ref = forms.mamba1_scan(s.u, s.delta, s.A, s.B, s.C, s.skip)
    assert relerr(y, ref) < TOL


def test_selective_scan_scalar_decay_is_the_ssd_scan():
    # A[d, n] = a_d for all n: one head per channel, P = 1, x = delta*u,
    # da = delta*a_d, shared B and C; the skip term multiplies u.
    s = _scan_inputs(b=2, T=23, Dm=4, N=6, seed=32)
    a = s.A[:, :1]
    A = a.expand(-1, s.A.shape[1]).contiguous()
    y = oracle.selective_scan(s.u, s.delta, A, s.B, s.C, s.skip)
    x = (s.delta.double() * s.u.double())[:, :, None, :, None].contiguous()
    da = (s.delta.double() * a[:, 0].double()).float().contiguous()
    ys, _ = oracle.ssd_oracle(x, da, s.B.double()[:, :, None, None, :].contiguous(),
                              s.C.double()[:, :, None, None, :].contiguous())
    got = ys[:, :, 0, :, 0] + forms.f64(s.skip) * forms.f64(s.u)
    assert relerr(y, got) < 1e-6          # da rounded to fp32 for the SSD oracle


def test_selective_scan_closed_form_constant_inputs():
    # Constant u, delta, B, C: h_t[n] = delta B_n u (1 - Abar_n^(t+1)) / (1 - Abar_n).
    T, Dm, N = 40, 3, 4
    g = torch.Generator().manual_seed(33)
    A = -torch.rand(Dm, N, generator=g) * 2 - 0.05
    dl, uu = 0.3, 1.7
    Bv = torch.randn(N, generator=g)
    Cv = torch.randn(N, generator=g)
    skip = torch.randn(Dm, generator=g)
    u = torch.full((1, T, Dm), uu)
    delta = torch.full((1, T, Dm), dl)
    Bm = Bv.expand(1, T, N).contiguous()
    Cm = Cv.expand(1, T, N).contiguous()
    y = oracle.selective_scan(u, delta, A, Bm, Cm, skip)
    dl, uu = float(delta[0, 0, 0]), float(u[0, 0, 0])                    # the stored fp32 values
    abar = np.exp(dl * forms.f64(A))                                       # [D,N]
    t = np.arange(T)[:, None, None]
    h = dl * forms.f64(Bv) * uu * (1 - abar[None] ** (t + 1)) / (1 - abar[None])   # [T,D,N]
    ref = (h * forms.f64(Cv)).sum(-1) + forms.f64(skip) * uu
    assert relerr(y[0], ref) < 1e-12


def test_selective_scan_golden_decay_factors():
    # The worked example's printed Abar for delta = 1 and its A row: a unit
    # impulse at t = 0 with B = C = 1 decays by Abar per step.
    gold = json.load(open(os.path.join(HERE, "golden", "selective_scan_abar.json")))
    T = 4
    for a, printed in zip(gold["A_row"], gold["Abar_printed"]):
        u = torch.zeros(1, T, 1)
        u[0, 0] = 1.0
        ones = torch.ones(1, T, 1)
        y = oracle.selective_scan(u, ones * gold["delta"], torch.tensor([[a]]), ones, ones.clone(),
                                  torch.zeros(1))
        ratio = y[0, 1:, 0] / y[0, :-1, 0]
        assert np.allclose(np.round(ratio, gold["decimals"]), printed)


def test_selective_scan_causal_and_channels_independent():
    s = _scan_inputs(b=1, T=30, Dm=6, N=5, seed=34)
    y = oracle.selective_scan(s.u, s.delta, s.A, s.B, s.C, s.skip)
    u2 = s.u.clone()
    u2[:, 17:, 2] += 3.0
    y2 = oracle.selective_scan(u2, s.delta, s.A, s.B, s.C, s.skip)
    assert np.array_equal(y[:, :17], y2[:, :17])
    others = [d for d in range(6) if d != 2]
    assert np.array_equal(y[:, :, others], y2[:, :, others])
    assert not np.allclose(y[:, 17:, 2], y2[:, 17:, 2])


def test_selective_scan_selected_channels():
    s = _scan_inputs(b=2, T=9, Dm=4, N=3, seed=35)
    y = oracle.selective_scan(s.u, s.delta, s.A, s.B, s.C, s.skip)
    sel = [0, 5, 7]
    ys = oracle.selective_scan(s.u, s.delta, s.A, s.B, s.C, s.skip, bd=sel)
    for i, bd in enumerate(sel):
        assert np.array_equal(ys[i], y[bd // 4, :, bd % 4])


SCAN_MUTANTS = {
    "scan_dropped_skip": ("acc += (double)skip[d] * ut;", "acc += 0.0 * skip[d] * ut;"),
    "scan_A_transposed": ("(double)A[d * N + n]", "(double)A[n * Dm + d]"),
    "scan_bbar_without_delta": ("const double bbar = dl * (double)B[row * N + n];",
                                "const double bbar = (double)B[row * N + n];"),
    "scan_read_before_write": ("h[n] = abar * h[n] + bbar * ut;\n                    acc += (double)C[row * N + n] * h[n];",
                               "acc += (double)C[row * N + n] * h[n];\n                    h[n] = abar * h[n] + bbar * ut;"),
    "scan_B_for_C": ("acc += (double)C[row * N + n] * h[n];", "acc += (double)B[row * N + n] * h[n];"),
}


def test_selective_scan_pins_catch_planted_mistakes(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")).read()
    s = _scan_inputs(b=2, T=17, Dm=5, N=3, seed=36)
    ref = forms.mamba1_scan(s.u, s.delta, s.A, s.B, s.C, s.skip)
    for name, (old, new) in SCAN_MUTANTS.items():
        assert src.count(old) == 1, name
        path = tmp_path / f"{name}.c"
        path.write_text(src.replace(old, new))
        so = str(tmp_path / f"{name}.so")
        subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", so, str(path), "-lm"], check=True)
        y = oracle.selective_scan(s.u, s.delta, s.A, s.B, s.C, s.skip, lib_path=so)
        assert relerr(y, ref) > 1e-6, f"planted mistake {name!r} was not caught"


# ---------------------------------------------------------------------------
# Mamba-3 trapezoid (two-write) recurrence
# ---------------------------------------------------------------------------

def _trap(ti, lib_path=None, **kw):
    bi = ti.base
    args = dict(prev_x=ti.prev_x, prev_B=ti.prev_B, init_state=bi.init_state, theta=bi.theta)
    args.update(kw)
    return oracle.trapezoid(bi.x, bi.da, bi.B, bi.C, ti.beta, ti.gamma, lib_path=lib_path, **args)


TRAP_SHAPES = [dict(seqlen=23, rotation=True, init_state=True, mimo_rank=2),
               dict(seqlen=17, rotation=False, init_state=False, mimo_rank=1, ngroups=3, nheads=3),
               dict(seqlen=11, rotation=True, init_state=True, mimo_rank=1, dtype="bf16")]


def test_trapezoid_beta0_gamma1_is_the_ssd_scan():
    # beta = 0, gamma = 1 leaves the single-write recurrence ("mamba3/scan.py",
    # docstring, with the trapezoid weights at their one-write values)
    ti = si.make_trapezoid_inputs(si.small_shape(seqlen=19, rotation=True, init_state=True,
                                                 mimo_rank=2), seed=40)
    bi = ti.base
    y, f = oracle.trapezoid(bi.x, bi.da, bi.B, bi.C, torch.zeros_like(ti.beta),
                            torch.ones_like(ti.gamma), ti.prev_x, ti.prev_B, bi.init_state,
                            bi.theta)
    ys, fs = oracle.ssd_oracle(ti.base.x, ti.base.da, ti.base.B, ti.base.C, None,
                               ti.base.init_state, ti.base.theta)
    assert relerr(y, ys) < 1e-12 and relerr(f, fs) < 1e-12


@pytest.mark.parametrize("kw", TRAP_SHAPES)
def test_trapezoid_matches_the_frame_form(kw):
    ti = si.make_trapezoid_inputs(si.small_shape(**kw), seed=41)
    y, f = _trap(ti)
    bi = ti.base
    yr, fr = forms.trapezoid_frame_form(bi.x, bi.da, bi.B, bi.C, ti.beta, ti.gamma, ti.prev_x,
                                        ti.prev_B, bi.init_state, bi.theta)
    assert relerr(y, yr) < TOL and relerr(f, fr) < TOL


def test_trapezoid_matches_the_two_channel_expansion():
    # "mamba3/moments.rs", module documentation: the trapezoid as one
    # scalar-decay system with 2R channels, x^ = [gamma x, beta x_prev],
    # b^ = [B~, B~_prev] (rotated B, the previous token's shifted in), run by
    # the single-write oracle without rotation in the rotated frame
    ti = si.make_trapezoid_inputs(si.small_shape(seqlen=21, rotation=True, init_state=True,
                                                 mimo_rank=2, nheads=2), seed=42)
    bi = ti.base
    y, f = _trap(ti)
    x, B, C = forms.f64(bi.x), forms.f64(bi.B), forms.f64(bi.C)
    b, T, R, H, P = x.shape
    N = B.shape[-1]
    Phi = np.cumsum(forms.f64(bi.theta), axis=1)                       # [b,T,H,N/2]
    Phi_prev = np.concatenate([np.zeros_like(Phi[:, :1]), Phi[:, :-1]], axis=1)
    Bh = np.repeat(B, H, axis=3) if B.shape[3] == 1 else B              # per head
    Ch = np.repeat(C, H, axis=3) if C.shape[3] == 1 else C
    Bt = forms.rotate_pairs(Bh, -Phi[:, :, None])                       # B~_t
    Ct = forms.rotate_pairs(Ch, -Phi[:, :, None])
    Bp = np.concatenate([np.repeat(forms.f64(ti.prev_B), H, axis=2)[:, None], Bh[:, :-1]], axis=1)
    Btp = forms.rotate_pairs(Bp, -Phi_prev[:, :, None])                 # B~_{t-1}
    xp = np.concatenate([forms.f64(ti.prev_x)[:, None], x[:, :-1]], axis=1)
    ga, be = forms.f64(ti.gamma), forms.f64(ti.beta)
    xh = np.concatenate([ga[:, :, None, :, None] * x, be[:, :, None, :, None] * xp], axis=2)
    bh = np.concatenate([Bt, Btp], axis=2)
    ch = np.concatenate([Ct, Ct], axis=2)
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    ye, fe = oracle.ssd_oracle(tt(xh), bi.da, tt(bh), tt(ch), None, bi.init_state)
    assert relerr(y, ye[:, :, :R]) < TOL
    fphys = forms.rotate_pairs(fe, Phi[:, -1][:, :, None, :])
    assert relerr(f, fphys) < TOL


def test_trapezoid_closed_form_constant_inputs():
    # no rotation, one rank, constant decay, weights and write S = x B^T, no
    # previous token: h_0 = gamma S, h_t = a h_{t-1} + (beta + gamma) S, so
    # h_t = a^t gamma S + (beta + gamma) S (1 - a^t) / (1 - a)
    b, T, H, P, N = 1, 12, 1, 3, 4
    rng = np.random.default_rng(5)
    xv = rng.standard_normal(P).astype(np.float32)
    bv = rng.standard_normal(N).astype(np.float32)
    cv = rng.standard_normal(N).astype(np.float32)
    x = torch.from_numpy(np.tile(xv, (b, T, 1, H, 1)))
    B = torch.from_numpy(np.tile(bv, (b, T, 1, 1, 1)))
    C = torch.from_numpy(np.tile(cv, (b, T, 1, 1, 1)))
    da = torch.full((b, T, H), -0.3)
    beta, gamma = torch.full((b, T, H), 0.45), torch.full((b, T, H), 0.7)
    y, f = oracle.trapezoid(x, da, B, C, beta, gamma)
    a, be, ga = math.exp(float(da[0, 0, 0])), float(beta[0, 0, 0]), float(gamma[0, 0, 0])
    S = np.outer(xv.astype(np.float64), bv.astype(np.float64))
    for t in range(T):
        ht = a ** t * ga * S + (be + ga) * S * (1 - a ** t) / (1 - a)
        assert np.allclose(y[0, t, 0, 0], ht @ cv.astype(np.float64), rtol=1e-12, atol=1e-12)
    assert np.allclose(f[0, 0], ht, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("split", [1, 9, 22])
def test_trapezoid_split_call_composition(split):
    # the second call takes the first's final state and its last token as the
    # previous-token entries ("mamba3/moments.rs": the beta stream's first
    # element comes from the cache)
    ti = si.make_trapezoid_inputs(si.small_shape(seqlen=23, rotation=True, init_state=True,
                                                 mimo_rank=2), seed=43)
    bi = ti.base
    y, f = _trap(ti)
    sl = lambda a, t0, t1: a[:, t0:t1].contiguous()
    y1, f1 = oracle.trapezoid(sl(bi.x, 0, split), sl(bi.da, 0, split), sl(bi.B, 0, split),
                              sl(bi.C, 0, split), sl(ti.beta, 0, split), sl(ti.gamma, 0, split),
                              ti.prev_x, ti.prev_B, bi.init_state, sl(bi.theta, 0, split))
    y2, f2 = oracle.trapezoid(sl(bi.x, split, 23), sl(bi.da, split, 23), sl(bi.B, split, 23),
                              sl(bi.C, split, 23), sl(ti.beta, split, 23), sl(ti.gamma, split, 23),
                              bi.x[:, split - 1].contiguous(), bi.B[:, split - 1].contiguous(),
                              torch.from_numpy(f1).float(), sl(bi.theta, split, 23))
    assert relerr(np.concatenate([y1, y2], axis=1), y) < 1e-6
    assert relerr(f2, f) < 1e-6


def test_trapezoid_selected_slices():
    ti = si.make_trapezoid_inputs(si.small_shape(seqlen=13, rotation=True, nheads=3), seed=44)
    y, f = _trap(ti)
    ys, fs = _trap(ti, bh=[5, 0, 3])
    H = ti.base.x.shape[3]
    for i, bh in enumerate([5, 0, 3]):
        bb, h = divmod(bh, H)
        assert np.array_equal(ys[i], y[bb, :, :, h]) and np.array_equal(fs[i], f[bb, h])


TRAP_MUTANTS = {
    # the docstring's literal form: the previous write added after the rotation
    "trap_beta_not_rotated": [
        ("for (int64_t i = 0; i < P * N; ++i) S[i] = a * S[i] + be * Wp[i];",
         "for (int64_t i = 0; i < P * N; ++i) S[i] = a * S[i];"),
        ("for (int64_t i = 0; i < P * N; ++i) S[i] += ga * Wc[i];",
         "for (int64_t i = 0; i < P * N; ++i) S[i] += ga * Wc[i] + be * Wp[i];")],
    "trap_no_shift": [("S[i] = a * S[i] + be * Wp[i];", "S[i] = a * S[i] + be * Wc[i];")],
    "trap_gamma_dropped": [("S[i] += ga * Wc[i];", "S[i] += Wc[i];")],
    "trap_prev_ignored": [("if (prev_x && prev_B) {", "if (0) {")],
    "trap_beta_undecayed": [("S[i] = a * S[i] + be * Wp[i];", "S[i] = a * (S[i] + be * Wp[i]);")],
}


def test_trapezoid_pins_catch_planted_mistakes(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")).read()
    ti = si.make_trapezoid_inputs(si.small_shape(seqlen=15, rotation=True, init_state=True,
                                                 mimo_rank=2), seed=45)
    bi = ti.base
    yr, fr = forms.trapezoid_frame_form(bi.x, bi.da, bi.B, bi.C, ti.beta, ti.gamma, ti.prev_x,
                                        ti.prev_B, bi.init_state, bi.theta)
    for name, edits in TRAP_MUTANTS.items():
        mutated = src
        for old, new in edits:
            assert mutated.count(old) == 1, (name, old)
            mutated = mutated.replace(old, new)
        path = tmp_path / f"{name}.c"
        path.write_text(mutated)
        so = str(tmp_path / f"{name}.so")
        subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", so, str(path), "-lm"], check=True)
        y, f = _trap(ti, lib_path=so)
        assert relerr(y, yr) > 1e-6 or relerr(f, fr) > 1e-6, name


# ---------------------------------------------------------------------------
# Physical-frame state moments ("mamba3/moments.rs", module documentation
# steps 1-4 and state_moments_phys)
# ---------------------------------------------------------------------------

def _moments(ti, trap=True, lib_path=None, **kw):
    bi = ti.base
    if trap:
        args = dict(beta=ti.beta, gamma=ti.gamma, prev_x=ti.prev_x, prev_B=ti.prev_B)
    else:
        args = {}
    args.update(init_state=bi.init_state, theta=bi.theta)
    args.update(kw)
    return oracle.state_moments(bi.x, bi.da, bi.B, lib_path=lib_path, **args)


def _sums(states, valid_len):
    """m2, m1 of states [b,T,H,P,N] over t < valid_len, written out."""
    h = states[:, :valid_len]
    m2 = np.einsum("bthpn,bthpk->bhnk", h, h)
    m1 = h.sum(axis=(1, 3))
    return m2, m1


MOMENT_CASES = [
    (True, dict(seqlen=19, rotation=True, init_state=True, mimo_rank=2), 19),
    (True, dict(seqlen=23, rotation=True, init_state=False, mimo_rank=1, nheads=3, ngroups=3), 15),
    (False, dict(seqlen=21, rotation=True, init_state=True, mimo_rank=4), 21),
    (False, dict(seqlen=17, rotation=False, init_state=True, mimo_rank=1, dtype="bf16"), 9),
    (True, dict(seqlen=13, rotation=True, init_state=True, mimo_rank=2, dtype="bf16"), 1),
]


@pytest.mark.parametrize("trap,kw,vl", MOMENT_CASES)
def test_moments_from_prefix_final_states(trap, kw, vl):
    # h_t is the final state of the prefix [0, t]: the moments from the
    # final states the pinned recurrences give for every prefix
    ti = si.make_trapezoid_inputs(si.small_shape(**kw), seed=50 + vl)
    bi = ti.base
    m2, m1 = _moments(ti, trap, valid_len=vl)
    b, T, R, H, P = bi.x.shape
    N = bi.B.shape[-1]
    states = np.empty((b, vl, H, P, N))
    sl = lambda a, t: None if a is None else a[:, :t + 1].contiguous()
    for t in range(vl):
        if trap:
            _, f = oracle.trapezoid(sl(bi.x, t), sl(bi.da, t), sl(bi.B, t), sl(bi.C, t),
                                    sl(ti.beta, t), sl(ti.gamma, t), ti.prev_x, ti.prev_B,
                                    bi.init_state, sl(bi.theta, t))
        else:
            _, f = oracle.ssd_oracle(sl(bi.x, t), sl(bi.da, t), sl(bi.B, t), sl(bi.C, t), None,
                                     bi.init_state, sl(bi.theta, t))
        states[:, t] = f
    r2, r1 = _sums(states, vl)
    assert relerr(m2, r2) < 1e-12 and relerr(m1, r1) < 1e-12


@pytest.mark.parametrize("trap,kw,vl", MOMENT_CASES)
def test_moments_match_the_frame_form_states(trap, kw, vl):
    ti = si.make_trapezoid_inputs(si.small_shape(**kw), seed=60 + vl)
    bi = ti.base
    m2, m1 = _moments(ti, trap, valid_len=vl)
    if trap:
        st = forms.trapezoid_frame_states(bi.x, bi.da, bi.B, ti.beta, ti.gamma, ti.prev_x,
                                          ti.prev_B, bi.init_state, bi.theta)
    else:
        st = forms.trapezoid_frame_states(bi.x, bi.da, bi.B, h0=bi.init_state, theta=bi.theta)
    r2, r1 = _sums(st, vl)
    assert relerr(m2, r2) < TOL and relerr(m1, r1) < TOL


def test_moments_ignore_padded_tokens():
    # tokens at t >= valid_len step the state but do not count, whatever
    # their values ("mamba3/moments.rs": the valid_len mask alone excludes
    # pad garbage)
    ti = si.make_trapezoid_inputs(si.small_shape(seqlen=30, rotation=True, init_state=True,
                                                 mimo_rank=2), seed=70)
    bi = ti.base
    m2, m1 = _moments(ti, valid_len=30)
    pad = si.make_trapezoid_inputs(si.small_shape(seqlen=41, rotation=True, init_state=True,
                                                  mimo_rank=2), seed=71)
    cat = lambda a, p: torch.cat([a, p[:, 30:]], dim=1)
    pb = pad.base
    q2, q1 = oracle.state_moments(cat(bi.x, pb.x), cat(bi.da, pb.da), cat(bi.B, pb.B),
                                  cat(ti.beta, pad.beta), cat(ti.gamma, pad.gamma), ti.prev_x,
                                  ti.prev_B, bi.init_state, cat(bi.theta, pb.theta), valid_len=30)
    assert np.array_equal(m2, q2) and np.array_equal(m1, q1)


def test_moments_pure_cumsum_closed_form():
    # da = 0, no rotation, no initial state, single write: h_t is the
    # cumulative sum of the writes x_s (outer) B_s
    shape = si.small_shape(seqlen=16, rotation=False, init_state=False, mimo_rank=2)
    inp = si.make_inputs(shape, seed=72)
    da = torch.zeros_like(inp.da)
    m2, m1 = oracle.state_moments(inp.x, da, inp.B)
    x, B = forms.f64(inp.x), forms.f64(inp.B)
    W = np.einsum("btrhp,btrhn->bthpn", x, B[:, :, :, forms._groups(x.shape[3], B.shape[3])])
    r2, r1 = _sums(np.cumsum(W, axis=1), 16)
    assert relerr(m2, r2) < 1e-12 and relerr(m1, r1) < 1e-12


def test_moments_selected_slices():
    ti = si.make_trapezoid_inputs(si.small_shape(seqlen=12, rotation=True, nheads=3), seed=73)
    m2, m1 = _moments(ti)
    s2, s1 = _moments(ti, bh=[4, 1])
    H = ti.base.x.shape[3]
    for i, bh in enumerate([4, 1]):
        bb, h = divmod(bh, H)
        assert np.array_equal(s2[i], m2[bb, h]) and np.array_equal(s1[i], m1[bb, h])


MOMENT_MUTANTS = {
    "mom_mask_off_by_one": [("if (t < valid_len) {", "if (t <= valid_len && t < T) {")],
    "mom_gram_diagonal": [("m2[n * N + n2] += hv * st[p * N + n2];",
                           "m2[n * N + n2] += hv * st[p * N + n];")],
    "mom_m1_squared": [("m1[n] += hv;", "m1[n] += hv * hv;")],
    "mom_turn_sign": [("st[p * N + 2 * k] = co * e0 - si * e1;", "st[p * N + 2 * k] = co * e0 + si * e1;")],
    "mom_counted_before_write": [
        ("for (int64_t i = 0; i < PN; ++i) st[i] += wg * wnow[i];\n        for (int64_t i = 0; i < PN; ++i) wlast[i] = wnow[i];",
         "for (int64_t i = 0; i < PN; ++i) wlast[i] = wnow[i];"),
        ("                    for (int64_t n2 = 0; n2 < N; ++n2) m2[n * N + n2] += hv * st[p * N + n2];\n                }\n        }",
         "                    for (int64_t n2 = 0; n2 < N; ++n2) m2[n * N + n2] += hv * st[p * N + n2];\n                }\n        }\n        for (int64_t i = 0; i < PN; ++i) st[i] += wg * wnow[i];")],
    "mom_init_dropped": [("st[i] = pr->init_state ? (double)pr->init_state[(b * H + h) * PN + i] : 0.0;",
                          "st[i] = 0.0;")],
}


def test_moments_pins_catch_planted_mistakes(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")).read()
    ti = si.make_trapezoid_inputs(si.small_shape(seqlen=15, rotation=True, init_state=True,
                                                 mimo_rank=2), seed=74)
    bi = ti.base
    st = forms.trapezoid_frame_states(bi.x, bi.da, bi.B, ti.beta, ti.gamma, ti.prev_x, ti.prev_B,
                                      bi.init_state, bi.theta)
    r2, r1 = _sums(st, 11)
    for name, edits in MOMENT_MUTANTS.items():
        mutated = src
        for old, new in edits:
            assert mutated.count(old) == 1, (name, old)
            mutated = mutated.replace(old, new)
        path = tmp_path / f"{name}.c"
        path.write_text(mutated)
        so = str(tmp_path / f"{name}.so")
        subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", so, str(path), "-lm"], check=True)
        m2, m1 = _moments(ti, lib_path=so, valid_len=11)
        assert relerr(m2, r2) > 1e-6 or relerr(m1, r1) > 1e-6, name


# ---------------------------------------------------------------------------
# Backward ("mamba3/scan.py", verify(): forward and backward checked
# separately against the recurrence at float64)
# ---------------------------------------------------------------------------

def _bwd_inputs(seed, T=13, H=3, G=1, P=4, N=6, R=2, rot=True, init=True, skip=True,
                dtype="f32", dfinal=True):
    shape = si.small_shape(seqlen=T, nheads=H, ngroups=G, headdim=P, dstate=N, mimo_rank=R,
                           dtype=dtype, rotation=rot, init_state=init,
                           skip="randn" if skip else "none", dt_shift=1.0)
    inp = si.make_inputs(shape, seed=seed)
    g = torch.Generator().manual_seed(seed + 1000)
    b = shape.batch
    dy = torch.randn((b, T, R, H, P), generator=g)
    df = torch.randn((b, H, P, N), generator=g) if dfinal else None
    return inp, dy, df


def _bwd(inp, dy, df, lib_path=None):
    return oracle.ssd_backward(inp.x, inp.da, inp.B, inp.C, dy, inp.D, inp.init_state, inp.theta,
                               df, lib_path=lib_path)


BWD_CASES = [dict(), dict(rot=False), dict(init=False, skip=False, dfinal=False),
             dict(R=1, G=3, H=3), dict(dtype="bf16", R=4, N=8), dict(T=1)]


@pytest.mark.parametrize("kw", BWD_CASES)
def test_backward_matches_float64_autograd(kw):
    inp, dy, df = _bwd_inputs(80 + len(kw), **kw)
    got = _bwd(inp, dy, df)
    ref = forms.autograd_gradients(inp.x, inp.da, inp.B, inp.C, dy, inp.D, inp.init_state,
                                   inp.theta, df)
    if inp.init_state is None:
        ref["dinit"] = None
    for k, v in ref.items():
        if v is None:
            continue
        assert relerr(got[k], v) < 1e-12, (k, relerr(got[k], v))


def test_backward_finite_differences():
    # central differences of L = <dy, y> + <dfinal, final> through the forward
    # oracle, for a few elements of x (float64 inputs) and of da
    inp, dy, df = _bwd_inputs(90, T=7, H=2, P=3, N=4, R=2)
    inp.x, inp.B, inp.C = inp.x.double(), inp.B.double(), inp.C.double()
    got = _bwd(inp, dy, df)
    d64 = lambda a: a.double().numpy()

    def loss(x=None, da=None):
        y, f = oracle.ssd_oracle(inp.x if x is None else x, inp.da if da is None else da, inp.B,
                                 inp.C, inp.D, inp.init_state, inp.theta)
        return float((y * d64(dy)).sum() + (f * d64(df)).sum())

    eps = 1e-6
    for idx in [(0, 0, 0, 0, 0), (1, 3, 1, 1, 2), (0, 6, 1, 0, 1)]:
        xp, xm = inp.x.clone(), inp.x.clone()
        xp[idx] += eps
        xm[idx] -= eps
        fd = (loss(x=xp) - loss(x=xm)) / (2 * eps)
        assert abs(fd - got["dx"][idx]) < 1e-6 * max(1.0, abs(fd)), (idx, fd, got["dx"][idx])
    for idx in [(0, 0, 0), (1, 4, 1), (0, 6, 1)]:
        # da is float32: the difference quotient uses the perturbation as stored
        h = 2.0 ** -12
        dp, dm = inp.da.clone(), inp.da.clone()
        dp[idx] += h
        dm[idx] -= h
        step = float(dp[idx].double() - dm[idx].double())
        fd = (loss(da=dp) - loss(da=dm)) / step
        assert abs(fd - got["dda"][idx]) < 1e-5 * max(1.0, abs(fd)), (idx, fd, got["dda"][idx])


def _reverse_cumsum(a, axis=1):
    return np.flip(np.cumsum(np.flip(a, axis), axis), axis)


def test_backward_dda_is_a_reverse_cumsum():
    # dda_t = sum_{s >= t} (dy_s . (y_s - D x_s) - x_s . (dx_s - D dy_s)) per
    # head, plus <dfinal, final> at the last step: the gradient of one decay
    # counts every (write before t, read at or after t) pair once
    inp, dy, df = _bwd_inputs(91, T=15, H=3, R=2)
    got = _bwd(inp, dy, df)
    y, f = oracle.ssd_oracle(inp.x, inp.da, inp.B, inp.C, inp.D, inp.init_state, inp.theta)
    x, dyv, D = forms.f64(inp.x), forms.f64(dy), forms.f64(inp.D)
    Dx = D[None, None, None, :, None]
    A = np.einsum("btrhp,btrhp->bth", dyv, y - Dx * x)
    Bc = np.einsum("btrhp,btrhp->bth", x, got["dx"] - Dx * dyv)
    A[:, -1] += np.einsum("bhpn,bhpn->bh", forms.f64(df), f)
    assert relerr(got["dda"], _reverse_cumsum(A - Bc)) < 1e-11


def test_backward_dtheta_is_a_reverse_cumsum():
    # dtheta_t,k = sum_{s >= t} of the pair cross products (dC_2k C_2k+1 -
    # dC_2k+1 C_2k) + (dB_2k B_2k+1 - dB_2k+1 B_2k) over ranks, plus the
    # final state's (dfinal_2k+1 h_2k - dfinal_2k h_2k+1) at the last step;
    # one head per group, so dB and dC are per head
    inp, dy, df = _bwd_inputs(92, T=11, H=2, G=2, R=2, N=6)
    got = _bwd(inp, dy, df)
    _, f = oracle.ssd_oracle(inp.x, inp.da, inp.B, inp.C, inp.D, inp.init_state, inp.theta)
    Bv, Cv = forms.f64(inp.B), forms.f64(inp.C)
    dB, dC = got["dB"], got["dC"]
    cross = lambda d, v: d[..., 0::2] * v[..., 1::2] - d[..., 1::2] * v[..., 0::2]
    Th = (cross(dC, Cv) + cross(dB, Bv)).sum(axis=2)                   # [b,T,G=H,N/2]
    dfv = forms.f64(df)
    Th[:, -1] += (dfv[..., 1::2] * f[..., 0::2] - dfv[..., 0::2] * f[..., 1::2]).sum(axis=2)
    assert relerr(got["dtheta"], _reverse_cumsum(Th)) < 1e-11


BWD_MUTANTS = {
    "bwd_turn_not_transposed": [("G[p * N + 2 * k] = co * g0 + si * g1;", "G[p * N + 2 * k] = co * g0 - si * g1;"),
                                ("G[p * N + 2 * k + 1] = -si * g0 + co * g1;", "G[p * N + 2 * k + 1] = si * g0 + co * g1;")],
    "bwd_dda_no_decay": [("dda[row] = at * acc;", "dda[row] = acc;")],
    "bwd_dC_previous_state": [("dC[crow + n] += dyv * sc[p * N + n];", "dC[crow + n] += dyv * sp[p * N + n];")],
    "bwd_dtheta_sign": [("dth[row * (N / 2) + k] = at * tk;", "dth[row * (N / 2) + k] = -at * tk;")],
    "bwd_dx_no_skip": [("dx[xrow + p] = acc + dh * dyv;", "dx[xrow + p] = acc;")],
    "bwd_read_before_write": [("G[p * N + n] += dyv * load_elem(pr->C, crow + n, pr->in_dtype);",
                               "G[p * N + n] += 0.0 * dyv;")],
}


def test_backward_pins_catch_planted_mistakes(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")).read()
    inp, dy, df = _bwd_inputs(93, T=9)
    ref = forms.autograd_gradients(inp.x, inp.da, inp.B, inp.C, dy, inp.D, inp.init_state,
                                   inp.theta, df)
    for name, edits in BWD_MUTANTS.items():
        mutated = src
        for old, new in edits:
            assert mutated.count(old) == 1, (name, old)
            mutated = mutated.replace(old, new)
        path = tmp_path / f"{name}.c"
        path.write_text(mutated)
        so = str(tmp_path / f"{name}.so")
        subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", so, str(path), "-lm"], check=True)
        got = _bwd(inp, dy, df, lib_path=so)
        worst = max(relerr(got[k], v) for k, v in ref.items())
        assert worst > 1e-6, name
