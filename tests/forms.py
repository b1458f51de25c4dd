"""Independent float64 formulations used to pin the oracle (CPU, tests only).

None of these retypes the oracle's token recurrence; each one computes the same
quantity another way, as the pages describe it:

* ``quadratic_form``: the whole sequence as one chunk. y = (L o C B^T) x plus
  the initial-state term exp(cumsum(da)) * (C h0), with L built from stable
  segment sums and masked before exp (burn-mamba "modules/misc/segsum.rs",
  segsum; "mamba3/ssd/serial.rs", k5_ssd_chunk_scan: Y_diag and Y_off). The
  rotation is folded in by cumulative angles, B~ = R(-Phi) B and C~ = R(-Phi) C
  ("mamba3/scan.py", docstring "THE TRICK" and cumulative_angles/rotate_by).
* ``chunked_form``: the K1..K5 chunk algorithm with a serial inter-chunk loop
  ("mamba3/ssd/serial.rs": k1_ssd_chunk_cumsum, k2_ssd_bmm, k3_ssd_chunk_state,
  k4_ssd_state_passing, k5_ssd_chunk_scan), zero-padding a ragged tail
  ("mamba3/moments.rs", build_moments_input: zero-pad to a chunk multiple).
* ``product_form``: brute force with explicit products of the per-step decays
  and explicit composed rotations R(Phi_t - Phi_s); for tiny T only.
* ``mamba1_scan``: the LeetGPU "SSM Selective Scan" statement (Abar, Bbar, h, y
  with skip), per channel d and state index n, written from that page.
* ``trapezoid_frame_form``: the Mamba-3 trapezoid as "mamba3/scan.py"'s
  scan_forward computes it: both writes turned into the cumulative frame
  separately (this step's by R(-Phi_t), the previous step's by R(-Phi_{t-1})),
  a plain first-order scan g_t = alpha_t g_{t-1} + w_t, then h_t = R(Phi_t) g_t.
"""
from __future__ import annotations

import numpy as np


def f64(t):
    """torch tensor / array -> float64 numpy (exact for fp32 and bf16)."""
    if t is None:
        return None
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu", dtype=torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def rotate_pairs(v, ang):
    """Turn pairs (2k, 2k+1) of the last axis of v by angle ang[..., k].

    even' = cos*a - sin*b, odd' = sin*a + cos*b (rotate_by in "mamba3/scan.py").
    """
    a, b = v[..., 0::2], v[..., 1::2]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(v)
    out[..., 0::2] = c * a - s * b
    out[..., 1::2] = s * a + c * b
    return out


def _groups(H, G):
    return np.arange(H) // (H // G)


def quadratic_form(x, da, B, C, D=None, h0=None, theta=None):
    """One-chunk quadratic (segsum) form. Returns y [b,T,R,H,P], final [b,H,P,N]."""
    x, da, B, C, D, h0, theta = map(f64, (x, da, B, C, D, h0, theta))
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    grp = _groups(H, G)
    y = np.zeros((b, T, R, H, P))
    fin = np.zeros((b, H, P, N))
    tf = np.repeat(np.arange(T), R)                      # time step of fused row f = t*R + r
    for bi in range(b):
        for h in range(H):
            g = grp[h]
            cum = np.cumsum(da[bi, :, h])                # inclusive prefix (K1)
            Bh, Ch = B[bi, :, :, g, :], C[bi, :, :, g, :]  # [T,R,N]
            if theta is not None:
                Phi = np.cumsum(theta[bi, :, h, :], axis=0)  # [T,N/2]
                Bh = rotate_pairs(Bh, -Phi[:, None, :])
                Ch = rotate_pairs(Ch, -Phi[:, None, :])
            Bf = Bh.reshape(T * R, N)
            Cf = Ch.reshape(T * R, N)
            Xf = x[bi, :, :, h, :].reshape(T * R, P)
            seg = cum[tf][:, None] - cum[tf][None, :]
            causal = tf[:, None] >= tf[None, :]
            Lm = np.exp(np.where(causal, seg, -np.inf))  # mask before exp
            Yd = (Lm * (Cf @ Bf.T)) @ Xf
            Yo = np.zeros_like(Yd)
            if h0 is not None:
                Yo = np.exp(cum[tf])[:, None] * (Cf @ h0[bi, h].T)
            Yf = Yd + Yo
            if D is not None:
                Yf = Yf + D[h] * Xf
            y[bi, :, :, h, :] = Yf.reshape(T, R, P)
            w = np.exp(cum[-1] - cum[tf])                # decay of each write to the end
            g_end = (Xf * w[:, None]).T @ Bf             # [P,N]
            if h0 is not None:
                g_end = g_end + np.exp(cum[-1]) * h0[bi, h]
            if theta is not None:
                g_end = rotate_pairs(g_end, np.broadcast_to(Phi[-1], (P, N // 2)))
            fin[bi, h] = g_end
    return y, fin


def chunked_form(x, da, B, C, D=None, h0=None, theta=None, chunk_len=16):
    """K1..K5 with a serial state-passing loop, zero-padded ragged tail."""
    x, da, B, C, D, h0, theta = map(f64, (x, da, B, C, D, h0, theta))
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    grp = _groups(H, G)
    l = int(chunk_len)
    nc = -(-T // l)
    Tp = nc * l
    pad = Tp - T
    y = np.zeros((b, T, R, H, P))
    fin = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = grp[h]
            Bh, Ch = B[bi, :, :, g, :], C[bi, :, :, g, :]
            if theta is not None:
                Phi = np.cumsum(theta[bi, :, h, :], axis=0)
                Bh = rotate_pairs(Bh, -Phi[:, None, :])
                Ch = rotate_pairs(Ch, -Phi[:, None, :])
            zp = lambda a: np.concatenate([a, np.zeros((pad,) + a.shape[1:])], 0)
            Xc = zp(x[bi, :, :, h, :]).reshape(nc, l * R, P)
            Bc = zp(Bh).reshape(nc, l * R, N)
            Cc = zp(Ch).reshape(nc, l * R, N)
            dac = zp(da[bi, :, h]).reshape(nc, l)
            # K1: intra-chunk inclusive cumsum and chunk totals
            cum = np.cumsum(dac, axis=1)                 # [nc,l]
            cum_end = cum[:, -1]
            cumf = np.repeat(cum, R, axis=1)             # fused rows
            # K2: CB on fused rows
            CB = Cc @ np.transpose(Bc, (0, 2, 1))        # [nc,L,L]
            # K3: chunk states from a zero start
            dec = np.exp(cum_end[:, None] - cumf)        # [nc,L]
            s = np.transpose(Xc * dec[:, :, None], (0, 2, 1)) @ Bc   # [nc,P,N]
            # K4: serial state passing
            st = np.zeros((P, N)) if h0 is None else h0[bi, h].copy()
            h_in = []
            for c in range(nc):
                h_in.append(st.copy())
                st = np.exp(cum_end[c]) * st + s[c]
            # K5: chunk scan, Y_off + Y_diag (mask i//R >= j//R before exp)
            tt = np.arange(l * R) // R
            causal = tt[:, None] >= tt[None, :]
            Yc = np.zeros((nc, l * R, P))
            for c in range(nc):
                Lm = np.exp(np.where(causal, cumf[c][:, None] - cumf[c][None, :], -np.inf))
                Yc[c] = (Lm * CB[c]) @ Xc[c]
                Yc[c] += np.exp(cumf[c])[:, None] * (Cc[c] @ h_in[c].T)
            Yf = Yc.reshape(Tp, R, P)[:T]
            if D is not None:
                Yf = Yf + D[h] * x[bi, :, :, h, :]
            y[bi, :, :, h, :] = Yf
            if theta is not None:
                st = rotate_pairs(st, np.broadcast_to(Phi[-1], (P, N // 2)))
            fin[bi, h] = st
    return y, fin


def product_form(x, da, B, C, D=None, h0=None, theta=None):
    """Brute force: explicit decay products and composed rotations (tiny T)."""
    x, da, B, C, D, h0, theta = map(f64, (x, da, B, C, D, h0, theta))
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    grp = _groups(H, G)
    alpha = np.exp(da)                                   # per-step decay factors
    y = np.zeros((b, T, R, H, P))
    fin = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = grp[h]
            Phi = np.zeros((T, N // 2)) if theta is None else np.cumsum(theta[bi, :, h, :], axis=0)
            for t in range(T):
                st = np.zeros((P, N))
                if h0 is not None:
                    prod = np.prod(alpha[bi, 0:t + 1, h])
                    st += prod * rotate_pairs(h0[bi, h], np.broadcast_to(Phi[t], (P, N // 2)))
                for s in range(t + 1):
                    prod = np.prod(alpha[bi, s + 1:t + 1, h])    # empty product = 1
                    W = x[bi, s, :, h, :].T @ B[bi, s, :, g, :]  # sum_r x_r (outer) B_r
                    ang = np.broadcast_to(Phi[t] - Phi[s], (P, N // 2))
                    st += prod * rotate_pairs(W, ang)
                for r in range(R):
                    y[bi, t, r, h] = st @ C[bi, t, r, g, :]
                    if D is not None:
                        y[bi, t, r, h] += D[h] * x[bi, t, r, h, :]
                if t == T - 1:
                    fin[bi, h] = st
    return y, fin


def mamba1_scan(u, delta, A, Bm, Cm, skip):
    """Selective scan with a per-(channel, state) decay, as the LeetGPU page states.

    u, delta: [b,T,D]; A: [D,N]; Bm, Cm: [b,T,N]; skip: [D]. Zero initial state.
    """
    u, delta, A, Bm, Cm, skip = map(f64, (u, delta, A, Bm, Cm, skip))
    b, T, Dm = u.shape
    N = A.shape[1]
    y = np.zeros((b, T, Dm))
    for bi in range(b):
        for d in range(Dm):
            h = np.zeros(N)
            for t in range(T):
                Abar = np.exp(delta[bi, t, d] * A[d])
                Bbar = delta[bi, t, d] * Bm[bi, t]
                h = Abar * h + Bbar * u[bi, t, d]
                y[bi, t, d] = Cm[bi, t] @ h + skip[d] * u[bi, t, d]
    return y


def trapezoid_frame_form(x, da, B, C, beta, gamma, prev_x=None, prev_B=None, h0=None,
                         theta=None):
    """y [b,T,R,H,P], final [b,H,P,N] via the cumulative-angle frame.

    The state is held as [N, P] per (b, h) as in scan.py (S = B x^T), so the
    rotation acts on its first axis.
    """
    x, da, B, C, beta, gamma = map(f64, (x, da, B, C, beta, gamma))
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    gi = _groups(H, G)
    Bh, Ch = B[:, :, :, gi, :], C[:, :, :, gi, :]                 # [b,T,R,H,N]
    S = np.einsum("btrhn,btrhp->bthnp", Bh, x)                     # this step's write
    if prev_x is not None:
        Sm1 = np.einsum("brhn,brhp->bhnp", f64(prev_B)[:, :, gi, :], f64(prev_x))
    else:
        Sm1 = np.zeros((b, H, N, P))
    Sprev = np.concatenate([Sm1[:, None], S[:, :-1]], axis=1)
    if theta is not None:
        Phi = np.cumsum(f64(theta), axis=1)                         # [b,T,H,N/2]
    else:
        Phi = np.zeros((b, T, H, N // 2))
    Phi_prev = np.concatenate([np.zeros_like(Phi[:, :1]), Phi[:, :-1]], axis=1)
    rot_n = lambda v, ang: np.swapaxes(rotate_pairs(np.swapaxes(v, -1, -2), ang[..., None, :]), -1, -2)
    w = (gamma[..., None, None] * rot_n(S, -Phi) + beta[..., None, None] * rot_n(Sprev, -Phi_prev))
    g = np.zeros((b, H, N, P)) if h0 is None else np.swapaxes(f64(h0), -1, -2).copy()
    alpha = np.exp(da)
    y = np.empty((b, T, R, H, P))
    for t in range(T):
        g = alpha[:, t, :, None, None] * g + w[:, t]
        h = rot_n(g, Phi[:, t])
        y[:, t] = np.einsum("brhn,bhnp->brhp", Ch[:, t], h)
    return y, np.swapaxes(h, -1, -2)


def trapezoid_frame_states(x, da, B, beta=None, gamma=None, prev_x=None, prev_B=None, h0=None,
                           theta=None):
    """Every physical state h_t [b,T,H,P,N] of the trapezoid (or, with beta
    and gamma None, the single-write) recurrence, via the cumulative-angle
    frame as ``trapezoid_frame_form`` builds it: the writes turned into the
    frame, a first-order scan g_t, then h_t = R(Phi_t) g_t ("mamba3/scan.py",
    scan_forward; "mamba3/moments.rs", module documentation: the cache-frame
    states de-rotated to the physical frame, step 3)."""
    x, da, B = map(f64, (x, da, B))
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    gi = _groups(H, G)
    Bh = B[:, :, :, gi, :]
    S = np.einsum("btrhn,btrhp->bthnp", Bh, x)
    if beta is None:
        beta, gamma = np.zeros((b, T, H)), np.ones((b, T, H))
        prev_x = prev_B = None
    else:
        beta, gamma = f64(beta), f64(gamma)
    if prev_x is not None:
        Sm1 = np.einsum("brhn,brhp->bhnp", f64(prev_B)[:, :, gi, :], f64(prev_x))
    else:
        Sm1 = np.zeros((b, H, N, P))
    Sprev = np.concatenate([Sm1[:, None], S[:, :-1]], axis=1)
    Phi = np.cumsum(f64(theta), axis=1) if theta is not None else np.zeros((b, T, H, N // 2))
    Phi_prev = np.concatenate([np.zeros_like(Phi[:, :1]), Phi[:, :-1]], axis=1)
    rot_n = lambda v, ang: np.swapaxes(rotate_pairs(np.swapaxes(v, -1, -2), ang[..., None, :]), -1, -2)
    w = gamma[..., None, None] * rot_n(S, -Phi) + beta[..., None, None] * rot_n(Sprev, -Phi_prev)
    g = np.zeros((b, H, N, P)) if h0 is None else np.swapaxes(f64(h0), -1, -2).copy()
    alpha = np.exp(da)
    out = np.empty((b, T, H, P, N))
    for t in range(T):
        g = alpha[:, t, :, None, None] * g + w[:, t]
        out[:, t] = np.swapaxes(rot_n(g, Phi[:, t]), -1, -2)
    return out


def autograd_gradients(x, da, B, C, dy, D=None, h0=None, theta=None, dfinal=None):
    """Float64 torch autograd of the token recurrence, written here as plain
    tensor ops ("mamba3/scan.py", verify(): the backward checked against the
    recurrence at float64). Loss = <dy, y> + <dfinal, final>, so the
    gradients are the vector-Jacobian products the oracle's backward gives.
    Returns a dict of float64 numpy arrays (dx, dda, dB, dC, dinit, dtheta,
    dD as present)."""
    import torch

    t64 = lambda a: None if a is None else torch.tensor(f64(a), dtype=torch.float64,
                                                       requires_grad=True)
    x, da, B, C = map(t64, (x, da, B, C))
    D, h0, theta = t64(D), t64(h0), t64(theta)
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    gi = torch.as_tensor(_groups(H, G))
    S = (h0 if h0 is not None else torch.zeros(b, H, P, N, dtype=torch.float64))
    ys = []
    for t in range(T):
        if theta is not None:
            c, s = torch.cos(theta[:, t]), torch.sin(theta[:, t])      # [b,H,N/2]
            e, o = S[..., 0::2], S[..., 1::2]
            S = torch.stack((c[:, :, None] * e - s[:, :, None] * o,
                             s[:, :, None] * e + c[:, :, None] * o), dim=-1).flatten(-2)
        S = torch.exp(da[:, t])[:, :, None, None] * S
        Bh, Ch = B[:, t][:, :, gi], C[:, t][:, :, gi]                  # [b,R,H,N]
        S = S + torch.einsum("brhp,brhn->bhpn", x[:, t], Bh)
        yt = torch.einsum("brhn,bhpn->brhp", Ch, S)
        if D is not None:
            yt = yt + D[None, None, :, None] * x[:, t]
        ys.append(yt)
    y = torch.stack(ys, dim=1)
    loss = (y * torch.tensor(f64(dy))).sum()
    if dfinal is not None:
        loss = loss + (S * torch.tensor(f64(dfinal))).sum()
    loss.backward()
    out = {"dx": x.grad.numpy(), "dda": da.grad.numpy(), "dB": B.grad.numpy(), "dC": C.grad.numpy(),
           "dinit": h0.grad.numpy() if h0 is not None else None}
    if theta is not None:
        out["dtheta"] = theta.grad.numpy()
    if D is not None:
        out["dD"] = D.grad.numpy()
    return {k: v for k, v in out.items() if v is not None}
