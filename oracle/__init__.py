"""Float64 CPU oracle for the chunked SSD scan (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path
(``chunked_ssd_scan_amd``) never imports, links or calls it, and the two share
no code.

The oracle itself is ``ssd_oracle.c``: the plain token-by-token recurrences in
double precision, of the chunked SSD scan, the Mamba-1 selective scan and the
Mamba-3 trapezoid, and the physical-frame state moments (see that file for the
definitions and the page passages they follow). This module builds it with gcc and wraps it with ctypes.
Pins that tie it to the pages and to mathematics live in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_libs = {}

GCC_FLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile ssd_oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(out):
        tmp = out + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
        os.replace(tmp, out)
    return out


def _load(path: Optional[str] = None):
    """Load the oracle library (``path`` selects another build of the same source)."""
    key = path or _LIB
    if key not in _libs:
        if path is None and (not os.path.exists(_LIB)
                             or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(key)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.ssd_oracle_f64.argtypes = [i64] * 7 + [ctypes.c_int] + [vp] * 7 + [vp, i64, vp, vp, ctypes.c_int]
        lib.ssd_oracle_f64.restype = ctypes.c_int
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        lib.selective_scan_f64.argtypes = [i64] * 4 + [vp] * 7 + [i64, vp, ctypes.c_int]
        lib.selective_scan_f64.restype = ctypes.c_int
        lib.trapezoid_f64.argtypes = [i64] * 7 + [ctypes.c_int] + [vp] * 10 + [vp, i64, vp, vp, ctypes.c_int]
        lib.trapezoid_f64.restype = ctypes.c_int
        lib.state_moments_f64.argtypes = ([i64] * 7 + [ctypes.c_int] + [vp] * 9 + [i64]
                                          + [vp, i64, vp, vp, ctypes.c_int])
        lib.state_moments_f64.restype = ctypes.c_int
        lib.ssd_backward_f64.argtypes = [i64] * 7 + [ctypes.c_int] + [vp] * 16 + [ctypes.c_int]
        lib.ssd_backward_f64.restype = ctypes.c_int
        _libs[key] = lib
    return _libs[key]


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous()
    return t.data_ptr()


def ssd_oracle(x: torch.Tensor, da: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
               D: Optional[torch.Tensor] = None, init_state: Optional[torch.Tensor] = None,
               theta: Optional[torch.Tensor] = None,
               bh: Optional[Sequence[int]] = None, want_y: bool = True,
               nthreads: int = 0, lib_path: Optional[str] = None):
    """Float64 oracle on CPU tensors.

    Shapes: x [b,T,R,H,P], da [b,T,H], B/C [b,T,R,G,N] (fp32 or bf16; the
    tests may pass float64 for all three),
    D [H], init_state [b,H,P,N], theta [b,T,H,N/2] (fp32).

    With ``bh=None`` returns (y [b,T,R,H,P], final [b,H,P,N]) as float64
    numpy arrays. With a list of slice indices bh = b*H + h it returns
    (y_sel [n,T,R,P], final_sel [n,P,N]) for just those slices.
    ``want_y=False`` skips storing y (y is returned as None).
    ``lib_path`` runs another build of the oracle source (the tests use it to
    check that planted mistakes are caught by the pins).
    """
    lib = _load(lib_path)
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    assert da.shape == (b, T, H)
    assert B.shape == C.shape == (b, T, R, G, N)
    if x.dtype == torch.bfloat16:
        dt = 1
    elif x.dtype == torch.float32:
        dt = 0
    elif x.dtype == torch.float64:
        dt = 2
    else:
        raise TypeError(f"unsupported input dtype {x.dtype}")
    assert B.dtype == x.dtype and C.dtype == x.dtype
    for t in (da, D, init_state, theta):
        assert t is None or t.dtype == torch.float32
    cont = lambda t: None if t is None else t.detach().cpu().contiguous()
    x, da, B, C, D, init_state, theta = map(cont, (x, da, B, C, D, init_state, theta))

    if bh is None:
        n = b * H
        bh_arr = None
    else:
        bh_arr = np.ascontiguousarray(np.asarray(bh, dtype=np.int64))
        n = int(bh_arr.size)
    y_sel = np.empty((n, T, R, P), dtype=np.float64) if want_y else None
    fin = np.empty((n, P, N), dtype=np.float64)
    rc = lib.ssd_oracle_f64(
        b, T, H, P, N, G, R, dt,
        _ptr(x), _ptr(da), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), _ptr(theta),
        None if bh_arr is None else bh_arr.ctypes.data, n,
        None if y_sel is None else y_sel.ctypes.data, fin.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_f64 failed with code {rc}")
    if bh is not None:
        return y_sel, fin
    y = None
    if want_y:
        y = y_sel.reshape(b, H, T, R, P).transpose(0, 2, 3, 1, 4).copy()
    return y, fin.reshape(b, H, P, N)


def ssd_oracle_inputs(inp, bh=None, want_y=True, nthreads=0):
    """Convenience wrapper taking an ``ssd_inputs.Inputs`` bundle."""
    return ssd_oracle(inp.x, inp.da, inp.B, inp.C, inp.D, inp.init_state, inp.theta,
                      bh=bh, want_y=want_y, nthreads=nthreads)


def time_oracle(inp, bh: Sequence[int], nthreads: int = 0):
    """Wall time of the oracle on the given slices (steady clock)."""
    t0 = time.perf_counter()
    ssd_oracle_inputs(inp, bh=bh, want_y=True, nthreads=nthreads)
    return time.perf_counter() - t0


def selective_scan(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                   C: torch.Tensor, skip: torch.Tensor, bd: Optional[Sequence[int]] = None,
                   nthreads: int = 0, lib_path: Optional[str] = None):
    """Float64 Mamba-1 selective scan ("SSM Selective Scan", problem statement).

    u, delta [b,T,D]; A [D,N]; B, C [b,T,N]; skip [D]; all fp32 CPU tensors.
    Returns y [b,T,D] as float64, or with ``bd`` (channel indices b*D + d)
    y_sel [n,T] for just those channels.
    """
    lib = _load(lib_path)
    b, T, Dm = u.shape
    N = A.shape[1]
    assert delta.shape == (b, T, Dm) and A.shape == (Dm, N) and skip.shape == (Dm,)
    assert B.shape == C.shape == (b, T, N)
    for t in (u, delta, A, B, C, skip):
        assert t.dtype == torch.float32
    cont = lambda t: t.detach().cpu().contiguous()
    u, delta, A, B, C, skip = map(cont, (u, delta, A, B, C, skip))
    if bd is None:
        bd_arr, n = None, b * Dm
        y = np.empty((b, T, Dm), dtype=np.float64)
    else:
        bd_arr = np.ascontiguousarray(np.asarray(bd, dtype=np.int64))
        n = int(bd_arr.size)
        y = np.empty((n, T), dtype=np.float64)
    rc = lib.selective_scan_f64(b, T, Dm, N, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(skip),
                                None if bd_arr is None else bd_arr.ctypes.data, n, y.ctypes.data,
                                int(nthreads))
    if rc != 0:
        raise RuntimeError(f"selective_scan_f64 failed with code {rc}")
    return y


def trapezoid(x: torch.Tensor, da: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
              beta: torch.Tensor, gamma: torch.Tensor, prev_x: Optional[torch.Tensor] = None,
              prev_B: Optional[torch.Tensor] = None, init_state: Optional[torch.Tensor] = None,
              theta: Optional[torch.Tensor] = None, bh: Optional[Sequence[int]] = None,
              nthreads: int = 0, lib_path: Optional[str] = None):
    """Float64 Mamba-3 trapezoid recurrence ("mamba3/scan.py", docstring and
    scan_forward; "mamba3/moments.rs", build_moments_input).

    Shapes as ssd_oracle (no D), plus beta, gamma [b,T,H] fp32, prev_x
    [b,R,H,P] and prev_B [b,R,G,N] (x's dtype; both or neither). Returns
    (y [b,T,R,H,P], final [b,H,P,N]) as float64, or with ``bh`` the selected
    slices (y_sel [n,T,R,P], final_sel [n,P,N]).
    """
    lib = _load(lib_path)
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    assert da.shape == beta.shape == gamma.shape == (b, T, H)
    assert B.shape == C.shape == (b, T, R, G, N)
    assert (prev_x is None) == (prev_B is None)
    if prev_x is not None:
        assert prev_x.shape == (b, R, H, P) and prev_B.shape == (b, R, G, N)
        assert prev_x.dtype == x.dtype and prev_B.dtype == x.dtype
    dt = {torch.bfloat16: 1, torch.float32: 0, torch.float64: 2}[x.dtype]
    assert B.dtype == x.dtype and C.dtype == x.dtype
    for t in (da, beta, gamma, init_state, theta):
        assert t is None or t.dtype == torch.float32
    cont = lambda t: None if t is None else t.detach().cpu().contiguous()
    x, da, B, C, beta, gamma, prev_x, prev_B, init_state, theta = map(
        cont, (x, da, B, C, beta, gamma, prev_x, prev_B, init_state, theta))
    if bh is None:
        n, bh_arr = b * H, None
    else:
        bh_arr = np.ascontiguousarray(np.asarray(bh, dtype=np.int64))
        n = int(bh_arr.size)
    y_sel = np.empty((n, T, R, P), dtype=np.float64)
    fin = np.empty((n, P, N), dtype=np.float64)
    rc = lib.trapezoid_f64(
        b, T, H, P, N, G, R, dt, _ptr(x), _ptr(da), _ptr(B), _ptr(C), _ptr(beta), _ptr(gamma),
        _ptr(prev_x), _ptr(prev_B), _ptr(init_state), _ptr(theta),
        None if bh_arr is None else bh_arr.ctypes.data, n, y_sel.ctypes.data, fin.ctypes.data,
        int(nthreads))
    if rc != 0:
        raise RuntimeError(f"trapezoid_f64 failed with code {rc}")
    if bh is not None:
        return y_sel, fin
    return y_sel.reshape(b, H, T, R, P).transpose(0, 2, 3, 1, 4).copy(), fin.reshape(b, H, P, N)


def state_moments(x: torch.Tensor, da: torch.Tensor, B: torch.Tensor,
                  beta: Optional[torch.Tensor] = None, gamma: Optional[torch.Tensor] = None,
                  prev_x: Optional[torch.Tensor] = None, prev_B: Optional[torch.Tensor] = None,
                  init_state: Optional[torch.Tensor] = None, theta: Optional[torch.Tensor] = None,
                  valid_len: Optional[int] = None, bh: Optional[Sequence[int]] = None,
                  nthreads: int = 0, lib_path: Optional[str] = None):
    """Float64 physical-frame state moments (burn-mamba "mamba3/moments.rs",
    module documentation and state_moments_phys).

    Shapes as ``trapezoid`` (without C); beta and gamma both None for the
    single-write recurrence. valid_len defaults to T. Returns (m2 [b,H,N,N],
    m1 [b,H,N]) as float64, or with ``bh`` the selected slices (m2 [n,N,N],
    m1 [n,N]).
    """
    lib = _load(lib_path)
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    assert da.shape == (b, T, H) and B.shape[:3] == (b, T, R)
    assert (beta is None) == (gamma is None)
    if beta is None:
        prev_x = prev_B = None
    else:
        assert beta.shape == gamma.shape == (b, T, H)
    assert (prev_x is None) == (prev_B is None)
    dt = {torch.bfloat16: 1, torch.float32: 0, torch.float64: 2}[x.dtype]
    assert B.dtype == x.dtype
    vl = T if valid_len is None else int(valid_len)
    cont = lambda t: None if t is None else t.detach().cpu().contiguous()
    x, da, B, beta, gamma, prev_x, prev_B, init_state, theta = map(
        cont, (x, da, B, beta, gamma, prev_x, prev_B, init_state, theta))
    if bh is None:
        n, bh_arr = b * H, None
    else:
        bh_arr = np.ascontiguousarray(np.asarray(bh, dtype=np.int64))
        n = int(bh_arr.size)
    m2 = np.empty((n, N, N), dtype=np.float64)
    m1 = np.empty((n, N), dtype=np.float64)
    rc = lib.state_moments_f64(
        b, T, H, P, N, G, R, dt, _ptr(x), _ptr(da), _ptr(B), _ptr(beta), _ptr(gamma),
        _ptr(prev_x), _ptr(prev_B), _ptr(init_state), _ptr(theta), vl,
        None if bh_arr is None else bh_arr.ctypes.data, n, m2.ctypes.data, m1.ctypes.data,
        int(nthreads))
    if rc != 0:
        raise RuntimeError(f"state_moments_f64 failed with code {rc}")
    if bh is not None:
        return m2, m1
    return m2.reshape(b, H, N, N), m1.reshape(b, H, N)


def ssd_backward(x: torch.Tensor, da: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                 dy: torch.Tensor, D: Optional[torch.Tensor] = None,
                 init_state: Optional[torch.Tensor] = None, theta: Optional[torch.Tensor] = None,
                 dfinal: Optional[torch.Tensor] = None, nthreads: int = 0,
                 lib_path: Optional[str] = None) -> dict:
    """Float64 gradients of the scan (reverse mode over the token recurrence).

    Inputs as ``ssd_oracle`` plus dy [b,T,R,H,P] and dfinal [b,H,P,N] (fp32;
    dfinal None means zero). Returns a dict of float64 arrays: dx, dda, dB,
    dC, dinit, and dtheta / dD when theta / D are given.
    """
    lib = _load(lib_path)
    b, T, R, H, P = x.shape
    G, N = B.shape[3], B.shape[4]
    assert da.shape == (b, T, H) and B.shape == C.shape == (b, T, R, G, N)
    assert dy.shape == (b, T, R, H, P) and dy.dtype == torch.float32
    assert dfinal is None or (dfinal.shape == (b, H, P, N) and dfinal.dtype == torch.float32)
    dt = {torch.bfloat16: 1, torch.float32: 0, torch.float64: 2}[x.dtype]
    assert B.dtype == x.dtype and C.dtype == x.dtype
    cont = lambda t: None if t is None else t.detach().cpu().contiguous()
    x, da, B, C, D, init_state, theta, dy, dfinal = map(
        cont, (x, da, B, C, D, init_state, theta, dy, dfinal))
    out = {"dx": np.empty((b, T, R, H, P)), "dda": np.empty((b, T, H)),
           "dB": np.empty((b, T, R, G, N)), "dC": np.empty((b, T, R, G, N)),
           "dinit": np.empty((b, H, P, N))}
    out["dtheta"] = np.empty((b, T, H, N // 2)) if theta is not None else None
    out["dD"] = np.empty((H,)) if D is not None else None
    pa = lambda a: None if a is None else a.ctypes.data
    rc = lib.ssd_backward_f64(b, T, H, P, N, G, R, dt, _ptr(x), _ptr(da), _ptr(B), _ptr(C), _ptr(D),
                              _ptr(init_state), _ptr(theta), _ptr(dy), _ptr(dfinal),
                              pa(out["dx"]), pa(out["dda"]), pa(out["dB"]), pa(out["dC"]),
                              pa(out["dtheta"]), pa(out["dinit"]), pa(out["dD"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_backward_f64 failed with code {rc}")
    return {k: v for k, v in out.items() if v is not None}
