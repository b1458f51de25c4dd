"""Python binding of the chunked SSD scan C ABI (``include/ssd_scan.h``).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libssd_scan.so``. PyTorch is used for device memory and the current stream.
Importing works without a GPU; calling the scan needs the built library and
a gfx950 device, and fails loudly otherwise (there is no CPU fallback).

C entry points, mirrored here under the same names:
  ssd_forward, ssd_forward_ex, ssd_workspace_bytes, ssd_selective_scan,
  ssd_selective_scan_ex, ssd_trapezoid_forward, ssd_forward_noalloc,
  ssd_state_moments, ssd_status_str
plus ``forward(...)``, ``selective_scan(...)`` and ``trapezoid(...)``,
tensor-level conveniences over ssd_forward_ex, ssd_selective_scan_ex and
ssd_trapezoid_forward.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd_scan.so")

SSD_F32, SSD_BF16 = 0, 1
SSD_OK = 0
SSD_ERR_NULL_ARG = 1
SSD_ERR_BAD_SHAPE = 2
SSD_ERR_UNSUPPORTED = 3
SSD_ERR_ALIAS = 4
SSD_ERR_HIP = 5
SSD_ERR_WORKSPACE = 6
SSD_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTED = ("ssd_forward", "ssd_forward_ex", "ssd_workspace_bytes", "ssd_selective_scan",
            "ssd_selective_scan_ex", "ssd_trapezoid_forward", "ssd_forward_noalloc",
            "ssd_state_moments", "ssd_backward", "ssd_status_str")


class SsdDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("in_dtype", ctypes.c_int32)]


class SsdLaunchOpts(ctypes.Structure):
    _fields_ = [("segments", ctypes.c_int32), ("block_slices", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2), ("walk_events", ctypes.c_void_p * 2)]


class SsdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {ssd_status_str(status)} ({status})")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libssd_scan.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library not built: {path} is missing "
                "(run `python -c 'import __graft_entry__ as g; g.build()'`)")
        lib = ctypes.CDLL(path)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        common = [ctypes.POINTER(SsdDims), vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp]
        lib.ssd_forward.argtypes = common + [vp]
        lib.ssd_forward.restype = ctypes.c_int
        lib.ssd_forward_ex.argtypes = common + [ctypes.POINTER(SsdLaunchOpts), vp]
        lib.ssd_forward_ex.restype = ctypes.c_int
        lib.ssd_forward_noalloc.argtypes = common + [ctypes.POINTER(SsdLaunchOpts), vp]
        lib.ssd_forward_noalloc.restype = ctypes.c_int
        lib.ssd_workspace_bytes.argtypes = [ctypes.POINTER(SsdDims), i64, i64]
        lib.ssd_workspace_bytes.restype = ctypes.c_size_t
        lib.ssd_selective_scan.argtypes = [vp] * 7 + [i64] * 4 + [vp]
        lib.ssd_selective_scan.restype = ctypes.c_int
        lib.ssd_selective_scan_ex.argtypes = [vp] * 7 + [i64] * 4 + [ctypes.POINTER(SsdLaunchOpts), vp]
        lib.ssd_selective_scan_ex.restype = ctypes.c_int
        lib.ssd_trapezoid_forward.argtypes = ([ctypes.POINTER(SsdDims)] + [vp] * 9 + [i64, i64]
                                              + [vp] * 3 + [ctypes.POINTER(SsdLaunchOpts), vp])
        lib.ssd_trapezoid_forward.restype = ctypes.c_int
        lib.ssd_state_moments.argtypes = ([ctypes.POINTER(SsdDims)] + [vp] * 8 + [i64, vp, i64]
                                          + [vp] * 3)
        lib.ssd_state_moments.restype = ctypes.c_int
        lib.ssd_backward.argtypes = [ctypes.POINTER(SsdDims)] + [vp] * 6 + [i64] + [vp] * 11
        lib.ssd_backward.restype = ctypes.c_int
        lib.ssd_status_str.argtypes = [ctypes.c_int32]
        lib.ssd_status_str.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def make_dims(batch, seqlen, nheads, headdim, dstate, ngroups, in_dtype) -> SsdDims:
    return SsdDims(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate),
                   int(ngroups), int(in_dtype))


# ---- raw C-ABI mirrors (pointers are ints or None) -------------------------

def ssd_forward(dims: Optional[SsdDims], x, da, B, C, D, init_state, chunk_len, R,
                theta, y, final_state, stream) -> int:
    lib = load_library()
    return int(lib.ssd_forward(None if dims is None else ctypes.byref(dims), x, da, B, C, D,
                               init_state, int(chunk_len), int(R), theta, y, final_state, stream))


def ssd_forward_ex(dims: Optional[SsdDims], x, da, B, C, D, init_state, chunk_len, R,
                   theta, y, final_state, opts: Optional[SsdLaunchOpts], stream) -> int:
    lib = load_library()
    return int(lib.ssd_forward_ex(None if dims is None else ctypes.byref(dims), x, da, B, C, D,
                                  init_state, int(chunk_len), int(R), theta, y, final_state,
                                  None if opts is None else ctypes.byref(opts), stream))


def ssd_forward_noalloc(dims: Optional[SsdDims], x, da, B, C, D, init_state, chunk_len, R,
                        theta, y, final_state, opts: Optional[SsdLaunchOpts], stream) -> int:
    lib = load_library()
    return int(lib.ssd_forward_noalloc(None if dims is None else ctypes.byref(dims), x, da, B, C,
                                       D, init_state, int(chunk_len), int(R), theta, y,
                                       final_state, None if opts is None else ctypes.byref(opts),
                                       stream))


def ssd_workspace_bytes(dims: SsdDims, chunk_len: int, R: int) -> int:
    return int(load_library().ssd_workspace_bytes(ctypes.byref(dims), int(chunk_len), int(R)))


def ssd_selective_scan(u, delta, A, B, C, skip, y, batch, seq_len, d_model, d_state,
                       stream) -> int:
    lib = load_library()
    return int(lib.ssd_selective_scan(u, delta, A, B, C, skip, y, int(batch), int(seq_len),
                                      int(d_model), int(d_state), stream))


def ssd_selective_scan_ex(u, delta, A, B, C, skip, y, batch, seq_len, d_model, d_state,
                          opts: Optional[SsdLaunchOpts], stream) -> int:
    lib = load_library()
    return int(lib.ssd_selective_scan_ex(u, delta, A, B, C, skip, y, int(batch), int(seq_len),
                                         int(d_model), int(d_state),
                                         None if opts is None else ctypes.byref(opts), stream))


def ssd_trapezoid_forward(dims: Optional[SsdDims], x, da, B, C, beta, gamma, prev_x, prev_B,
                          init_state, chunk_len, R, theta, y, final_state,
                          opts: Optional[SsdLaunchOpts], stream) -> int:
    lib = load_library()
    return int(lib.ssd_trapezoid_forward(None if dims is None else ctypes.byref(dims), x, da, B, C,
                                         beta, gamma, prev_x, prev_B, init_state, int(chunk_len),
                                         int(R), theta, y, final_state,
                                         None if opts is None else ctypes.byref(opts), stream))


def ssd_state_moments(dims: Optional[SsdDims], x, da, B, beta, gamma, prev_x, prev_B,
                      init_state, R, theta, valid_len, m2, m1, stream) -> int:
    lib = load_library()
    return int(lib.ssd_state_moments(None if dims is None else ctypes.byref(dims), x, da, B, beta,
                                     gamma, prev_x, prev_B, init_state, int(R), theta,
                                     int(valid_len), m2, m1, stream))


def ssd_backward(dims: Optional[SsdDims], x, da, B, C, D, init_state, R, theta, dy, dfinal,
                 dx, dda, dB, dC, dtheta, dinit, dD, stream) -> int:
    lib = load_library()
    return int(lib.ssd_backward(None if dims is None else ctypes.byref(dims), x, da, B, C, D,
                                init_state, int(R), theta, dy, dfinal, dx, dda, dB, dC, dtheta,
                                dinit, dD, stream))


def ssd_status_str(status: int) -> str:
    return load_library().ssd_status_str(int(status)).decode()


# ---- tensor-level convenience ---------------------------------------------

def _dptr(t):
    return None if t is None else t.data_ptr()


def _event_handles(events, stream, dev):
    """hipEvent_t handles of a pair of torch.cuda.Event (or of ints, taken as handles)."""
    import torch

    handles = []
    for ev in events:
        if isinstance(ev, int):
            handles.append(ev)
            continue
        if ev.cuda_event == 0:
            # torch creates an event's HIP handle at its first record
            ev.record(torch.cuda.ExternalStream(stream, device=dev))
        handles.append(ev.cuda_event)
    return handles


def _check(name, t, shape, dtype, dev, optional=False):
    """Raise unless ``t`` is a contiguous tensor of ``shape`` and ``dtype`` on ``dev``.

    Shape and dtype are checked before the device, so that the checks can be
    exercised on any device; nothing is launched.
    """
    import torch

    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _in_dtype(x):
    import torch

    if x.dtype == torch.bfloat16:
        return SSD_BF16
    if x.dtype == torch.float32:
        return SSD_F32
    raise TypeError(f"x must be bf16 or fp32, got {x.dtype}")


def _need_device(x, what):
    if x.device.type != "cuda":
        raise ValueError(f"chunked_ssd_scan_amd.{what} needs device tensors (x is on {x.device})")


def _ssd_sizes(x, B, prev_x=None, prev_B=None):
    """(x5, B5, (b, T, R, H, P, G, N), prev_x, prev_B): rank-4 Mamba-2 layouts
    get a rank axis of 1."""
    if x.dim() not in (4, 5):
        raise ValueError(f"x must be [b,T,H,P] or [b,T,R,H,P], got {tuple(x.shape)}")
    if B.dim() != x.dim():
        raise ValueError(f"B must have x's rank ({x.dim()}), got {tuple(B.shape)}")
    if x.dim() == 4:
        x5, B5 = x.unsqueeze(2), B.unsqueeze(2)
        if prev_x is not None:
            prev_x = prev_x.unsqueeze(1)
        if prev_B is not None:
            prev_B = prev_B.unsqueeze(1)
    else:
        x5, B5 = x, B
    b, T, R, H, P = x5.shape
    G, N = B5.shape[3], B5.shape[4]
    if tuple(B5.shape[:3]) != (b, T, R):
        raise ValueError(f"B has shape {tuple(B.shape)}, which does not match x {tuple(x.shape)}")
    return (b, T, R, H, P, G, N), prev_x, prev_B


def forward(x, da, B, C, D=None, init_state=None, chunk_len: int = 256, theta=None,
            y=None, final_state=None, segments: int = 0, block_slices: int = 0,
            stream=None, walk_events=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Run the scan on device tensors; returns (y, final_state).

    x [b,T,R,H,P] (or [b,T,H,P] for R = 1), da [b,T,H], B/C [b,T,R,G,N]
    (or [b,T,G,N]); D [H], init_state [b,H,P,N], theta [b,T,H,N/2] fp32.
    y / final_state may be given (fp32, contiguous) to write in place;
    final_state may be init_state itself. ``segments``, ``block_slices`` and
    ``walk_events`` (a pair of torch.cuda.Event, or of hipEvent_t handles as
    ints, recorded around the output walk kernel) are the launch options of
    ssd_forward_ex.
    """
    import torch

    (b, T, R, H, P, G, N), _, _ = _ssd_sizes(x, B)
    in_dtype = _in_dtype(x)
    f32 = torch.float32
    dev = None if x.device.type == "cpu" else x.device
    _check("x", x, x.shape, x.dtype, dev)
    _check("B", B, B.shape, x.dtype, dev)
    _check("C", C, B.shape, x.dtype, dev)
    _check("da", da, (b, T, H), f32, dev)
    _check("D", D, (H,), f32, dev, optional=True)
    _check("init_state", init_state, (b, H, P, N), f32, dev, optional=True)
    _check("theta", theta, (b, T, H, N // 2), f32, dev, optional=True)
    _check("y", y, x.shape, f32, dev, optional=True)
    _check("final_state", final_state, (b, H, P, N), f32, dev, optional=True)
    _need_device(x, "forward")
    dev = x.device
    for name, t in (("B", B), ("C", C), ("da", da), ("D", D), ("init_state", init_state),
                    ("theta", theta), ("y", y), ("final_state", final_state)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if y is None:
        y = torch.empty(x.shape, device=dev, dtype=torch.float32)
    if final_state is None:
        final_state = torch.empty((b, H, P, N), device=dev, dtype=torch.float32)
    dims = make_dims(b, T, H, P, N, G, in_dtype)
    opts = SsdLaunchOpts()
    opts.segments = int(segments)
    opts.block_slices = int(block_slices)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    if walk_events is not None:
        opts.walk_events[0], opts.walk_events[1] = _event_handles(walk_events, stream, dev)
    with torch.cuda.device(dev):
        st = ssd_forward_ex(dims, x.data_ptr(), da.data_ptr(), B.data_ptr(), C.data_ptr(),
                            _dptr(D), _dptr(init_state), chunk_len, R, _dptr(theta),
                            y.data_ptr(), final_state.data_ptr(), opts, stream)
    if st != SSD_OK:
        raise SsdError(st, "ssd_forward_ex")
    return y, final_state


def selective_scan(u, delta, A, B, C, skip, y=None, stream=None, chunks: int = 0,
                   walk_events=None) -> "torch.Tensor":
    """Run the diagonal selective scan on device tensors; returns y.

    u, delta [b,T,D], A [D,N], B/C [b,T,N], skip [D]: fp32, contiguous, one
    device. y (fp32 [b,T,D], contiguous) may be given to write in place.
    ``chunks`` (0: automatic) and ``walk_events`` (recorded around the output
    pass) are the launch options of ssd_selective_scan_ex.
    """
    import torch

    if not isinstance(u, torch.Tensor) or u.dim() != 3:
        raise ValueError("u must be a [batch, seq_len, d_model] tensor")
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError("A must be a [d_model, d_state] tensor")
    b, T, Dm = u.shape
    N = A.shape[-1]
    f32 = torch.float32
    dev = None if u.device.type == "cpu" else u.device
    want = {"u": (b, T, Dm), "delta": (b, T, Dm), "A": (Dm, N), "B": (b, T, N),
            "C": (b, T, N), "skip": (Dm,)}
    for name, t in (("u", u), ("delta", delta), ("A", A), ("B", B), ("C", C), ("skip", skip)):
        _check(name, t, want[name], f32, dev)
    _check("y", y, (b, T, Dm), f32, dev, optional=True)
    if u.device.type != "cuda":
        raise ValueError("chunked_ssd_scan_amd.selective_scan needs device tensors")
    dev = u.device
    for name, t in (("delta", delta), ("A", A), ("B", B), ("C", C), ("skip", skip), ("y", y)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if y is None:
        y = torch.empty((b, T, Dm), device=dev, dtype=torch.float32)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    opts = SsdLaunchOpts()
    opts.segments = int(chunks)
    if walk_events is not None:
        opts.walk_events[0], opts.walk_events[1] = _event_handles(walk_events, stream, dev)
    with torch.cuda.device(dev):
        st = ssd_selective_scan_ex(u.data_ptr(), delta.data_ptr(), A.data_ptr(), B.data_ptr(),
                                   C.data_ptr(), skip.data_ptr(), y.data_ptr(), b, T, Dm, N,
                                   opts, stream)
    if st != SSD_OK:
        raise SsdError(st, "ssd_selective_scan_ex")
    return y


def trapezoid(x, da, B, C, beta, gamma, prev_x=None, prev_B=None, init_state=None,
              chunk_len: int = 256, theta=None, y=None, final_state=None, segments: int = 0,
              stream=None, walk_events=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Run the Mamba-3 trapezoid forward on device tensors; returns (y, final_state).

    Shapes as ``forward`` (no D), plus beta, gamma [b,T,H] fp32 and the
    optional previous-token entries prev_x [b,R,H,P], prev_B [b,R,G,N] in
    x's dtype (both or neither).
    """
    import torch

    if (prev_x is None) != (prev_B is None):
        raise ValueError("prev_x and prev_B go together (both or neither)")
    (b, T, R, H, P, G, N), px5, pB5 = _ssd_sizes(x, B, prev_x, prev_B)
    in_dtype = _in_dtype(x)
    f32 = torch.float32
    dev = None if x.device.type == "cpu" else x.device
    _check("x", x, x.shape, x.dtype, dev)
    _check("B", B, B.shape, x.dtype, dev)
    _check("C", C, B.shape, x.dtype, dev)
    _check("da", da, (b, T, H), f32, dev)
    _check("beta", beta, (b, T, H), f32, dev)
    _check("gamma", gamma, (b, T, H), f32, dev)
    if px5 is not None:
        _check("prev_x", px5, (b, R, H, P), x.dtype, None)
        _check("prev_B", pB5, (b, R, G, N), x.dtype, None)
        _check("prev_x", prev_x, prev_x.shape, x.dtype, dev)
        _check("prev_B", prev_B, prev_B.shape, x.dtype, dev)
    _check("init_state", init_state, (b, H, P, N), f32, dev, optional=True)
    _check("theta", theta, (b, T, H, N // 2), f32, dev, optional=True)
    _check("y", y, x.shape, f32, dev, optional=True)
    _check("final_state", final_state, (b, H, P, N), f32, dev, optional=True)
    _need_device(x, "trapezoid")
    dev = x.device
    for name, t in (("B", B), ("C", C), ("da", da), ("beta", beta), ("gamma", gamma),
                    ("prev_x", prev_x), ("prev_B", prev_B), ("init_state", init_state),
                    ("theta", theta), ("y", y), ("final_state", final_state)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if y is None:
        y = torch.empty(x.shape, device=dev, dtype=torch.float32)
    if final_state is None:
        final_state = torch.empty((b, H, P, N), device=dev, dtype=torch.float32)
    dims = make_dims(b, T, H, P, N, G, in_dtype)
    opts = SsdLaunchOpts()
    opts.segments = int(segments)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    if walk_events is not None:
        opts.walk_events[0], opts.walk_events[1] = _event_handles(walk_events, stream, dev)
    with torch.cuda.device(dev):
        st = ssd_trapezoid_forward(dims, x.data_ptr(), da.data_ptr(), B.data_ptr(), C.data_ptr(),
                                   beta.data_ptr(), gamma.data_ptr(), _dptr(prev_x), _dptr(prev_B),
                                   _dptr(init_state), chunk_len, R, _dptr(theta), y.data_ptr(),
                                   final_state.data_ptr(), opts, stream)
    if st != SSD_OK:
        raise SsdError(st, "ssd_trapezoid_forward")
    return y, final_state


def state_moments(x, da, B, beta=None, gamma=None, prev_x=None, prev_B=None, init_state=None,
                  theta=None, valid_len=None, m2=None, m1=None, stream=None):
    """Physical-frame state moments on device tensors; returns (m2, m1).

    Shapes as ``trapezoid`` without C (beta and gamma both None for the
    single-write recurrence of ``forward``); valid_len defaults to T.
    m2 [b,H,N,N] and m1 [b,H,N] fp32 may be given to write in place.
    """
    import torch

    if (beta is None) != (gamma is None):
        raise ValueError("beta and gamma go together (both or neither)")
    if (prev_x is None) != (prev_B is None):
        raise ValueError("prev_x and prev_B go together (both or neither)")
    if prev_x is not None and beta is None:
        raise ValueError("prev_x and prev_B belong to the trapezoid (beta, gamma)")
    (b, T, R, H, P, G, N), px5, pB5 = _ssd_sizes(x, B, prev_x, prev_B)
    in_dtype = _in_dtype(x)
    f32 = torch.float32
    dev = None if x.device.type == "cpu" else x.device
    _check("x", x, x.shape, x.dtype, dev)
    _check("B", B, B.shape, x.dtype, dev)
    _check("da", da, (b, T, H), f32, dev)
    _check("beta", beta, (b, T, H), f32, dev, optional=True)
    _check("gamma", gamma, (b, T, H), f32, dev, optional=True)
    if px5 is not None:
        _check("prev_x", px5, (b, R, H, P), x.dtype, None)
        _check("prev_B", pB5, (b, R, G, N), x.dtype, None)
        _check("prev_x", prev_x, prev_x.shape, x.dtype, dev)
        _check("prev_B", prev_B, prev_B.shape, x.dtype, dev)
    _check("init_state", init_state, (b, H, P, N), f32, dev, optional=True)
    _check("theta", theta, (b, T, H, N // 2), f32, dev, optional=True)
    _check("m2", m2, (b, H, N, N), f32, dev, optional=True)
    _check("m1", m1, (b, H, N), f32, dev, optional=True)
    vl = T if valid_len is None else int(valid_len)
    if not 1 <= vl <= T:
        raise ValueError(f"valid_len {vl} outside 1..{T}")
    _need_device(x, "state_moments")
    dev = x.device
    for name, t in (("B", B), ("da", da), ("beta", beta), ("gamma", gamma), ("prev_x", prev_x),
                    ("prev_B", prev_B), ("init_state", init_state), ("theta", theta), ("m2", m2),
                    ("m1", m1)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if m2 is None:
        m2 = torch.empty((b, H, N, N), device=dev, dtype=f32)
    if m1 is None:
        m1 = torch.empty((b, H, N), device=dev, dtype=f32)
    dims = make_dims(b, T, H, P, N, G, in_dtype)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = ssd_state_moments(dims, x.data_ptr(), da.data_ptr(), B.data_ptr(), _dptr(beta),
                               _dptr(gamma), _dptr(prev_x), _dptr(prev_B), _dptr(init_state), R,
                               _dptr(theta), vl, m2.data_ptr(), m1.data_ptr(), stream)
    if st != SSD_OK:
        raise SsdError(st, "ssd_state_moments")
    return m2, m1


def backward(x, da, B, C, dy, D=None, init_state=None, theta=None, dfinal=None,
             want_dinit: bool = True, out=None, stream=None) -> dict:
    """Gradients of ``forward`` on device tensors; returns a dict of fp32 tensors.

    Inputs as ``forward`` plus dy (fp32, shaped like x) and dfinal [b,H,P,N]
    fp32 (None: zero). Keys: dx (shaped like x), dda, dB and dC (shaped like
    B), dinit (when want_dinit), dtheta (when theta is given), dD (when D is
    given). ``out`` may hold tensors under those keys to write in place.
    """
    import torch

    (b, T, R, H, P, G, N), _, _ = _ssd_sizes(x, B)
    in_dtype = _in_dtype(x)
    f32 = torch.float32
    dev = None if x.device.type == "cpu" else x.device
    _check("x", x, x.shape, x.dtype, dev)
    _check("B", B, B.shape, x.dtype, dev)
    _check("C", C, B.shape, x.dtype, dev)
    _check("da", da, (b, T, H), f32, dev)
    _check("D", D, (H,), f32, dev, optional=True)
    _check("init_state", init_state, (b, H, P, N), f32, dev, optional=True)
    _check("theta", theta, (b, T, H, N // 2), f32, dev, optional=True)
    _check("dy", dy, x.shape, f32, dev)
    _check("dfinal", dfinal, (b, H, P, N), f32, dev, optional=True)
    out = dict(out or {})
    shapes = {"dx": x.shape, "dda": (b, T, H), "dB": B.shape, "dC": B.shape}
    if want_dinit:
        shapes["dinit"] = (b, H, P, N)
    if theta is not None:
        shapes["dtheta"] = (b, T, H, N // 2)
    if D is not None:
        shapes["dD"] = (H,)
    for k in out:
        if k not in shapes:
            raise ValueError(f"out[{k!r}] is not an output of this call")
    for k, shp in shapes.items():
        _check(k, out.get(k), shp, f32, dev, optional=True)
    _need_device(x, "backward")
    dev = x.device
    for name, t in [("B", B), ("C", C), ("da", da), ("D", D), ("init_state", init_state),
                    ("theta", theta), ("dy", dy), ("dfinal", dfinal)] + list(out.items()):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    for k, shp in shapes.items():
        if out.get(k) is None:
            out[k] = torch.empty(shp, device=dev, dtype=f32)
    dims = make_dims(b, T, H, P, N, G, in_dtype)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = ssd_backward(dims, x.data_ptr(), da.data_ptr(), B.data_ptr(), C.data_ptr(), _dptr(D),
                          _dptr(init_state), R, _dptr(theta), dy.data_ptr(), _dptr(dfinal),
                          out["dx"].data_ptr(), out["dda"].data_ptr(), out["dB"].data_ptr(),
                          out["dC"].data_ptr(), _dptr(out.get("dtheta")), _dptr(out.get("dinit")),
                          _dptr(out.get("dD")), stream)
    if st != SSD_OK:
        raise SsdError(st, "ssd_backward")
    return out
