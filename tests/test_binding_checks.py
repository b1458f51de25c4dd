"""The Python binding rejects malformed tensors before anything reaches the C
ABI (no GPU needed: the checks run on the host and raise before any call).

Shape and dtype are checked first, then the device, so CPU tensors with a
wrong shape or dtype raise the shape or dtype error here; a tensor on another
device than x is caught with the meta device standing in for a second one.
"""
from __future__ import annotations

import pytest
import torch

import chunked_ssd_scan_amd as ssd

b, T, R, H, P, G, N = 2, 10, 2, 4, 16, 2, 32


def ssd_args(**over):
    a = dict(
        x=torch.zeros(b, T, R, H, P, dtype=torch.bfloat16),
        da=torch.zeros(b, T, H),
        B=torch.zeros(b, T, R, G, N, dtype=torch.bfloat16),
        C=torch.zeros(b, T, R, G, N, dtype=torch.bfloat16),
        D=torch.zeros(H),
        init_state=torch.zeros(b, H, P, N),
        theta=torch.zeros(b, T, H, N // 2),
        y=torch.zeros(b, T, R, H, P),
        final_state=torch.zeros(b, H, P, N),
    )
    a.update(over)
    return a


def call_forward(**over):
    a = ssd_args(**over)
    return ssd.forward(a["x"], a["da"], a["B"], a["C"], a["D"], a["init_state"], 64, a["theta"],
                       y=a["y"], final_state=a["final_state"])


BAD_FORWARD = [
    ("y", torch.zeros(b, T, R, H, P - 1), ValueError),                  # short
    ("y", torch.zeros(b, T, R, H, P, dtype=torch.bfloat16), TypeError),  # wrong dtype
    ("y", torch.zeros(b, T, R, H, 2 * P)[..., :P], ValueError),          # strided
    ("final_state", torch.zeros(b, H, P, N - 2), ValueError),
    ("final_state", torch.zeros(b, H, P, N, dtype=torch.float64), TypeError),
    ("da", torch.zeros(b, T, H + 1), ValueError),
    ("da", torch.zeros(b, T, H, dtype=torch.float16), TypeError),
    ("C", torch.zeros(b, T, R, G, N + 8, dtype=torch.bfloat16), ValueError),
    ("C", torch.zeros(b, T, R, G, N), TypeError),
    ("D", torch.zeros(H + 1), ValueError),
    ("init_state", torch.zeros(b, H, P, N // 2), ValueError),
    ("theta", torch.zeros(b, T, H, N), ValueError),
    ("theta", torch.zeros(b, T, H, N // 2, dtype=torch.float64), TypeError),
    ("B", torch.zeros(b, T + 1, R, G, N, dtype=torch.bfloat16), ValueError),
    ("x", torch.zeros(b, T, R, H, P, dtype=torch.float16), TypeError),
]


@pytest.mark.parametrize("name,bad,exc", BAD_FORWARD)
def test_forward_rejects(name, bad, exc):
    with pytest.raises(exc, match=name if exc is ValueError and name != "x" else None):
        call_forward(**{name: bad})


def test_forward_needs_device_tensors():
    with pytest.raises(ValueError, match="device tensors"):
        call_forward()


def test_forward_rejects_other_device():
    meta = {k: (v.to("meta") if v is not None else None) for k, v in ssd_args().items()}
    meta["y"] = torch.zeros(b, T, R, H, P)           # on the host, x on another device
    with pytest.raises(ValueError, match="y is on"):
        ssd.forward(meta["x"], meta["da"], meta["B"], meta["C"], meta["D"], meta["init_state"],
                    64, meta["theta"], y=meta["y"], final_state=meta["final_state"])


def call_trapezoid(**over):
    a = ssd_args(**over)
    beta = over.get("beta", torch.zeros(b, T, H))
    gamma = over.get("gamma", torch.zeros(b, T, H))
    prev_x = over.get("prev_x", torch.zeros(b, R, H, P, dtype=torch.bfloat16))
    prev_B = over.get("prev_B", torch.zeros(b, R, G, N, dtype=torch.bfloat16))
    return ssd.trapezoid(a["x"], a["da"], a["B"], a["C"], beta, gamma, prev_x, prev_B,
                         a["init_state"], 64, a["theta"], y=a["y"], final_state=a["final_state"])


BAD_TRAPEZOID = [
    ("beta", torch.zeros(b, T - 1, H), ValueError),
    ("gamma", torch.zeros(b, T, H, dtype=torch.bfloat16), TypeError),
    ("prev_x", torch.zeros(b, R, H, P + 16, dtype=torch.bfloat16), ValueError),
    ("prev_B", torch.zeros(b, R, G, N), TypeError),
    ("y", torch.zeros(b, T, R, H, P - 4), ValueError),
    ("final_state", torch.zeros(b, H, N, P), ValueError),
    ("theta", torch.zeros(b, T, H, N // 2 + 1), ValueError),
    ("da", torch.zeros(b, T, H, dtype=torch.float64), TypeError),
]


@pytest.mark.parametrize("name,bad,exc", BAD_TRAPEZOID)
def test_trapezoid_rejects(name, bad, exc):
    with pytest.raises(exc):
        call_trapezoid(**{name: bad})


def test_trapezoid_prev_both_or_neither():
    with pytest.raises(ValueError, match="both or neither"):
        call_trapezoid(prev_B=None)


def test_trapezoid_needs_device_tensors():
    with pytest.raises(ValueError, match="device tensors"):
        call_trapezoid()


def scan_args(**over):
    Bs, Ts, Dm, Ns = 2, 9, 5, 4
    a = dict(u=torch.zeros(Bs, Ts, Dm), delta=torch.zeros(Bs, Ts, Dm), A=torch.zeros(Dm, Ns),
             B=torch.zeros(Bs, Ts, Ns), C=torch.zeros(Bs, Ts, Ns), skip=torch.zeros(Dm),
             y=torch.zeros(Bs, Ts, Dm))
    a.update(over)
    return a


BAD_SCAN = [
    ("y", torch.zeros(2, 9, 4), ValueError),
    ("y", torch.zeros(2, 9, 5, dtype=torch.float64), TypeError),
    ("delta", torch.zeros(2, 8, 5), ValueError),
    ("B", torch.zeros(2, 9, 3), ValueError),
    ("skip", torch.zeros(5, dtype=torch.bfloat16), TypeError),
]


@pytest.mark.parametrize("name,bad,exc", BAD_SCAN)
def test_selective_scan_rejects(name, bad, exc):
    a = scan_args(**{name: bad})
    with pytest.raises(exc):
        ssd.selective_scan(a["u"], a["delta"], a["A"], a["B"], a["C"], a["skip"], y=a["y"])


def test_selective_scan_needs_device_tensors():
    a = scan_args()
    with pytest.raises(ValueError, match="device tensors"):
        ssd.selective_scan(a["u"], a["delta"], a["A"], a["B"], a["C"], a["skip"], y=a["y"])
