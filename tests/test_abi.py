"""The C-ABI library: it loads, exports every symbol the header declares, and
rejects bad arguments on the host (no GPU needed: validation precedes any HIP
call, and these calls never reach one)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import chunked_ssd_scan_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd_scan.h")

# fake, 256-byte aligned device addresses: never dereferenced by these calls
X, DA, BB, CC, DD, H0, TH, Y, FS = (0x10000000 * (i + 1) for i in range(9))


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIB_PATH):
        pytest.skip("libssd_scan.so not built")
    return ssd.load_library()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert set(declared) == set(ssd.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    names = {0: "SSD_OK", 1: "SSD_ERR_NULL_ARG", 2: "SSD_ERR_BAD_SHAPE",
             3: "SSD_ERR_UNSUPPORTED", 4: "SSD_ERR_ALIAS", 5: "SSD_ERR_HIP",
             6: "SSD_ERR_WORKSPACE"}
    for k, v in names.items():
        assert ssd.ssd_status_str(k) == v
    assert ssd.ssd_status_str(99) == "unknown status"
    assert ssd.ssd_status_str(-1) == "unknown status"


def dims(**kw):
    base = dict(batch=2, seqlen=100, nheads=4, headdim=64, dstate=128, ngroups=1,
                in_dtype=ssd.SSD_BF16)
    base.update(kw)
    return ssd.make_dims(**base)


def call(d=None, x=X, da=DA, B=BB, C=CC, D=DD, init=H0, chunk=64, R=1, theta=None,
         y=Y, fin=FS, opts=None, use_default=False):
    if d is None and not use_default:
        d = dims()
    if opts is None:
        return ssd.ssd_forward(d, x, da, B, C, D, init, chunk, R, theta, y, fin, None)
    return ssd.ssd_forward_ex(d, x, da, B, C, D, init, chunk, R, theta, y, fin, opts, None)


@pytest.mark.parametrize("field", ["x", "da", "B", "C", "y", "fin"])
def test_null_required_pointer(lib, field):
    assert call(**{field: None}) == ssd.SSD_ERR_NULL_ARG


def test_null_dims(lib):
    assert call(d=None, use_default=True) == ssd.SSD_ERR_NULL_ARG


@pytest.mark.parametrize("kw", [dict(seqlen=0), dict(batch=0), dict(nheads=0), dict(headdim=0),
                                dict(dstate=0), dict(ngroups=0), dict(nheads=4, ngroups=3),
                                dict(seqlen=-5)])
def test_bad_shape(lib, kw):
    assert call(d=dims(**kw)) == ssd.SSD_ERR_BAD_SHAPE


def test_bad_chunk_and_rank(lib):
    assert call(chunk=0) == ssd.SSD_ERR_BAD_SHAPE
    assert call(R=0) == ssd.SSD_ERR_BAD_SHAPE
    # an odd state size cannot be rotated pairwise
    assert call(d=dims(dstate=17), theta=TH) == ssd.SSD_ERR_BAD_SHAPE


@pytest.mark.parametrize("kw,R", [(dict(headdim=48), 1), (dict(headdim=256), 1), (dict(headdim=8), 1),
                                  (dict(dstate=512), 1), (dict(dstate=96), 1), (dict(dstate=8), 1),
                                  (dict(in_dtype=7), 1), (dict(), 3), (dict(), 32)])
def test_unsupported(lib, kw, R):
    assert call(d=dims(**kw), R=R) == ssd.SSD_ERR_UNSUPPORTED


def test_misaligned(lib):
    assert call(x=X + 2) == ssd.SSD_ERR_UNSUPPORTED
    assert call(y=Y + 4) == ssd.SSD_ERR_UNSUPPORTED
    assert call(da=DA + 1) == ssd.SSD_ERR_UNSUPPORTED


def test_alias(lib):
    assert call(y=X) == ssd.SSD_ERR_ALIAS
    assert call(fin=DA) == ssd.SSD_ERR_ALIAS
    assert call(y=FS) == ssd.SSD_ERR_ALIAS
    assert call(fin=Y + 4096) == ssd.SSD_ERR_ALIAS          # inside y
    assert call(fin=H0 + 256) == ssd.SSD_ERR_ALIAS          # overlaps init but is not it


def test_bad_launch_options(lib):
    opts = ssd.SsdLaunchOpts()
    opts.segments = -1
    assert call(opts=opts) == ssd.SSD_ERR_BAD_SHAPE
    opts = ssd.SsdLaunchOpts()
    opts.block_slices = -2
    assert call(opts=opts) == ssd.SSD_ERR_BAD_SHAPE
    opts = ssd.SsdLaunchOpts()
    opts.reserved[1] = 1
    assert call(opts=opts) == ssd.SSD_ERR_BAD_SHAPE
    opts = ssd.SsdLaunchOpts()
    opts.walk_events[0] = 1           # one event without the other
    assert call(opts=opts) == ssd.SSD_ERR_BAD_SHAPE
    opts = ssd.SsdLaunchOpts()
    opts.block_slices = 7             # not a column-block width
    assert call(opts=opts) == ssd.SSD_ERR_UNSUPPORTED


def test_workspace_bytes(lib):
    # enough (batch, head) pairs to fill the chip: one segment; the only scratch
    # is the shared C B^T tile pack, 32x32 floats per (batch, group, 32-row tile)
    tiles = 8 * (8192 // 32)
    assert ssd.ssd_workspace_bytes(dims(batch=8, seqlen=8192, nheads=80), 256, 1) == tiles * 768 * 4
    # few pairs on a long sequence: segments, and scratch for their states
    n = ssd.ssd_workspace_bytes(dims(batch=1, seqlen=131072, nheads=64), 256, 1)
    assert n >= 64 * 2 * 64 * 128 * 4 + (131072 // 32) * 768 * 4
    assert ssd.ssd_workspace_bytes(dims(seqlen=0), 256, 1) == 0


# ---- ssd_selective_scan ----------------------------------------------------

U, DL, AA, SB, SC, SK, SY = (0x10000000 * (i + 20) for i in range(7))


def sel_call(u=U, delta=DL, A=AA, B=SB, C=SC, skip=SK, y=SY, b=2, T=100, D=512, N=16):
    return ssd.ssd_selective_scan(u, delta, A, B, C, skip, y, b, T, D, N, None)


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "skip", "y"])
def test_selective_null_pointer(lib, field):
    assert sel_call(**{field: None}) == ssd.SSD_ERR_NULL_ARG


@pytest.mark.parametrize("kw", [dict(b=0), dict(T=0), dict(D=0), dict(N=0), dict(T=-3)])
def test_selective_bad_shape(lib, kw):
    assert sel_call(**kw) == ssd.SSD_ERR_BAD_SHAPE


def test_selective_unsupported(lib):
    assert sel_call(N=65) == ssd.SSD_ERR_UNSUPPORTED
    assert sel_call(b=65536) == ssd.SSD_ERR_UNSUPPORTED
    assert sel_call(b=1, T=1, D=(1 << 22) + 1) == ssd.SSD_ERR_UNSUPPORTED
    assert sel_call(u=U + 2) == ssd.SSD_ERR_UNSUPPORTED
    assert sel_call(y=SY + 1) == ssd.SSD_ERR_UNSUPPORTED


def test_selective_alias(lib):
    assert sel_call(y=U) == ssd.SSD_ERR_ALIAS
    assert sel_call(y=DL + 4096) == ssd.SSD_ERR_ALIAS        # inside delta
    assert sel_call(y=AA - 4) == ssd.SSD_ERR_ALIAS           # runs into A


def test_selective_launch_options(lib):
    def ex(opts):
        return ssd.ssd_selective_scan_ex(U, DL, AA, SB, SC, SK, SY, 2, 100, 512, 16, opts, None)
    opts = ssd.SsdLaunchOpts()
    opts.segments = -1
    assert ex(opts) == ssd.SSD_ERR_BAD_SHAPE
    opts = ssd.SsdLaunchOpts()
    opts.reserved[0] = 3
    assert ex(opts) == ssd.SSD_ERR_BAD_SHAPE
    opts = ssd.SsdLaunchOpts()
    opts.walk_events[1] = 1
    assert ex(opts) == ssd.SSD_ERR_BAD_SHAPE
    opts = ssd.SsdLaunchOpts()
    opts.block_slices = 2
    assert ex(opts) == ssd.SSD_ERR_UNSUPPORTED
    assert ssd.ssd_selective_scan_ex(None, DL, AA, SB, SC, SK, SY, 2, 100, 512, 16, None,
                                     None) == ssd.SSD_ERR_NULL_ARG


# ---- ssd_trapezoid_forward -------------------------------------------------

BE, GA, PX, PB = (0x10000000 * (i + 40) for i in range(4))


def trap_call(d=None, x=X, da=DA, B=BB, C=CC, beta=BE, gamma=GA, px=PX, pb=PB, init=H0,
              chunk=64, R=1, theta=None, y=Y, fin=FS, opts=None):
    if d is None:
        d = dims()
    return ssd.ssd_trapezoid_forward(d, x, da, B, C, beta, gamma, px, pb, init, chunk, R, theta,
                                     y, fin, opts, None)


@pytest.mark.parametrize("field", ["x", "da", "B", "C", "beta", "gamma", "y", "fin"])
def test_trapezoid_null_pointer(lib, field):
    assert trap_call(**{field: None}) == ssd.SSD_ERR_NULL_ARG


def test_trapezoid_prev_both_or_neither(lib):
    assert trap_call(px=None) == ssd.SSD_ERR_NULL_ARG
    assert trap_call(pb=None) == ssd.SSD_ERR_NULL_ARG
    assert ssd.ssd_trapezoid_forward(None, X, DA, BB, CC, BE, GA, None, None, None, 64, 1, None, Y,
                                     FS, None, None) == ssd.SSD_ERR_NULL_ARG


def test_trapezoid_shape_and_envelope(lib):
    assert trap_call(d=dims(seqlen=0)) == ssd.SSD_ERR_BAD_SHAPE
    assert trap_call(d=dims(nheads=4, ngroups=3)) == ssd.SSD_ERR_BAD_SHAPE
    assert trap_call(d=dims(dstate=17), theta=TH) == ssd.SSD_ERR_BAD_SHAPE
    assert trap_call(d=dims(headdim=48)) == ssd.SSD_ERR_UNSUPPORTED
    assert trap_call(R=3) == ssd.SSD_ERR_UNSUPPORTED
    assert trap_call(x=X + 2) == ssd.SSD_ERR_UNSUPPORTED
    assert trap_call(beta=BE + 2) == ssd.SSD_ERR_UNSUPPORTED
    assert trap_call(px=PX + 8) == ssd.SSD_ERR_UNSUPPORTED
    assert trap_call(pb=PB + 2) == ssd.SSD_ERR_UNSUPPORTED


def test_trapezoid_alias(lib):
    assert trap_call(y=X) == ssd.SSD_ERR_ALIAS
    assert trap_call(y=BE) == ssd.SSD_ERR_ALIAS
    assert trap_call(fin=GA) == ssd.SSD_ERR_ALIAS
    assert trap_call(fin=H0 + 256) == ssd.SSD_ERR_ALIAS
    assert trap_call(y=FS) == ssd.SSD_ERR_ALIAS
    opts = ssd.SsdLaunchOpts()
    opts.reserved[0] = 1
    assert trap_call(opts=opts) == ssd.SSD_ERR_BAD_SHAPE


def test_noalloc_checks_before_anything(lib):
    # the no-allocation entry point validates as ssd_forward_ex does and
    # rejects a plan larger than its fixed scratch, all on the host
    d = dims()
    assert ssd.ssd_forward_noalloc(None, X, DA, BB, CC, DD, H0, 64, 1, None, Y, FS, None,
                                   None) == ssd.SSD_ERR_NULL_ARG
    assert ssd.ssd_forward_noalloc(d, X, DA, BB, CC, DD, H0, 0, 1, None, Y, FS, None,
                                   None) == ssd.SSD_ERR_BAD_SHAPE
    assert ssd.ssd_forward_noalloc(d, X, DA, BB, CC, DD, H0, 64, 1, None, X, FS, None,
                                   None) == ssd.SSD_ERR_ALIAS
    big = dims(batch=64, seqlen=65536)
    assert ssd.ssd_workspace_bytes(big, 256, 1) > ssd.SSD_NOALLOC_SCRATCH_BYTES
    far = [(i + 1) << 36 for i in range(6)]    # spans of this size do not overlap
    assert ssd.ssd_forward_noalloc(big, far[0], far[1], far[2], far[3], None, None, 256, 1, None,
                                   far[4], far[5], None, None) == ssd.SSD_ERR_WORKSPACE


def test_state_moments_checks(lib):
    # host-side checks of ssd_state_moments (fake pointers, never dereferenced)
    d = dims()
    M2, M1 = (0x10000000 * (i + 20) for i in range(2))
    bt, gm = 0x10000000 * 30, 0x10000000 * 31
    call_m = lambda **kw: ssd.ssd_state_moments(
        kw.get("d", d), X, DA, BB, kw.get("beta"), kw.get("gamma"), kw.get("px"), kw.get("pB"),
        H0, kw.get("R", 1), kw.get("theta"), kw.get("vl", 100), kw.get("m2", M2), kw.get("m1", M1),
        None)
    assert call_m(d=None) == ssd.SSD_ERR_NULL_ARG
    assert call_m(m2=None) == ssd.SSD_ERR_NULL_ARG
    assert call_m(beta=bt) == ssd.SSD_ERR_NULL_ARG                 # beta without gamma
    assert call_m(px=X) == ssd.SSD_ERR_NULL_ARG                    # prev_x without prev_B
    assert call_m(px=X, pB=BB) == ssd.SSD_ERR_BAD_SHAPE            # previous token without beta
    assert call_m(vl=0) == ssd.SSD_ERR_BAD_SHAPE
    assert call_m(vl=101) == ssd.SSD_ERR_BAD_SHAPE
    assert call_m(d=dims(dstate=256)) == ssd.SSD_ERR_UNSUPPORTED
    assert call_m(m2=X) == ssd.SSD_ERR_ALIAS
    assert call_m(m1=M2) == ssd.SSD_ERR_ALIAS
    assert call_m(theta=TH + 4) == ssd.SSD_ERR_UNSUPPORTED         # theta not 16-byte aligned


def test_backward_checks(lib):
    # host-side checks of ssd_backward (fake pointers, never dereferenced)
    d = dims()
    DY, DF, DX, DDA, DB, DC, DTH, DI, DDD = (0x10000000 * (i + 40) for i in range(9))

    def call_b(**kw):
        g = lambda k, v: kw[k] if k in kw else v
        return ssd.ssd_backward(g("d", d), X, DA, BB, CC, g("D", None), H0, g("R", 1),
                                g("theta", None), g("dy", DY), g("dfinal", DF), g("dx", DX),
                                DDA, DB, DC, g("dtheta", None), g("dinit", DI), g("dD", None),
                                None)
    assert call_b(d=None) == ssd.SSD_ERR_NULL_ARG
    assert call_b(dy=None) == ssd.SSD_ERR_NULL_ARG
    assert call_b(dx=None) == ssd.SSD_ERR_NULL_ARG
    assert call_b(theta=TH) == ssd.SSD_ERR_NULL_ARG                # theta without dtheta
    assert call_b(dtheta=DTH) == ssd.SSD_ERR_NULL_ARG              # dtheta without theta
    assert call_b(D=DD) == ssd.SSD_ERR_NULL_ARG                    # D without dD
    assert call_b(dD=DDD) == ssd.SSD_ERR_NULL_ARG
    assert call_b(d=dims(dstate=256)) == ssd.SSD_ERR_UNSUPPORTED
    assert call_b(d=dims(headdim=48)) == ssd.SSD_ERR_UNSUPPORTED
    assert call_b(d=dims(nheads=3, ngroups=2)) == ssd.SSD_ERR_BAD_SHAPE
    assert call_b(R=3) == ssd.SSD_ERR_UNSUPPORTED
    assert call_b(dx=X) == ssd.SSD_ERR_ALIAS                       # dx over x
    assert call_b(dx=DY) == ssd.SSD_ERR_ALIAS                      # dx over dy
    assert call_b(dinit=DX) == ssd.SSD_ERR_ALIAS                   # two outputs overlap
    assert call_b(dfinal=DF + 8) == ssd.SSD_ERR_UNSUPPORTED        # dfinal not 16-byte aligned
    assert call_b(theta=TH + 4, dtheta=DTH) == ssd.SSD_ERR_UNSUPPORTED
