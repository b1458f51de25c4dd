"""ssd_forward_noalloc: the entry point that allocates nothing, against
ssd_forward_ex on the same inputs (needs a gfx950 GPU).

Both run the same plan and kernels, so their outputs must agree bit for bit
(the bar for this pair is tighter than the oracle tolerance). Two calls in a
row share the one scratch array of the GPU; the second is smaller, so stale
contents of the first would show up if a kernel read what it did not write.
"""
from __future__ import annotations

import pytest
import torch

import ssd_inputs as si

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _ssd():
    import chunked_ssd_scan_amd as ssd
    ssd.load_library()
    return ssd


def _call(fn, shape, g, segments):
    ssd = _ssd()
    b, T, R, H, P = g.x.shape
    y = torch.full((b, T, R, H, P), float("nan"), device=g.x.device)
    fin = torch.full((b, H, P, shape.dstate), float("nan"), device=g.x.device)
    dims = ssd.make_dims(b, T, H, P, shape.dstate, shape.ngroups,
                         ssd.SSD_BF16 if shape.dtype == "bf16" else ssd.SSD_F32)
    opts = ssd.SsdLaunchOpts()
    opts.segments = segments
    p = lambda t: None if t is None else t.data_ptr()
    st = fn(dims, g.x.data_ptr(), g.da.data_ptr(), g.B.data_ptr(), g.C.data_ptr(), p(g.D),
            p(g.init_state), shape.chunk_len, R, p(g.theta), y.data_ptr(), fin.data_ptr(), opts,
            torch.cuda.current_stream().cuda_stream)
    assert st == ssd.SSD_OK, ssd.ssd_status_str(st)
    return y, fin


def _pair(shape, seed, segments):
    ssd = _ssd()
    g = si.make_inputs(shape, seed=seed).to(_dev())
    dims = ssd.make_dims(shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate,
                         shape.ngroups, ssd.SSD_BF16 if shape.dtype == "bf16" else ssd.SSD_F32)
    need = ssd.ssd_workspace_bytes(dims, shape.chunk_len, shape.mimo_rank)
    y0, f0 = _call(ssd.ssd_forward_ex, shape, g, segments)
    y1, f1 = _call(ssd.ssd_forward_noalloc, shape, g, segments)
    torch.cuda.synchronize()
    print(f"{shape.name or 'shape'} S{segments}: workspace {need} B; "
          f"equal y {torch.equal(y0, y1)} final {torch.equal(f0, f1)}", flush=True)
    assert torch.equal(y0, y1) and torch.equal(f0, f1)


# (large first, smaller second): shared C B^T pack and segment states; then
# the rotating walk (segment states only); then a plan with no scratch at all
CASES = [
    [(dict(batch=2, seqlen=3000, nheads=10, headdim=64, dstate=128, dtype="bf16",
           init_state=True, name="shared pack, segments"), 4),
     (dict(batch=1, seqlen=700, nheads=5, headdim=64, dstate=128, dtype="bf16",
           name="smaller, shared pack, segments"), 3)],
    [(dict(batch=2, seqlen=1500, nheads=4, headdim=64, dstate=128, mimo_rank=4, dtype="bf16",
           rotation=True, init_state=True, name="rotating, segments"), 3),
     (dict(batch=1, seqlen=400, nheads=2, headdim=64, dstate=64, mimo_rank=4, dtype="bf16",
           rotation=True, init_state=True, name="smaller rotating, segments"), 2)],
    [(dict(batch=2, seqlen=300, nheads=3, headdim=32, dstate=64, mimo_rank=2, dtype="f32",
           rotation=True, init_state=True, name="general walk, segments"), 3),
     (dict(batch=1, seqlen=100, nheads=2, headdim=32, dstate=64, mimo_rank=2, dtype="f32",
           rotation=True, name="general walk, no scratch"), 1)],
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_forward_ex(case):
    for i, (kw, segments) in enumerate(CASES[case]):
        _pair(si.small_shape(**kw), seed=40 + 3 * case + i, segments=segments)


def test_noalloc_rejects_oversized_plan():
    # a plan whose C B^T pack alone exceeds the fixed array: rejected on the
    # host before any launch (the pointers are never dereferenced)
    ssd = _ssd()
    _dev()
    dims = ssd.make_dims(64, 65536, 4, 64, 128, 1, ssd.SSD_BF16)
    assert ssd.ssd_workspace_bytes(dims, 256, 1) > ssd.SSD_NOALLOC_SCRATCH_BYTES
    fake = [(i + 1) << 36 for i in range(7)]     # far apart: spans do not overlap
    st = ssd.ssd_forward_noalloc(dims, fake[0], fake[1], fake[2], fake[3], None, None, 256, 1,
                                 None, fake[4], fake[5], None, None)
    assert st == ssd.SSD_ERR_WORKSPACE, ssd.ssd_status_str(st)
