"""GPU parity on seeded random geometries: kernel size, stride, dilation,
padding, offset_scale (negative too), groups and channels per group, dtype,
DCNv3 softmax or DCNv4 raw mask, remove_center, the split or the packed
offset+mask layout, and offset spreads from sub-pixel to beyond the tiles'
margins.  Each case runs the forward and the backward through the C ABI and
compares every output with the binary64 oracle, element by element, to the
bounds of tests/tolerance.py.  The draws are a fixed function of the case
number, so a failure names a reproducible geometry.

Half-precision grad_input is a binary32 sum rounded once (the bounds' rtol
covers that rounding, no store_roundings); a softmax grad_mask of half
precision may carry one more rounding (the untiled kernel stores the raw mask
gradient in the dtype and reads it back for the Jacobian).
"""
import random
import sys

import pytest
import torch

import deformable_convolution_core_amd as dcn
import oracle
from deformable_convolution_core_amd import inputs
from tests import tolerance
from tests.test_gpu_parity import DEV, cfg_of, oracle_bwd, oracle_fwd

pytestmark = pytest.mark.gpu
NCASES = 160


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def draw(case):
    """The geometry of one case: a Workload and the layout flag."""
    r = random.Random(20261203 + 7919 * case)
    while True:
        dt = r.choice(["f32", "f16", "bf16"])
        K = r.choice([1, 3, 3, 3, 5, 7])
        rc = K >= 3 and r.random() < 0.25
        d = r.choice([1, 1, 2])
        s = r.choice([1, 1, 2, 3])
        c0 = d * (K - 1) // 2
        p = r.randint(0, c0 + 1)
        G = r.randint(1, 4)
        Cg = r.choice([1, 2, 4, 8, 16, 16, 32])
        H, W = r.randint(max(1, K * d - 2 * p), 20), r.randint(max(1, K * d - 2 * p), 20)
        Ho, Wo = oracle.out_size(H, K, s, p, d), oracle.out_size(W, K, s, p, d)
        if Ho < 1 or Wo < 1:
            continue
        N = r.choice([1, 2])
        alpha = r.choice([1.0, 1.0, 0.7, 1.3, -1.1])
        sm = r.random() < 0.4
        sigma = r.choice([0.5, 1.5, 1.5, 3.0, 8.0])
        packed = r.random() < 0.3
        w = inputs.Workload(name=f"rand{case}", N=N, H=H, W=W, G=G, Cg=Cg, Ho=Ho, Wo=Wo, K=K, stride=s, pad=p,
                            dilation=d, offset_scale=alpha, softmax=sm, dtype=dt, offset_sigma=sigma,
                            mask_sigma=1.0 if sm else 0.5, seed_base=990000 + 101 * case, backward=True,
                            remove_center=rc)
        return w, packed


def describe(w, packed):
    return (f"{w.name}: {w.dtype} N={w.N} {w.H}x{w.W} G={w.G} Cg={w.Cg} K={w.K} s={w.stride} p={w.pad} "
            f"d={w.dilation} alpha={w.offset_scale} softmax={w.softmax} rc={w.remove_center} "
            f"sigma={w.offset_sigma} packed={packed}")


@pytest.mark.parametrize("case", range(NCASES))
def test_random_geometry(case):
    w, packed = draw(case)
    what = describe(w, packed)
    print(f"[gpu-case] {what}", file=sys.stderr, flush=True)
    t = inputs.make(w, with_grad=True)
    d = {k: v.to(DEV) for k, v in t.items()}
    kw = cfg_of(w)
    if packed:
        om = inputs.pack_offset_mask(t["offset"], t["mask"], w.G, w.P).to(DEV)
        out = dcn.forward_packed(d["input"], om, **kw)
        gi, gom = dcn.backward_packed(d["input"], om, d["grad_out"], **kw)
        goff, gm = inputs.unpack_offset_mask(gom, w.G, w.P)
    else:
        out = dcn.forward(d["input"], d["offset"], d["mask"], **kw)
        gi, goff, gm = dcn.backward(d["input"], d["offset"], d["mask"], d["grad_out"], **kw)
    torch.cuda.synchronize()

    ref, S = oracle_fwd(t, w)
    st = tolerance.compare(out.float().cpu().numpy(), ref, S, 4 * w.P, w.dtype)
    assert st["ok"], (what, "output", st)

    r = oracle_bwd(t, w)
    half = w.dtype != "f32"
    for key, got, S, n, extra in (
            ("grad_input", gi, r["gi_abs"], r["gi_cnt"], 0),
            ("grad_offset", goff, r["goff_abs"], 4 * w.Cg, 0),
            ("grad_mask", gm, r["gmask_abs"], 4 * w.Cg * (w.P + 1) if w.softmax else 4 * w.Cg,
             1 if half and w.softmax else 0)):
        st = tolerance.compare(got.float().cpu().numpy().reshape(r[key].shape), r[key], S, n, w.dtype,
                               store_roundings=extra)
        assert st["ok"], (what, key, st)


def test_draws_cover_every_path():
    """The fixed draws include each dtype, both mask modes, both layouts,
    remove_center, every K, strides above 1, dilation 2 and negative
    offset_scale (checked on the host)."""
    ws = [draw(c) for c in range(NCASES)]
    assert {w.dtype for w, _ in ws} == {"f32", "f16", "bf16"}
    assert {w.softmax for w, _ in ws} == {False, True}
    assert {p for _, p in ws} == {False, True}
    assert any(w.remove_center for w, _ in ws)
    assert {w.K for w, _ in ws} == {1, 3, 5, 7}
    assert any(w.stride > 1 for w, _ in ws) and any(w.dilation == 2 for w, _ in ws)
    assert any(w.offset_scale < 0 for w, _ in ws)
