"""GPU parity at the edge of the definition's skip rule.

The fallback of "没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读"
(section 4, step 4) samples with zero padding: a sample whose bilinear
neighbourhood lies off the map contributes nothing.  In pixel coordinates a
sample is skipped unless -1 < x < W and -1 < y < H; at x = -1 exactly its
right-hand corners sit on column 0 with weight zero, and the definition still
skips it, so an Inf or NaN in column 0 must not reach the output (0 * Inf
would be NaN).  Likewise a raw mask of Inf on a skipped sample must not meet
the zeros of the padding.

The input carries +Inf in row 0 and NaN in column 0.  Output pixels near the
top-left corner get one tap at exactly x = -1 (or y = -1) with its other
corners away from row 0 / column 0, and every other tap far off the map with
an Inf raw mask (finite logits under softmax).  The oracle gives exact zeros
there; the rest of the image has random offsets, and wherever a sample
touches row 0 or column 0 the oracle's Inf/NaN must be matched exactly.
Shapes: a map larger than one staged region (left/top tiles whose regions
reach past the map) and a small map whose region is the whole map.
"""
import sys

import numpy as np
import pytest
import torch

import deformable_convolution_core_amd as dcn
import oracle
from deformable_convolution_core_amd import inputs
from tests import tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def skip_rule_inputs(N, H, W, G, Cg, dtype, softmax, seed):
    """Inputs (rounded to dtype) and the boolean map of designed pixels."""
    x = inputs.normal((N, H, W, G * Cg), seed, 1.0, "f32")
    x[:, 0, :, :] = float("inf")
    x[:, :, 0, :] = float("nan")
    off = inputs.normal((N, H, W, G, 9, 2), seed + 1, 1.5, "f32")
    m = inputs.normal((N, H, W, G, 9), seed + 2, 1.0 if softmax else 0.5, "f32")
    far_mask = -1e4 if softmax else float("inf")
    designed = torch.zeros(N, H, W, dtype=torch.bool)
    # K = 3, stride 1, pad 1, dilation 1, offset_scale 1: tap (i, j) samples
    # x = wo - 1 + i + dx, y = ho - 1 + j + dy; tap 0 is (i, j) = (0, 0)
    for ho in range(2, min(H, 12)):
        for wo in range(0, min(W, 6)):
            off[:, ho, wo, :, 0, 0] = -float(wo)        # x = -1 exactly
            off[:, ho, wo, :, 0, 1] = 0.5               # y = ho - 0.5: rows ho-1, ho (not row 0)
            designed[:, ho, wo] = True
    for ho in range(0, min(H, 6)):
        for wo in range(2, min(W, 12)):
            off[:, ho, wo, :, 0, 0] = 0.5               # x = wo - 0.5: columns wo-1, wo (not column 0)
            off[:, ho, wo, :, 0, 1] = -float(ho)        # y = -1 exactly
            designed[:, ho, wo] = True
    sel = designed[:, :, :, None, None].expand(N, H, W, G, 8)
    o = off[..., 1:, :]
    o[sel[..., None].expand_as(o)] = -1e4               # every other tap far off the map
    mk = m[..., 1:]
    mk[sel] = far_mask
    T = inputs.DTYPES[dtype]
    return (x.to(T), off.reshape(N, H, W, G * 18).to(T), m.reshape(N, H, W, G * 9).to(T), designed)


def assert_same_nonfinite_and_close(got, ref, S, n_terms, dtype, what):
    got = np.asarray(got, np.float64)
    for name, f in (("nan", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
        diff = f(got) != f(ref)
        assert not diff.any(), (what, name, int(diff.sum()), np.argwhere(diff)[:4].tolist())
    fin = np.isfinite(ref)
    st = tolerance.compare(got[fin], ref[fin], S[fin], n_terms if np.isscalar(n_terms) else n_terms[fin], dtype)
    assert st["ok"], (what, st)


CASES = [  # N, H, W, dtype, softmax
    (2, 40, 37, "bf16", False),
    (2, 40, 37, "f32", False),
    (1, 40, 37, "f16", True),
    (2, 14, 14, "bf16", False),
    (1, 14, 14, "f32", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"_{c[3]}_{'sm' if c[4] else 'raw'}")
def test_forward_skip_rule_edges(case):
    N, H, W, dt, sm = case
    G, Cg = 4, 16
    x, off, m, designed = skip_rule_inputs(N, H, W, G, Cg, dt, sm, 61000 + H + W)
    out = dcn.forward(x.to(DEV), off.to(DEV), m.to(DEV), group=G, softmax=sm)
    torch.cuda.synchronize()
    ref, S = oracle.forward(inputs.to_f64(x), inputs.to_f64(off), inputs.to_f64(m), K=3, stride=1, pad=1,
                            dilation=1, offset_scale=1.0, softmax=sm, group=G, coord_mode=oracle.COORD_BINARY32)
    got = out.float().cpu().numpy()
    d = designed.numpy()
    assert np.all(ref[d] == 0.0)
    assert np.all(got[d] == 0.0), np.argwhere(got[d] != 0.0)[:4]
    assert_same_nonfinite_and_close(got, ref, S, 36, dt, "forward")


@pytest.mark.parametrize("case", [(2, 40, 37, "f32", False), (1, 40, 37, "bf16", False), (1, 14, 14, "f32", True)],
                         ids=lambda c: "x".join(map(str, c[:3])) + f"_{c[3]}_{'sm' if c[4] else 'raw'}")
def test_backward_skip_rule_edges(case):
    """The same inputs through the backward: skipped samples give zero
    offset and mask gradients and add nothing to grad_input."""
    N, H, W, dt, sm = case
    G, Cg = 4, 16
    x, off, m, designed = skip_rule_inputs(N, H, W, G, Cg, dt, sm, 62000 + H + W)
    g = inputs.normal((N, H, W, G * Cg), 62999, 1.0, dt)
    gi, goff, gm = dcn.backward(x.to(DEV), off.to(DEV), m.to(DEV), g.to(DEV), group=G, softmax=sm)
    torch.cuda.synchronize()
    r = oracle.backward(inputs.to_f64(x), inputs.to_f64(off), inputs.to_f64(m), inputs.to_f64(g), K=3, stride=1,
                        pad=1, dilation=1, offset_scale=1.0, softmax=sm, group=G, coord_mode=oracle.COORD_BINARY32)
    d = designed.numpy()
    goff_np = goff.float().cpu().numpy().reshape(r["grad_offset"].shape)
    gm_np = gm.float().cpu().numpy().reshape(r["grad_mask"].shape)
    gi_np = gi.float().cpu().numpy().reshape(r["grad_input"].shape)
    # designed pixels: every sample but tap 0 is skipped, tap 0 too (x or y = -1)
    assert np.all(r["grad_offset"].reshape(N, H, W, -1)[d] == 0.0)
    assert np.all(goff_np.reshape(N, H, W, -1)[d] == 0.0)
    if not sm:
        assert np.all(gm_np.reshape(N, H, W, -1)[d] == 0.0)
    assert_same_nonfinite_and_close(gi_np, r["grad_input"], r["gi_abs"], r["gi_cnt"], dt, "grad_input")
    assert_same_nonfinite_and_close(goff_np, r["grad_offset"], r["goff_abs"], 4 * Cg, dt, "grad_offset")
    assert_same_nonfinite_and_close(gm_np, r["grad_mask"], r["gmask_abs"], 4 * Cg * 10 if sm else 4 * Cg, dt,
                                    "grad_mask")
