"""GPU parity of the DCNv4 layer around the core: the centre-feature gate
kernel against the float64 gate of the layer oracle (element by element),
and the whole layer (library GEMMs + HIP core + HIP gate) against the layer
oracle, forward and backward.

The layer's binary32 run is compared normwise: its projections are BLAS
GEMMs whose rounding feeds the sampling coordinates, so an element's error
has no per-element sum to scale with.  For each tensor,
    max |gpu - ref| <= 1e-5 * max |ref|
(a few binary32 roundings per stage, each far below 1e-5 of the largest
element).  In half precision every stage boundary rounds to the dtype, so
the layer is checked stage by stage instead: the core and the gate on the
layer's own intermediates against the oracle, with the core's and the gate's
element-wise bounds, and the layer's output against the same stages
composed by hand.
"""
import random
import sys

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import deformable_convolution_core_amd as dcn
import oracle
from deformable_convolution_core_amd import inputs
from deformable_convolution_core_amd.layer import DCNv4
from oracle import module as om_oracle
from tests import tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def f64(t):
    return t.detach().cpu().double().numpy()


# -------------------------------------------------------------------- gate
GATE = [  # M, G, Cg, dtype   (Cg*b a multiple of 16: vector path; else one element per access)
    (1000, 4, 16, "f32"), (1000, 4, 16, "f16"), (999, 8, 16, "bf16"),
    (777, 3, 5, "f32"), (777, 3, 5, "f16"), (513, 2, 12, "bf16"),
]


def gate_inputs(M, G, Cg, dt, seed):
    y = inputs.normal((M, G * Cg), seed + 1, 1.0, dt)
    v = inputs.normal((M, G * Cg), seed + 2, 1.0, dt)
    z = inputs.normal((M, G), seed + 3, 3.0, dt)
    z.view(-1)[:8] = torch.tensor([30.0, -30.0, 100.0, -100.0, 0.0, 1e-3, -1e-3, 16.0]).to(z.dtype)
    go = inputs.normal((M, G * Cg), seed + 4, 1.0, dt)
    return y, v, z, go


@pytest.mark.parametrize("case", GATE, ids=lambda c: f"M{c[0]}_G{c[1]}_Cg{c[2]}_{c[3]}")
def test_gate_matches_oracle(case):
    M, G, Cg, dt = case
    y, v, z, go = gate_inputs(M, G, Cg, dt, 5000 + M + Cg)
    yd, vd, zd, god = (t.to(DEV) for t in (y, v, z, go))
    out = dcn.center_gate_forward(yd, vd, zd, group=G)
    gy, gv, gz = dcn.center_gate_backward(yd, vd, zd, god, group=G)
    torch.cuda.synchronize()
    Y, V, Z, GO = f64(y), f64(v), f64(z), f64(go)
    s, t = om_oracle.sigmoid(Z)[..., None], om_oracle.sigmoid(-Z)[..., None]
    S_out = (np.abs(Y).reshape(M, G, Cg) * t + np.abs(V).reshape(M, G, Cg) * s).reshape(M, G * Cg)
    ref = om_oracle.gate_forward(Y, V, Z, G)
    # logits of +-100 give gate weights below 2^-126: a few subnormal spacings of absolute error
    atol = {"f32": 2.0 ** -146, "bf16": 2.0 ** -130, "f16": None}[dt]
    st = tolerance.compare(f64(out), ref, S_out, 2, dt, atol=atol)
    assert st["ok"], ("forward", st)
    rgy, rgv, rgz = om_oracle.gate_backward(Y, V, Z, GO, G)
    S_gz = (np.abs(GO).reshape(M, G, Cg) * (np.abs(V) + np.abs(Y)).reshape(M, G, Cg)).sum(-1) * (s[..., 0] * t[..., 0])
    for name, got, want, S, n in (("grad_y", gy, rgy, np.abs(rgy), 1), ("grad_v", gv, rgv, np.abs(rgv), 1),
                                  ("grad_z", gz, rgz, S_gz, 2 * Cg)):
        st = tolerance.compare(f64(got), want, S, n, dt, atol=atol)
        assert st["ok"], (name, st)


def test_gate_in_place_and_empty():
    y, v, z, _ = gate_inputs(300, 4, 16, "f32", 777)
    yd, vd, zd = (t.to(DEV) for t in (y, v, z))
    want = dcn.center_gate_forward(yd, vd, zd, group=4)
    got = dcn.center_gate_forward(yd, vd, zd, group=4, out=yd)     # output over y
    torch.cuda.synchronize()
    assert got.data_ptr() == yd.data_ptr()
    assert torch.equal(got, want)
    e = torch.empty(0, 64, device=DEV)
    assert dcn.center_gate_forward(e, e, torch.empty(0, 4, device=DEV), group=4).numel() == 0


# -------------------------------------------------------------------- layer
LAYER = [  # N, H, W, G, Cg, K, remove_center, center_feature_scale, offset_scale
    (2, 14, 14, 4, 16, 3, False, False, 1.0),
    (2, 14, 13, 4, 16, 3, False, True, 1.0),
    (1, 12, 12, 4, 16, 3, True, True, 0.8),
    (1, 11, 12, 2, 32, 5, False, True, 1.0),
    (1, 9, 10, 3, 8, 3, False, True, 1.0),      # C = 24: not tiled, core and gate as two kernels
]


def make_layer(N, H, W, G, Cg, K, rc, cfs, alpha, dtype, seed):
    C = G * Cg
    torch.manual_seed(seed)
    layer = DCNv4(C, kernel_size=K, group=G, offset_scale=alpha, center_feature_scale=cfs,
                  remove_center=rc, device=DEV, dtype=torch.float32)
    rng = np.random.default_rng(seed)
    P = K * K - (1 if rc else 0)
    with torch.no_grad():
        for lin, std in ((layer.value_proj, 1.0), (layer.output_proj, 1.0), (layer.offset_mask, 1.5)):
            lin.weight.copy_(torch.from_numpy(rng.standard_normal(lin.weight.shape) * std / np.sqrt(C)))
            lin.bias.copy_(torch.from_numpy(rng.standard_normal(lin.bias.shape) * 0.1))
        # mask rows of the merged projection: raw weights of about 0.3
        w = layer.offset_mask.weight.view(G, 3 * P, C)
        w[:, 2 * P:, :] *= 0.3 / 1.5
        if cfs:
            layer.center_feature_scale_proj.weight.copy_(
                torch.from_numpy(rng.standard_normal((G, C)) / np.sqrt(C)))
            layer.center_feature_scale_proj.bias.copy_(torch.from_numpy(rng.standard_normal(G) * 0.3))
    layer = layer.to(dtype=inputs.DTYPES[dtype])
    x = inputs.normal((N, H, W, C), seed + 11, 1.0, dtype).to(DEV)
    gout = inputs.normal((N, H, W, C), seed + 12, 1.0, dtype).to(DEV)
    return layer, x, gout


def normwise_ok(got, want, tol):
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    scale = float(np.max(np.abs(want))) if want.size else 0.0
    return err <= tol * scale, err / scale if scale else err


@pytest.mark.parametrize("case", LAYER, ids=lambda c: f"N{c[0]}_{c[1]}x{c[2]}_G{c[3]}_Cg{c[4]}_K{c[5]}"
                                                          f"_rc{int(c[6])}_cfs{int(c[7])}")
def test_layer_fp32_matches_oracle(case):
    check_layer_fp32(case, 6100 + 7 * case[5] + case[1])


def draw_layer(case):
    """Seeded random layer: sizes 3-16, G 1-4, Cg 4-32, K 3 or 5, with or
    without the centre tap and the gate, offset_scale of either sign."""
    r = random.Random(61700 + 211 * case)
    K = r.choice([3, 3, 5])
    return (r.choice([1, 2]), r.randint(3, 16), r.randint(3, 16), r.choice([1, 2, 3, 4]), r.choice([4, 8, 16, 32]),
            K, r.random() < 0.3, r.random() < 0.6, r.choice([1.0, 0.7, -1.2]))


@pytest.mark.parametrize("case", range(6))
def test_layer_fp32_random_shapes(case):
    check_layer_fp32(draw_layer(case), 6300 + 13 * case)


def check_layer_fp32(case, seed):
    N, H, W, G, Cg, K, rc, cfs, alpha = case
    layer, x, gout = make_layer(*case, "f32", seed)
    xi = x.clone().requires_grad_(True)
    out = layer(xi)
    out.backward(gout)
    torch.cuda.synchronize()
    cfg = dict(kernel_size=K, group=G, remove_center=rc, center_feature_scale=cfs, offset_scale=alpha)
    p = layer.numpy_params()
    ref = om_oracle.module_forward(f64(x), p, cfg)["out"]
    ok, r = normwise_ok(f64(out), ref, 1e-5)
    assert ok, ("out", r)
    g = om_oracle.module_backward(f64(x), p, cfg, f64(gout))
    grads = dict(x=xi.grad, Wv=layer.value_proj.weight.grad, bv=layer.value_proj.bias.grad,
                 Wom=layer.offset_mask.weight.grad, bom=layer.offset_mask.bias.grad,
                 Wo=layer.output_proj.weight.grad, bo=layer.output_proj.bias.grad)
    if cfs:
        grads.update(Wc=layer.center_feature_scale_proj.weight.grad, bc=layer.center_feature_scale_proj.bias.grad)
    for name, got in grads.items():
        ok, r = normwise_ok(f64(got), g[name], 1e-5)
        assert ok, (name, r)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_layer_half_stagewise(dt):
    """Half precision: the layer's output equals its stages composed by hand
    (bit for bit; the core and the gate as the one fused call the layer
    makes), and the projections, the HIP core and the gate match the float64
    definitions on the layer's own intermediates."""
    N, H, W, G, Cg, K = 2, 14, 14, 4, 16, 3
    layer, x, gout = make_layer(N, H, W, G, Cg, K, False, True, 1.0, dt, 6400)
    out = layer(x)
    v = dcn.linear(x, layer.value_proj.weight, layer.value_proj.bias)
    om = dcn.linear(x, layer.offset_mask.weight, layer.offset_mask.bias)
    z = dcn.linear(x, layer.center_feature_scale_proj.weight, layer.center_feature_scale_proj.bias)
    yg, y = dcn.forward_packed_gated(v, om, z, kernel_size=K, group=G, keep_core_output=True)
    want = dcn.linear(yg, layer.output_proj.weight, layer.output_proj.bias)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    # the projections against the float64 product of the same (half-precision) operands
    for got, a, lin in ((v, x, layer.value_proj), (om, x, layer.offset_mask),
                        (z, x, layer.center_feature_scale_proj), (want, yg, layer.output_proj)):
        A, Wt, B = f64(a).reshape(-1, a.shape[-1]), f64(lin.weight), f64(lin.bias)
        ref = A @ Wt.T + B
        S = np.abs(A) @ np.abs(Wt).T + np.abs(B)
        st = tolerance.compare(f64(got).reshape(ref.shape), ref, S, A.shape[1] + 1, dt)
        assert st["ok"], ("projection", st)
    P = K * K
    off, mask = inputs.unpack_offset_mask(om.cpu(), G, P)
    ref, S = oracle.forward(f64(v), f64(off), f64(mask), K=K, stride=1, pad=1, dilation=1, offset_scale=1.0,
                            softmax=False, group=G)
    st = tolerance.compare(f64(y), ref, S, 4 * P, dt)
    assert st["ok"], ("core", st)
    # the fused gate takes the unrounded y: against the gate of the oracle's y
    V, Z = f64(v), f64(z)
    s, t = om_oracle.sigmoid(Z)[..., None], om_oracle.sigmoid(-Z)[..., None]
    S_g = (S.reshape(N, H, W, G, Cg) * t + np.abs(V).reshape(N, H, W, G, Cg) * s).reshape(ref.shape)
    st = tolerance.compare(f64(yg), om_oracle.gate_forward(ref, V, Z, G), S_g, 4 * P + 2, dt)
    assert st["ok"], ("gate", st)
    # the backward runs end to end in half precision
    xi = x.clone().requires_grad_(True)
    layer(xi).backward(gout)
    torch.cuda.synchronize()
    assert torch.isfinite(xi.grad.float()).all()
