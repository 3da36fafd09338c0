"""GPU parity of the DCNv4 layer around the core: the centre-feature gate
kernel against the float64 gate of the layer oracle (element by element),
and the whole layer (projections + HIP core + HIP gate), forward and
backward, checked stage by stage.

The layer's projections round (in binary32 or half precision), and that
rounding moves the sampling coordinates, so the layer's output has no
per-element sum of terms to bound its distance from an all-float64 layer.
Instead each stage is checked on the layer's own intermediates:

* the layer's output and every gradient equal the same package calls made
  stage by stage here (bit for bit where the order of additions is fixed,
  else within one rounding per addition), so the stages are the layer's;
* each stage -- the four projections and their input, weight and bias
  gradients, the sampling core and its backward, the gate and its backward
  -- matches its float64 definition (oracle/module.py's linear and gate
  formulas, the C oracle for the core) evaluated on that stage's own inputs,
  element by element to the bounds of tests/tolerance.py.
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
    check_layer_stages(case, "f32", seed)


def _proj_bw(g, a, lin, dt):
    """The _Projection backward the layer runs: input gradient g @ W and the
    weight and bias gradients (the package's kernels, or their fallbacks)."""
    from deformable_convolution_core_amd.layer import _matmul_t, _param_grads
    g2 = g.reshape(-1, g.shape[-1]).contiguous()
    gx = _matmul_t(g2, lin.weight.t().contiguous()).view(a.shape)
    gw, gb = _param_grads(g2, a.reshape(-1, a.shape[-1]), True, True)
    return gx, gw, gb


def layer_stages(layer, x, gout, core_backward):
    """The layer's forward and backward as the package calls it makes, stage
    by stage (the same calls as DCNv4.forward and the autograd functions'
    backward), keeping every intermediate.  core_backward: the (gi, gom) the
    layer's own backward got from the core -- its grad_input is summed in an
    unfixed order, so a second call would differ in the last bits."""
    from deformable_convolution_core_amd.layer import _matmul_t
    K, G, P = layer.kernel_size, layer.group, dcn.points(layer.kernel_size, layer.remove_center)
    kw = dict(kernel_size=K, dilation=layer.dilation, offset_scale=layer.offset_scale, group=G,
              remove_center=layer.remove_center)
    st = dict(x=x)
    st["v"] = _matmul_t(x, layer.value_proj.weight, layer.value_proj.bias)
    st["om"] = _matmul_t(x, layer.offset_mask.weight, layer.offset_mask.bias)
    gate = layer.center_feature_scale_proj is not None
    fused = False
    if gate:
        st["z"] = _matmul_t(x, layer.center_feature_scale_proj.weight, layer.center_feature_scale_proj.bias)
        try:
            st["yg"], st["y"] = dcn.forward_packed_gated(st["v"], st["om"], st["z"], keep_core_output=True, **kw)
            fused = True
        except dcn.DCNError as e:
            assert e.status == 2
            st["y"] = dcn.forward_packed(st["v"], st["om"], stride=1, pad=layer.pad, **kw)
            st["yg"] = dcn.center_gate_forward(st["y"], st["v"], st["z"], group=G)
    else:
        st["y"] = dcn.forward_packed(st["v"], st["om"], stride=1, pad=layer.pad, **kw)
        st["yg"] = st["y"]
    st["out"] = _matmul_t(st["yg"], layer.output_proj.weight, layer.output_proj.bias)
    # backward, stage by stage
    st["g_yg"], st["dWo"], st["dbo"] = _proj_bw(gout, st["yg"], layer.output_proj, x.dtype)
    if gate:
        st["g_y"], st["gv_gate"], st["gz"] = dcn.center_gate_backward(st["y"], st["v"], st["z"], st["g_yg"],
                                                                     group=G)
    else:
        st["g_y"] = st["g_yg"]
    st["gi"], st["gom"] = core_backward
    st["gv"] = st["gi"] + st["gv_gate"] if gate else st["gi"]
    st["gx_v"], st["dWv"], st["dbv"] = _proj_bw(st["gv"], x, layer.value_proj, x.dtype)
    st["gx_om"], st["dWom"], st["dbom"] = _proj_bw(st["gom"], x, layer.offset_mask, x.dtype)
    if gate:
        st["gx_z"], st["dWc"], st["dbc"] = _proj_bw(st["gz"], x, layer.center_feature_scale_proj, x.dtype)
    st["fused"] = fused
    st["P"] = P
    return st


def check_projection(out, a, W, b, dt, what):
    """out = a @ W.T + b against float64 on the same (rounded) operands."""
    A, Wt = f64(a).reshape(-1, a.shape[-1]), f64(W)
    ref = A @ Wt.T + (0.0 if b is None else f64(b))
    S = np.abs(A) @ np.abs(Wt).T + (0.0 if b is None else np.abs(f64(b)))
    st = tolerance.compare(f64(out).reshape(ref.shape), ref, S, A.shape[1] + 1, dt)
    assert st["ok"], (what, st)


def check_param_grads(dW, db, g, a, dt, what):
    """dW = g^T a and db = sum of g over rows, against float64."""
    G2, A2 = f64(g).reshape(-1, g.shape[-1]), f64(a).reshape(-1, a.shape[-1])
    ref, S = G2.T @ A2, np.abs(G2).T @ np.abs(A2)
    st = tolerance.compare(f64(dW), ref, S, G2.shape[0], dt)
    assert st["ok"], (what + " weight", st)
    st = tolerance.compare(f64(db), G2.sum(0), np.abs(G2).sum(0), G2.shape[0], dt)
    assert st["ok"], (what + " bias", st)


def check_layer_stages(case, dt, seed):
    # platform-BLAS fallbacks (shapes the package's GEMM declines) accumulate
    # in binary32 here, as the bounds assume
    mm = torch.backends.cuda.matmul
    saved = (mm.allow_fp16_reduced_precision_reduction, mm.allow_bf16_reduced_precision_reduction)
    mm.allow_fp16_reduced_precision_reduction = False
    mm.allow_bf16_reduced_precision_reduction = False
    try:
        _check_layer_stages(case, dt, seed)
    finally:
        mm.allow_fp16_reduced_precision_reduction, mm.allow_bf16_reduced_precision_reduction = saved


def _check_layer_stages(case, dt, seed):
    N, H, W, G, Cg, K, rc, cfs, alpha = case
    layer, x, gout = make_layer(*case, dt, seed)
    xi = x.clone().requires_grad_(True)
    out = layer(xi)
    # the layer's backward calls the core's backward once: keep what it returns
    calls = []
    orig = dcn.backward_packed

    def recording(*a, **k):
        r = orig(*a, **k)
        calls.append((a, k, r))
        return r
    dcn.backward_packed = recording
    try:
        out.backward(gout)
    finally:
        dcn.backward_packed = orig
    torch.cuda.synchronize()
    assert len(calls) == 1
    with torch.no_grad():
        st = layer_stages(layer, x, gout, calls[0][2])
    torch.cuda.synchronize()
    # the core's backward got the stage-wise upstream gradient and inputs
    a, k, _ = calls[0]
    assert torch.equal(a[0], st["v"]) and torch.equal(a[1], st["om"]) and torch.equal(a[2], st["g_y"])
    name = f"{case} {dt}"
    # the stages are the layer's: output and parameter gradients bit for bit
    assert torch.equal(out, st["out"]), name
    pg = [("Wo", layer.output_proj, "dWo", "dbo"), ("Wv", layer.value_proj, "dWv", "dbv"),
          ("Wom", layer.offset_mask, "dWom", "dbom")]
    if cfs:
        pg.append(("Wc", layer.center_feature_scale_proj, "dWc", "dbc"))
    for nm, lin, kw_, kb in pg:
        assert torch.equal(lin.weight.grad, st[kw_]), (name, nm)
        assert torch.equal(lin.bias.grad, st[kb]), (name, nm)
    # the input gradient: autograd adds the projections' three (or two)
    # input gradients in its own order, one rounding per addition
    parts = [st["gx_v"], st["gx_om"]] + ([st["gx_z"]] if cfs else [])
    ref = sum(f64(t) for t in parts)
    S = sum(np.abs(f64(t)) for t in parts)
    s_ = tolerance.compare(f64(xi.grad), ref, S, len(parts), dt, store_roundings=len(parts) - 1)
    assert s_["ok"], (name, "input gradient sum", s_)
    # each stage against its float64 definition on its own inputs
    P = st["P"]
    check_projection(st["v"], x, layer.value_proj.weight, layer.value_proj.bias, dt, "value projection")
    check_projection(st["om"], x, layer.offset_mask.weight, layer.offset_mask.bias, dt, "offset+mask projection")
    check_projection(st["out"], st["yg"], layer.output_proj.weight, layer.output_proj.bias, dt, "output projection")
    core_kw = dict(K=K, stride=1, pad=layer.pad, dilation=1, offset_scale=alpha, softmax=False, group=G,
                   coord_mode=oracle.COORD_BINARY32, remove_center=rc)
    off, mask = inputs.unpack_offset_mask(st["om"].cpu(), G, P)
    yref, S = oracle.forward(f64(st["v"]), f64(off), f64(mask), **core_kw)
    s_ = tolerance.compare(f64(st["y"]), yref, S, 4 * P, dt)
    assert s_["ok"], (name, "core", s_)
    V = f64(st["v"])
    if cfs:
        check_projection(st["z"], x, layer.center_feature_scale_proj.weight, layer.center_feature_scale_proj.bias,
                         dt, "gate projection")
        Z = f64(st["z"])
        s, t = om_oracle.sigmoid(Z)[..., None], om_oracle.sigmoid(-Z)[..., None]
        # the fused gate takes the unrounded core result, the two-kernel gate the rounded one
        Y = yref if st["fused"] else f64(st["y"])
        SY = S if st["fused"] else np.abs(Y)
        S_g = (SY.reshape(N, H, W, G, Cg) * t + np.abs(V).reshape(N, H, W, G, Cg) * s).reshape(Y.shape)
        s_ = tolerance.compare(f64(st["yg"]), om_oracle.gate_forward(Y, V, Z, G), S_g, 4 * P + 2, dt,
                               store_roundings=0 if st["fused"] else 1)
        assert s_["ok"], (name, "gate", s_)
    # backward stages
    check_projection(st["g_yg"], gout, layer.output_proj.weight.t(), None, dt, "output projection input grad")
    check_param_grads(st["dWo"], st["dbo"], gout, st["yg"], dt, "output projection")
    if cfs:
        Y, GO = f64(st["y"]), f64(st["g_yg"])
        gy, gv, gz = om_oracle.gate_backward(Y, V, Z, GO, G)
        go5 = np.abs(GO).reshape(N, H, W, G, Cg)
        s_ = tolerance.compare(f64(st["g_y"]), gy, np.abs(gy), 1, dt)
        assert s_["ok"], (name, "gate backward: grad of y", s_)
        s_ = tolerance.compare(f64(st["gv_gate"]), gv, np.abs(gv), 1, dt)
        assert s_["ok"], (name, "gate backward: grad of v", s_)
        Sz = (go5 * (np.abs(V) + np.abs(Y)).reshape(go5.shape)).sum(-1) * (s[..., 0] * t[..., 0])
        s_ = tolerance.compare(f64(st["gz"]), gz, Sz, Cg + 4, dt)
        assert s_["ok"], (name, "gate backward: grad of the logits", s_)
    r = oracle.backward(f64(st["v"]), f64(off), f64(mask), f64(st["g_y"]), **core_kw)
    s_ = tolerance.compare(f64(st["gi"]).reshape(r["grad_input"].shape), r["grad_input"], r["gi_abs"], r["gi_cnt"], dt)
    assert s_["ok"], (name, "core backward: grad of v", s_)
    goff, gmask = inputs.unpack_offset_mask(st["gom"].cpu(), G, P)
    s_ = tolerance.compare(f64(goff).reshape(r["grad_offset"].shape), r["grad_offset"], r["goff_abs"], 4 * Cg, dt)
    assert s_["ok"], (name, "core backward: grad of the offsets", s_)
    s_ = tolerance.compare(f64(gmask).reshape(r["grad_mask"].shape), r["grad_mask"], r["gmask_abs"], 4 * Cg, dt)
    assert s_["ok"], (name, "core backward: grad of the mask", s_)
    if cfs:
        s_ = tolerance.compare(f64(st["gv"]), f64(st["gi"]) + f64(st["gv_gate"]),
                               np.abs(f64(st["gi"])) + np.abs(f64(st["gv_gate"])), 2, dt)
        assert s_["ok"], (name, "grad of v: core + gate", s_)
    for g, lin, a, what in ((st["gv"], layer.value_proj, x, "value"), (st["gom"], layer.offset_mask, x, "offset+mask")) \
            + (((st["gz"], layer.center_feature_scale_proj, x, "gate"),) if cfs else ()):
        gx = {"value": st["gx_v"], "offset+mask": st["gx_om"], "gate": st.get("gx_z")}[what]
        check_projection(gx, g, lin.weight.t(), None, dt, what + " projection input grad")
        dW, db = {"value": (st["dWv"], st["dbv"]), "offset+mask": (st["dWom"], st["dbom"]),
                  "gate": (st.get("dWc"), st.get("dbc"))}[what]
        check_param_grads(dW, db, g, a, dt, what + " projection")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("case", [(2, 14, 14, 4, 16, 3, False, True, 1.0), (1, 12, 11, 4, 16, 3, True, False, 0.8),
                                  (1, 9, 10, 3, 8, 3, False, True, 1.0)],
                         ids=["gated", "rc_nogate", "two_kernel_gate"])
def test_layer_half_stagewise(case, dt):
    """Half precision, forward and backward, every stage element by element
    on the layer's own intermediates (C = 24 runs the core and the gate as
    two kernels)."""
    check_layer_stages(case, dt, 6400 + case[1])
