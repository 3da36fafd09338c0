"""GPU parity of the DCNv4 core with the layer's centre-feature gate fused
into its epilogue (dcn_core_forward_gated), against the binary64 oracle:

    out = y (1 - s) + v s,  y = the sampled result (oracle, binary64),
    v = the input at the output pixel, s = sigmoid(z) per (pixel, group)

bounded element by element as rtol |ref| + (4P + 34) 2^-24 S_out with
S_out = (1 - s) S_y + s |v| (the gate adds two binary32 roundings; y enters
unrounded).  The pre-gate output must equal the plain forward bit for bit,
and the fused output must agree with the two-kernel path (core, then gate)
to the tolerance as well; the autograd wrapper's gradients are compared
with the two-kernel path's autograd."""
import random
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


CASES = [  # name, N, H, W, G, Cg, K, dilation, alpha, remove_center, dtype
    ("g_c2_f16", 4, 56, 56, 4, 16, 3, 1, 1.0, False, "f16"),
    ("g_28_bf16", 2, 28, 28, 8, 16, 3, 1, 1.0, False, "bf16"),
    ("g_7_bf16_whole", 3, 7, 7, 32, 16, 3, 1, 1.0, False, "bf16"),
    ("g_f32_rc", 2, 20, 22, 4, 16, 3, 1, 0.8, True, "f32"),
    ("g_k5_d2_f16", 1, 19, 21, 2, 32, 5, 2, 1.0, False, "f16"),
    ("g_k7_f32", 1, 15, 17, 2, 32, 7, 1, 1.0, False, "f32"),
]


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_gated_forward_matches_oracle(case):
    check_gated(*case)


def draw_gated(case):
    """Seeded random shape the fused kernel serves: group rows of 32, 64 or
    128 bytes, channel rows a multiple of 128 bytes, odd K, dilation 1-2,
    offset_scale of either sign, remove_center, any dtype."""
    r = random.Random(97000 + 389 * case)
    dt = r.choice(["f32", "f16", "bf16"])
    b = 4 if dt == "f32" else 2
    Cg = r.choice([32, 64, 128]) // b
    G = r.choice([g for g in (1, 2, 3, 4, 6, 8) if (g * Cg * b) % 128 == 0])
    K = r.choice([1, 3, 3, 5, 7])
    d = r.choice([1, 1, 2])
    return (f"rand{case}", r.choice([1, 2]), r.randint(1, 24), r.randint(1, 24), G, Cg, K, d,
            r.choice([1.0, 0.6, -1.3]), K >= 3 and r.random() < 0.3, dt)


@pytest.mark.parametrize("case", range(24))
def test_gated_forward_random_shapes(case):
    check_gated(*draw_gated(case))


def check_gated(name, N, H, W, G, Cg, K, d, alpha, rc, dt):
    pad = d * (K - 1) // 2
    w = inputs.Workload(name=name, N=N, H=H, W=W, G=G, Cg=Cg, Ho=H, Wo=W, K=K, stride=1, pad=pad, dilation=d,
                        offset_scale=alpha, softmax=False, dtype=dt, offset_sigma=1.5, mask_sigma=0.5,
                        seed_base=96000 + 13 * len(name), remove_center=rc)
    t = inputs.make(w, with_grad=False)
    z = inputs.normal((N, H, W, G), w.seed_base + 9, 2.0, dt)
    om = inputs.pack_offset_mask(t["offset"], t["mask"], G, w.P)
    x_d, om_d, z_d = t["input"].to(DEV), om.to(DEV), z.to(DEV)
    kw = dict(kernel_size=K, dilation=d, offset_scale=alpha, group=G, remove_center=rc)
    out, core = dcn.forward_packed_gated(x_d, om_d, z_d, keep_core_output=True, **kw)
    plain = dcn.forward_packed(x_d, om_d, stride=1, pad=pad, **kw)
    two = dcn.center_gate_forward(plain, x_d, z_d, group=G)
    out_nc, none = dcn.forward_packed_gated(x_d, om_d, z_d, **kw)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(core, plain), name
    assert torch.equal(out_nc, out), name
    y, S = oracle.forward(inputs.to_f64(t["input"]), inputs.to_f64(t["offset"]), inputs.to_f64(t["mask"]), K=K,
                          stride=1, pad=pad, dilation=d, offset_scale=alpha, softmax=False, group=G,
                          coord_mode=oracle.COORD_BINARY32, remove_center=rc)
    s = sigmoid(inputs.to_f64(z))[..., :, None]
    v = inputs.to_f64(t["input"]).reshape(N, H, W, G, Cg)
    ref = (y.reshape(N, H, W, G, Cg) * (1 - s) + v * s).reshape(N, H, W, G * Cg)
    S_out = (S.reshape(N, H, W, G, Cg) * (1 - s) + np.abs(v) * s).reshape(N, H, W, G * Cg)
    st = tolerance.compare(out.float().cpu().numpy(), ref, S_out, 4 * w.P + 2, dt)
    assert st["ok"], (name, "fused", st)
    # the two-kernel path rounds y to the dtype before the gate: one more rounding
    st = tolerance.compare(two.float().cpu().numpy(), ref, S_out, 4 * w.P + 2, dt, store_roundings=1)
    assert st["ok"], (name, "two kernels", st)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gated_autograd_matches_two_kernels(dt):
    N, H, W, G, Cg, K = 2, 12, 13, 4, 16, 3
    T = inputs.DTYPES[dt]
    P = K * K
    x = inputs.normal((N, H, W, G * Cg), 5101, 1.0, dt).to(DEV)
    om = inputs.normal((N, H, W, G * 3 * P), 5102, 1.0, dt).to(DEV)
    z = inputs.normal((N, H, W, G), 5103, 1.0, dt).to(DEV)
    g = inputs.normal((N, H, W, G * Cg), 5104, 1.0, dt).to(DEV)
    leaves = [t.clone().requires_grad_(True) for t in (x, om, z)]
    out = dcn.DCNv4GatedFunction.apply(*leaves, K, 1, 1.0, G, False)
    out.backward(g)
    leaves2 = [t.clone().requires_grad_(True) for t in (x, om, z)]
    y = dcn.dcnv4_core(leaves2[0], leaves2[1], K, 1, 1, 1, 1.0, G)
    out2 = dcn.center_gate(y, leaves2[0], leaves2[2], G)
    out2.backward(g)
    torch.cuda.synchronize()
    # the gate's backward reads the same rounded y on both paths; the core's
    # grad_input atomics may add in another order
    for a, b, name in zip(leaves, leaves2, ("input", "offset_mask", "logits")):
        ga, gb = a.grad.float(), b.grad.float()
        tol = 1e-5 if dt == "f32" else 2e-2
        assert torch.allclose(ga, gb, rtol=tol, atol=tol * float(gb.abs().max())), name
    o1, o2 = out.detach().float(), out2.detach().float()
    assert torch.allclose(o1, o2, rtol=1e-5 if dt == "f32" else 1e-2,
                          atol=(1e-6 if dt == "f32" else 1e-2) * float(o2.abs().max()))


def test_gated_unsupported_shapes_say_so():
    x = torch.randn(1, 8, 8, 24, device=DEV)            # C = 24: no tiled plan
    om = torch.randn(1, 8, 8, 3 * 27, device=DEV)
    z = torch.randn(1, 8, 8, 3, device=DEV)
    with pytest.raises(dcn.DCNError) as e:
        dcn.forward_packed_gated(x, om, z, group=3)
    assert e.value.status == 2
