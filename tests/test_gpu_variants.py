"""GPU parity of the kernel variants: remove_center (P = K*K - 1, the centre
tap left out) and DCNv4's packed offset-and-mask record (one (N,Ho,Wo,G*3P)
tensor), through the C ABI's _ex entry points, against the binary64 oracle.

A packed call must also agree bit for bit with the split-layout call on the
same values: both run the same arithmetic and differ only in where the
offsets and mask are read from (grad_input aside, whose order of adds is not
fixed).  The packed cases include records on 2-byte boundaries (half
precision with odd P) and images that start on one (odd Ho*Wo*G).
"""
import sys

import pytest
import torch

import deformable_convolution_core_amd as dcn
import oracle
from deformable_convolution_core_amd import inputs
from tests import tolerance
from tests.test_gpu_parity import DEV, cfg_of, check_backward, check_forward, oracle_bwd, oracle_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def workload(name, N, H, W, G, Cg, K, s, p, d, a, sm, dt, rc, sigma=1.5, backward=False, seed=0):
    Ho, Wo = oracle.out_size(H, K, s, p, d), oracle.out_size(W, K, s, p, d)
    return inputs.Workload(name=name, N=N, H=H, W=W, G=G, Cg=Cg, Ho=Ho, Wo=Wo, K=K, stride=s, pad=p,
                           dilation=d, offset_scale=a, softmax=sm, dtype=dt, offset_sigma=sigma,
                           mask_sigma=1.0 if sm else 0.5, seed_base=seed or 97000 + 37 * len(name),
                           backward=backward, remove_center=rc)


# ------------------------------------------------------------ remove_center
RC_FWD = [  # name, N, H, W, G, Cg, K, stride, pad, dil, alpha, softmax, dtype
    ("rc_k3_f32_softmax", 2, 20, 22, 4, 16, 3, 1, 1, 1, 1.0, True, "f32"),
    ("rc_k3_f16_raw", 2, 56, 56, 4, 16, 3, 1, 1, 1, 1.0, False, "f16"),
    ("rc_k3_bf16_7x7", 3, 7, 7, 32, 16, 3, 1, 1, 1, 1.0, False, "bf16"),
    ("rc_k5_bf16_softmax", 1, 21, 19, 2, 32, 5, 1, 2, 1, 0.8, True, "bf16"),
    ("rc_k7_f32", 1, 15, 17, 2, 16, 7, 1, 3, 1, 1.0, False, "f32"),
    ("rc_k3_s2_d2_f16", 1, 25, 23, 4, 16, 3, 2, 2, 2, 1.2, False, "f16"),
    ("rc_k3_c24_f32_untiled", 1, 9, 11, 3, 8, 3, 1, 1, 1, 1.0, True, "f32"),
    ("rc_k3_c24_f16_untiled", 2, 9, 11, 3, 8, 3, 1, 1, 1, -0.7, False, "f16"),
]


@pytest.mark.parametrize("case", RC_FWD, ids=lambda c: c[0])
def test_remove_center_forward(case):
    check_forward(workload(*case, rc=True))


RC_BWD = [  # name, N, H, W, G, Cg, K, stride, pad, dil, alpha, softmax, dtype, sigma
    ("rcb_k3_f32_softmax", 2, 20, 22, 4, 16, 3, 1, 1, 1, 1.0, True, "f32", 1.5),
    ("rcb_k3_f16", 2, 28, 28, 4, 16, 3, 1, 1, 1, 1.0, False, "f16", 1.5),
    ("rcb_k5_bf16_softmax", 1, 21, 19, 2, 32, 5, 1, 2, 1, 0.8, True, "bf16", 2.0),
    ("rcb_k7_f32", 1, 15, 17, 2, 16, 7, 1, 3, 1, 1.0, False, "f32", 1.5),
    ("rcb_k3_c24_f32_untiled", 1, 9, 11, 3, 8, 3, 1, 1, 1, 1.0, True, "f32", 1.5),
]


@pytest.mark.parametrize("case", RC_BWD, ids=lambda c: c[0])
def test_remove_center_backward(case):
    *geo, sigma = case
    check_backward(workload(*geo, rc=True, sigma=sigma, backward=True))


def test_remove_center_differs_from_full_grid():
    """The centre tap really is dropped: with zero offsets and a mask that
    keeps only the centre point, the full grid returns the input itself; the
    remove_center grid with every weight one sums the eight neighbours only
    (checked against the oracle), which is not the input."""
    N, H, W, G, Cg = 1, 6, 7, 2, 16
    x = torch.randn(N, H, W, G * Cg, device=DEV)
    off9 = torch.zeros(N, H, W, G * 9 * 2, device=DEV)
    m9 = torch.zeros(N, H, W, G, 9, device=DEV)
    m9[..., 4] = 1.0
    full = dcn.forward(x, off9, m9.reshape(N, H, W, G * 9).contiguous(), group=G)
    assert torch.equal(full, x)      # zero offsets: the centre tap reads the pixel itself
    off8 = torch.zeros(N, H, W, G * 8 * 2, device=DEV)
    m8 = torch.ones(N, H, W, G * 8, device=DEV)
    rc = dcn.forward(x, off8, m8, group=G, remove_center=True)
    # the eight neighbours summed with weight one: compare with the oracle
    ref, _ = oracle.forward(x.cpu().double().numpy(), off8.cpu().double().numpy(), m8.cpu().double().numpy(),
                            K=3, stride=1, pad=1, dilation=1, offset_scale=1.0, softmax=False, group=G,
                            remove_center=True)
    assert torch.allclose(rc.cpu().double(), torch.from_numpy(ref), rtol=1e-6, atol=1e-5)
    assert not torch.allclose(rc, full)


# ------------------------------------------------------------- packed layout
PACKED = [  # name, N, H, W, G, Cg, K, stride, pad, dil, alpha, softmax, dtype, remove_center, backward
    ("pk_k3_f16", 2, 24, 20, 4, 16, 3, 1, 1, 1, 1.0, False, "f16", False, True),
    ("pk_k3_bf16_image_lead", 3, 9, 11, 3, 64, 3, 1, 1, 1, 1.0, False, "bf16", False, True),
    ("pk_k3_f16_7x7", 3, 7, 7, 32, 16, 3, 1, 1, 1, 1.0, False, "f16", False, True),
    ("pk_k3_rc_f16", 2, 14, 14, 16, 16, 3, 1, 1, 1, 1.0, False, "f16", True, True),
    ("pk_k5_bf16", 1, 19, 21, 4, 16, 5, 1, 2, 1, 0.9, False, "bf16", False, True),
    ("pk_k5_rc_f16", 1, 19, 21, 4, 16, 5, 1, 2, 1, 0.9, False, "f16", True, True),
    ("pk_k3_f32", 2, 24, 20, 2, 32, 3, 1, 1, 1, 1.0, False, "f32", False, True),
    ("pk_k3_f32_image_lead", 3, 9, 11, 3, 32, 3, 1, 1, 1, 1.0, False, "f32", False, True),
    ("pk_k7_f32_softmax", 1, 15, 17, 2, 16, 7, 1, 3, 1, 1.0, True, "f32", False, True),
    ("pk_k3_s2_bf16_softmax", 2, 25, 23, 4, 16, 3, 2, 1, 1, 1.0, True, "bf16", False, True),
    ("pk_k3_c24_f16_untiled", 2, 9, 11, 3, 8, 3, 1, 1, 1, 1.0, False, "f16", False, False),
    ("pk_k3_c24_f32_untiled", 2, 9, 11, 3, 8, 3, 1, 1, 1, 1.0, False, "f32", False, True),
]


def packed_cfg(w):
    return dict(kernel_size=w.K, stride=w.stride, pad=w.pad, dilation=w.dilation,
                offset_scale=w.offset_scale, softmax=w.softmax, group=w.G, remove_center=w.remove_center)


@pytest.mark.parametrize("case", PACKED, ids=lambda c: c[0])
def test_packed_layout(case):
    *geo, rc, bwd = case
    w = workload(*geo, rc=rc, backward=bwd)
    t = inputs.make(w, with_grad=bwd)
    om = inputs.pack_offset_mask(t["offset"], t["mask"], w.G, w.P)
    d = {k: v.to(DEV) for k, v in t.items()}
    om_d = om.to(DEV)
    out_p = dcn.forward_packed(d["input"], om_d, **packed_cfg(w))
    out_s = dcn.forward(d["input"], d["offset"], d["mask"], **cfg_of(w))
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_s), w.name
    ref, S = oracle_fwd(t, w)
    st = tolerance.compare(out_p.float().cpu().numpy(), ref, S, 4 * w.P, w.dtype)
    assert st["ok"], (w.name, st)
    if not bwd:
        return
    gi_p, gom_p = dcn.backward_packed(d["input"], om_d, d["grad_out"], **packed_cfg(w))
    gi_s, goff_s, gm_s = dcn.backward(d["input"], d["offset"], d["mask"], d["grad_out"], **cfg_of(w))
    torch.cuda.synchronize()
    goff_p, gm_p = inputs.unpack_offset_mask(gom_p, w.G, w.P)
    assert torch.equal(goff_p, goff_s), w.name
    assert torch.equal(gm_p, gm_s), w.name
    r = oracle_bwd(t, w)
    for key, got, S, n, extra in (("grad_input", gi_p, r["gi_abs"], r["gi_cnt"], 0),
                                  ("grad_offset", goff_p, r["goff_abs"], 4 * w.Cg, 0),
                                  ("grad_mask", gm_p, r["gmask_abs"],
                                   4 * w.Cg * (w.P + 1) if w.softmax else 4 * w.Cg, 0)):
        st = tolerance.compare(got.float().cpu().numpy().reshape(r[key].shape), r[key], S, n, w.dtype,
                               store_roundings=extra)
        assert st["ok"], (w.name, key, st)


def test_packed_headline_shape_matches_split():
    """The 56x56 DCNv4 stage in fp16 (N reduced), packed against split."""
    w = inputs.scaled(inputs.WORKLOADS["c2_dcnv4_f16_56"], N=4)
    t = inputs.make(w, with_grad=False)
    om = inputs.pack_offset_mask(t["offset"], t["mask"], w.G, w.P).to(DEV)
    d = {k: v.to(DEV) for k, v in t.items()}
    out_p = dcn.forward_packed(d["input"], om, **packed_cfg(w))
    out_s = dcn.forward(d["input"], d["offset"], d["mask"], **cfg_of(w))
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_s)


def test_dcnv4_autograd_matches_backward_packed():
    w = workload("pk_autograd", 2, 12, 12, 4, 16, 3, 1, 1, 1, 1.0, False, "f32", False, backward=True)
    t = {k: v.to(DEV) for k, v in inputs.make(w, with_grad=True).items()}
    om = inputs.pack_offset_mask(t["offset"], t["mask"], w.G, w.P)
    gi, gom = dcn.backward_packed(t["input"], om, t["grad_out"], **packed_cfg(w))
    xi = t["input"].clone().requires_grad_(True)
    omi = om.clone().requires_grad_(True)
    out = dcn.dcnv4_core(xi, omi, w.K, w.stride, w.pad, w.dilation, w.offset_scale, w.G)
    out.backward(t["grad_out"])
    assert torch.allclose(xi.grad, gi, rtol=1e-5, atol=1e-5)
    assert torch.equal(omi.grad, gom)
