"""GPU parity of the two plain C entry points, dcn_core_forward and
dcn_core_backward, called through ctypes with raw device pointers, the
argument list of the core ("没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读",
section 4: input, offset, mask, kernel size, stride, pad, dilation, group,
group channels, offset scale; the mask softmax of section 3 as a flag).

The binding and the other tests go through the _ex/_ws entry points; these
cases make the plain calls compute on the GPU and compare every element with
the binary64 oracle: DCNv3 with softmax (the 8x8 fp32 workload), DCNv4 with
a raw mask (the 56x56 fp32 workload at full size, forward and backward), and
the bf16 forwards of the 56x56 stage and the stride-2 DCNv3 stage.
"""
import ctypes
import sys

import pytest
import torch

import deformable_convolution_core_amd as dcn
from deformable_convolution_core_amd import inputs
from tests import tolerance
from tests.test_gpu_parity import DEV, oracle_bwd, oracle_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def vp(t):
    return ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def geo_args(w):
    return (w.N, w.H, w.W, w.G, w.Cg, w.K, w.stride, w.pad, w.dilation, ctypes.c_float(w.offset_scale),
            int(w.softmax), inputs.DTYPE_CODE[w.dtype])


@pytest.mark.parametrize("name", ["c1_dcnv3_f32_8x8", "c5_dcnv4_f32_56_fwdbwd", "c3a_dcnv4_bf16_56",
                                  "c4s2_dcnv3_bf16_128"])
def test_plain_forward(name):
    w = inputs.WORKLOADS[name]
    t = inputs.make(w, with_grad=False)
    d = {k: v.to(DEV) for k, v in t.items()}
    out = torch.full(w.shapes()["output"], float("nan"), dtype=d["input"].dtype, device=DEV)
    lib = dcn.load_library()
    rc = lib.dcn_core_forward(vp(d["input"]), vp(d["offset"]), vp(d["mask"]), vp(out), *geo_args(w), stream())
    assert rc == 0, lib.dcn_status_string(rc)
    torch.cuda.synchronize()
    ref, S = oracle_fwd(t, w)
    st = tolerance.compare(out.float().cpu().numpy(), ref, S, 4 * w.P, w.dtype)
    assert st["ok"], (name, st)


@pytest.mark.parametrize("name", ["c1_dcnv3_f32_8x8", "c5_dcnv4_f32_56_fwdbwd"])
def test_plain_backward(name):
    w = inputs.WORKLOADS[name]
    t = inputs.make(w, with_grad=True)
    d = {k: v.to(DEV) for k, v in t.items()}
    nan = float("nan")
    gi = torch.full_like(d["input"], nan)
    goff = torch.full_like(d["offset"], nan)
    gm = torch.full_like(d["mask"], nan)
    lib = dcn.load_library()
    rc = lib.dcn_core_backward(vp(d["input"]), vp(d["offset"]), vp(d["mask"]), vp(d["grad_out"]), vp(gi), vp(goff),
                               vp(gm), *geo_args(w), stream())
    assert rc == 0, lib.dcn_status_string(rc)
    torch.cuda.synchronize()
    r = oracle_bwd(t, w)
    for key, got, S, n in (("grad_input", gi, r["gi_abs"], r["gi_cnt"]),
                           ("grad_offset", goff, r["goff_abs"], 4 * w.Cg),
                           ("grad_mask", gm, r["gmask_abs"], 4 * w.Cg * (w.P + 1) if w.softmax else 4 * w.Cg)):
        st = tolerance.compare(got.float().cpu().numpy().reshape(r[key].shape), r[key], S, n, w.dtype)
        assert st["ok"], (name, key, st)
