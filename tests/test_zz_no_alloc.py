"""dcn_core_backward_static (the backward for callers that cannot allocate:
its binary32 workspace is the library's static device array) against
dcn_core_backward_ws with a caller-allocated workspace, through the C ABI.

Three half-precision calls in a row share the one array: a large call on
the tiled kernels, a smaller one on the same kernels (its owner tiles start
from the array, so anything left from the first call would show), and a
smaller one on the untiled workspace kernel; then a binary32 call, which
needs no scratch.  grad_offset and grad_mask come from deterministic kernels
and must equal the workspace call's bit for bit; grad_input (summed in an
unfixed order) is compared with the binary64 oracle, element by element, at
the bounds of tests/tolerance.py, for both calls.
"""
import ctypes
import sys

import pytest
import torch

import deformable_convolution_core_amd as dcn
import oracle
from deformable_convolution_core_amd import inputs
from tests import tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def geo(w):
    flags = dcn.FLAG_SOFTMAX if w.softmax else 0
    return (w.N, w.H, w.W, w.G, w.Cg, w.K, w.stride, w.pad, w.dilation, ctypes.c_float(w.offset_scale), flags,
            inputs.DTYPE_CODE[w.dtype])


def run(lib, w, d, static):
    nan = float("nan")
    gi, goff, gm = torch.full_like(d["input"], nan), torch.full_like(d["offset"], nan), torch.full_like(d["mask"], nan)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = (vp(d["input"]), vp(d["offset"]), vp(d["mask"]), vp(d["grad_out"]), vp(gi), vp(goff), vp(gm), *geo(w))
    if static:
        rc = lib.dcn_core_backward_static(*args, stream)
    else:
        need = w.N * w.H * w.W * w.C * 4 if w.dtype != "f32" else 0
        ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=DEV)
        rc = lib.dcn_core_backward_ws(*args, vp(ws) if need else None, need, stream)
    assert rc == 0, lib.dcn_status_string(rc)
    torch.cuda.synchronize()
    return gi, goff, gm


CALLS = [  # name, N, H, W, G, Cg, dtype, softmax, sigma
    ("large_tiled_bf16", 8, 56, 56, 4, 16, "bf16", False, 3.0),
    ("smaller_tiled_f16", 2, 28, 30, 4, 16, "f16", True, 5.0),
    ("smaller_untiled_bf16", 1, 20, 18, 2, 8, "bf16", False, 2.0),
    ("binary32", 2, 24, 24, 4, 16, "f32", False, 2.0),
]


def test_static_scratch_backward_matches_workspace_backward():
    lib = dcn.load_library()
    for k, (name, N, H, W, G, Cg, dt, sm, sigma) in enumerate(CALLS):
        print(f"[gpu-case] no-alloc backward {name}", file=sys.stderr, flush=True)
        w = inputs.Workload(name=name, N=N, H=H, W=W, G=G, Cg=Cg, Ho=H, Wo=W, dtype=dt, softmax=sm,
                            offset_sigma=sigma, mask_sigma=1.0 if sm else 0.5, seed_base=77000 + 100 * k,
                            backward=True)
        t = inputs.make(w, with_grad=True)
        d = {key: v.to(DEV) for key, v in t.items()}
        gi_s, goff_s, gm_s = run(lib, w, d, static=True)
        gi_w, goff_w, gm_w = run(lib, w, d, static=False)
        assert torch.equal(goff_s, goff_w), name
        assert torch.equal(gm_s, gm_w), name
        r = oracle.backward(*(inputs.to_f64(t[key]) for key in ("input", "offset", "mask", "grad_out")),
                            K=3, stride=1, pad=1, dilation=1, offset_scale=1.0, softmax=sm, group=G,
                            coord_mode=oracle.COORD_BINARY32)
        for which, gi in (("static", gi_s), ("workspace", gi_w)):
            st = tolerance.compare(gi.float().cpu().numpy().reshape(r["grad_input"].shape), r["grad_input"],
                                   r["gi_abs"], r["gi_cnt"], dt)
            assert st["ok"], (name, which, st)
        st = tolerance.compare(goff_s.float().cpu().numpy().reshape(r["grad_offset"].shape), r["grad_offset"],
                               r["goff_abs"], 4 * Cg, dt)
        assert st["ok"], (name, "grad_offset", st)
