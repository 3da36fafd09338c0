"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, computes output sizes, and rejects invalid calls on the host
before any HIP call (no valid compute call is made here)."""
import ctypes
import math
import os
import re

import pytest
import torch

import deformable_convolution_core_amd as dcn
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcn_core.h")
OK, INVALID, UNSUPPORTED = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = dcn.load_library()
    names = declared_functions()
    assert set(names) == set(dcn.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_out_size_matches_oracle():
    for n in (1, 2, 3, 7, 8, 14, 56, 128):
        for K in (1, 2, 3, 5, 7):
            for s in (1, 2, 3):
                for p in (0, 1, 2, 3):
                    for d in (1, 2):
                        assert dcn.out_size(n, K, s, p, d) == oracle.out_size(n, K, s, p, d)
    assert dcn.out_size(0, 3, 1, 1, 1) <= 0
    assert dcn.out_size(8, 0, 1, 1, 1) <= 0
    assert dcn.out_size(8, 3, 0, 1, 1) <= 0
    assert dcn.out_size(8, 3, 1, -1, 1) <= 0
    assert dcn.out_size(8, 3, 1, 1, 0) <= 0
    assert dcn.out_size(2, 5, 1, 0, 1) <= 0   # window larger than the padded map


def fwd(lib, ptrs=(0x1000, 0x2000, 0x3000, 0x4000), N=1, H=8, W=8, G=2, Cg=8, K=3, s=1, p=1, d=1,
        alpha=1.0, softmax=0, dtype=0):
    vp = [ctypes.c_void_p(x) if x else None for x in ptrs]
    return lib.dcn_core_forward(*vp, N, H, W, G, Cg, K, s, p, d, alpha, softmax, dtype, None)


def bwd(lib, N=1, H=8, W=8, G=2, Cg=8, K=3, s=1, p=1, d=1, alpha=1.0, softmax=0, dtype=0, null=False):
    vp = [None if null else ctypes.c_void_p(0x1000 * (i + 1)) for i in range(7)]
    return lib.dcn_core_backward(*vp, N, H, W, G, Cg, K, s, p, d, alpha, softmax, dtype, None)


INVALID_FWD = [
    dict(N=-1), dict(H=0), dict(W=-3), dict(G=0), dict(Cg=0), dict(K=0), dict(s=0), dict(d=0),
    dict(p=-1), dict(dtype=3), dict(dtype=-1), dict(softmax=2), dict(alpha=float("nan")),
    dict(alpha=float("inf")), dict(H=2, W=2, K=5, p=0),       # empty output grid
    dict(ptrs=(0, 0x2000, 0x3000, 0x4000)), dict(ptrs=(0x1000, 0, 0x3000, 0x4000)),
    dict(ptrs=(0x1000, 0x2000, 0, 0x4000)), dict(ptrs=(0x1000, 0x2000, 0x3000, 0)),
    dict(ptrs=(0x1000, 0x2002, 0x3000, 0x4000), dtype=1),   # offset pair not 4-byte aligned (f16)
    dict(ptrs=(0x1000, 0x2004, 0x3000, 0x4000), dtype=0),   # offset pair not 8-byte aligned (f32)
    dict(ptrs=(0x1000, 0x2000, 0x3001, 0x4000), dtype=2),   # mask not element aligned
    dict(ptrs=(0x1001, 0x2000, 0x3000, 0x4000), dtype=0),   # input not element aligned
    dict(ptrs=(0x1000, 0x2000, 0x3000, 0x4003), dtype=0),   # output not element aligned
]


@pytest.mark.parametrize("kw", INVALID_FWD)
def test_forward_rejects_invalid_arguments_on_host(kw):
    assert fwd(dcn.load_library(), **kw) == INVALID


@pytest.mark.parametrize("kw", [dict(K=17, H=40, W=40, p=8), dict(N=1, H=40000, W=40000, G=1, Cg=8),
                                dict(N=1, H=8, W=8, G=1 << 20, Cg=1 << 12),
                                # one pixel row past the largest image the GPU tests run (1448 x 1448 x 512 bf16)
                                dict(N=1, H=1449, W=1449, G=16, Cg=32, dtype=2)])
def test_forward_unsupported_sizes(kw):
    assert fwd(dcn.load_library(), **kw) == UNSUPPORTED


def test_forward_empty_batch_is_noop():
    lib = dcn.load_library()
    assert fwd(lib, N=0) == OK
    assert fwd(lib, N=0, ptrs=(0, 0, 0, 0)) == OK


def test_gated_forward_validation():
    lib = dcn.load_library()
    vp = ctypes.c_void_p
    p = [vp(0x10000 * (i + 1)) for i in range(6)]
    geo = [1, 8, 8, 4, 16]
    one = ctypes.c_float(1.0)
    PK = 4                                                      # packed record flag
    # K even, stride 2, pad off-centre, softmax: not the layer's geometry
    assert lib.dcn_core_forward_gated(p[0], p[1], None, p[3], p[4], None, *geo, 4, 1, 1, 1, one, PK, 0, None) == UNSUPPORTED
    assert lib.dcn_core_forward_gated(p[0], p[1], None, p[3], p[4], None, *geo, 3, 2, 1, 1, one, PK, 0, None) == UNSUPPORTED
    assert lib.dcn_core_forward_gated(p[0], p[1], None, p[3], p[4], None, *geo, 3, 1, 0, 1, one, PK, 0, None) == UNSUPPORTED
    assert lib.dcn_core_forward_gated(p[0], p[1], None, p[3], p[4], None, *geo, 3, 1, 1, 1, one, PK | 1, 0, None) == UNSUPPORTED
    # no logits, misaligned logits or pre-gate output
    assert lib.dcn_core_forward_gated(p[0], p[1], None, None, p[4], None, *geo, 3, 1, 1, 1, one, PK, 0, None) == INVALID
    assert lib.dcn_core_forward_gated(p[0], p[1], None, vp(0x30001), p[4], None, *geo, 3, 1, 1, 1, one, PK, 1, None) == INVALID
    assert lib.dcn_core_forward_gated(p[0], p[1], None, p[3], p[4], vp(0x50008), *geo, 3, 1, 1, 1, one, PK, 0, None) == INVALID
    # an empty batch is a no-op
    assert lib.dcn_core_forward_gated(None, None, None, None, None, None, 0, 8, 8, 4, 16, 3, 1, 1, 1, one, PK, 0, None) == OK


def test_weight_grad_entry_points():
    lib = dcn.load_library()
    vp = ctypes.c_void_p
    assert lib.dcn_linear_weight_grad_workspace_size(0, 8, 8) == 0
    assert lib.dcn_linear_weight_grad_workspace_size(-1, 8, 8) == -INVALID
    assert lib.dcn_linear_weight_grad_workspace_size(10, 0, 8) == -INVALID
    # partials of every chunk: at least one 128 x (64 + 16) binary32 block, and
    # more rows never need fewer chunks
    small = lib.dcn_linear_weight_grad_workspace_size(64, 108, 64)
    big = lib.dcn_linear_weight_grad_workspace_size(200704, 108, 64)
    assert small >= 128 * 80 * 4 and big >= small and big % 16 == 0
    p = [vp(0x10000), vp(0x20000), vp(0x30000), vp(0x40000)]
    ws = vp(0x100000)
    assert lib.dcn_linear_weight_grad(*p, 64, 8, 8, 7, 0, ws, 1 << 20, None) == INVALID         # dtype
    assert lib.dcn_linear_weight_grad(*p, 64, 8, 8, 0, 3, ws, 1 << 20, None) == INVALID         # out_dtype
    assert lib.dcn_linear_weight_grad(*p, 64, 8, 8, 0, -1, ws, 1 << 20, None) == INVALID
    assert lib.dcn_linear_weight_grad(*p, -1, 8, 8, 0, 0, ws, 1 << 20, None) == INVALID         # M
    assert lib.dcn_linear_weight_grad(p[0], p[1], None, None, 64, 8, 8, 0, 0, ws, 1 << 20, None) == INVALID
    assert lib.dcn_linear_weight_grad(*p, 64, 8, 8, 0, 0, None, 0, None) == INVALID            # no workspace
    need = lib.dcn_linear_weight_grad_workspace_size(64, 8, 8)
    assert lib.dcn_linear_weight_grad(*p, 64, 8, 8, 0, 0, ws, need - 1, None) == INVALID       # too small
    assert lib.dcn_linear_weight_grad(*p, 64, 8, 8, 0, 0, vp(0x100008), need, None) == INVALID # misaligned
    assert lib.dcn_linear_weight_grad(vp(0x10001), p[1], p[2], p[3], 64, 8, 8, 1, 0, ws, need, None) == INVALID
    # outputs aligned to their own element: 2-byte dw is fine in half precision, not in binary32
    assert lib.dcn_linear_weight_grad(p[0], p[1], vp(0x30002), p[3], 64, 8, 8, 0, 0, ws, need, None) == INVALID
    assert lib.dcn_linear_weight_grad(p[0], p[1], vp(0x30001), p[3], 64, 8, 8, 0, 1, ws, need, None) == INVALID


def test_backward_workspace_entry_points():
    lib = dcn.load_library()
    vp = ctypes.c_void_p
    p3 = [vp(0x1000), vp(0x2000), vp(0x3000)]
    geo = (1, 8, 8, 2, 8, 3, 1, 1, 1, ctypes.c_float(1.0), 0)
    assert lib.dcn_core_backward_workspace_size(*p3, *geo, 0) == 0            # binary32 needs none
    assert lib.dcn_core_backward_workspace_size(*p3, *geo, 1) == 8 * 8 * 16 * 4   # C = 16 half
    geo64 = (2, 8, 8, 4, 16, 3, 1, 1, 1, ctypes.c_float(1.0), 0)
    assert lib.dcn_core_backward_workspace_size(*p3, *geo64, 2) == 2 * 8 * 8 * 64 * 4   # tiled half too
    assert lib.dcn_core_backward_workspace_size(*p3, *geo64, 0) == 0
    assert lib.dcn_core_backward_workspace_size(*p3, 1, 8, 8, 2, 8, 0, 1, 1, 1, ctypes.c_float(1.0), 0, 1) == -1
    ptrs = [vp(0x1000 * (i + 1)) for i in range(7)]
    ws = vp(0x100000)
    args = (1, 8, 8, 2, 8, 3, 1, 1, 1, ctypes.c_float(1.0), 0, 1)
    assert lib.dcn_core_backward_ws(*ptrs, *args, ws, 8 * 8 * 16 * 4 - 4, None) == INVALID   # too small
    assert lib.dcn_core_backward_ws(*ptrs, *args, vp(0x100002), 8 * 8 * 16 * 4, None) == INVALID   # misaligned
    assert lib.dcn_core_backward_ws(*ptrs, *args, vp(0x100008), 8 * 8 * 16 * 4, None) == INVALID   # not 16-byte
    assert lib.dcn_core_backward_ws(*ptrs, *args, None, 0, None) == UNSUPPORTED   # needs one, none given
    assert lib.dcn_core_backward_ws(*ptrs, *args, ws, -1, None) == INVALID


def test_backward_validation():
    lib = dcn.load_library()
    # half precision sums grad_input in a binary32 workspace, which only
    # dcn_core_backward_ws takes: the plain call declines fp16 and bf16,
    # on the tiled channel widths (C = 64) as well
    assert bwd(lib, dtype=1) == UNSUPPORTED
    assert bwd(lib, dtype=2) == UNSUPPORTED
    assert bwd(lib, dtype=1, G=4, Cg=16) == UNSUPPORTED
    assert bwd(lib, dtype=2, G=4, Cg=16) == UNSUPPORTED
    assert bwd(lib, K=0) == INVALID
    assert bwd(lib, null=True) == INVALID
    assert bwd(lib, N=0, null=True) == OK
    assert bwd(lib, Cg=12) == UNSUPPORTED    # lanes per group would not be a power of two
    assert bwd(lib, Cg=3) == UNSUPPORTED


def fwd_ex(lib, ptrs=(0x1000, 0x2000, 0x3000, 0x4000), N=1, H=8, W=8, G=2, Cg=8, K=3, s=1, p=1, d=1,
           alpha=1.0, flags=0, dtype=0):
    vp = [ctypes.c_void_p(x) if x else None for x in ptrs]
    return lib.dcn_core_forward_ex(*vp, N, H, W, G, Cg, K, s, p, d, alpha, flags, dtype, None)


def bwd_ex(lib, ptrs=(0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000), N=1, H=8, W=8, G=2, Cg=8,
           K=3, s=1, p=1, d=1, alpha=1.0, flags=0, dtype=0):
    vp = [ctypes.c_void_p(x) if x else None for x in ptrs]
    return lib.dcn_core_backward_ex(*vp, N, H, W, G, Cg, K, s, p, d, alpha, flags, dtype, None)


PACKED_PTRS = (0x1000, 0x2000, 0, 0x4000)
INVALID_EX = [
    dict(flags=8), dict(flags=-1), dict(flags=1 << 30),
    dict(flags=2, K=4, p=1),                     # remove_center needs an odd K
    dict(flags=2, K=2, p=0), dict(flags=2, K=1, p=0),
    dict(flags=4),                               # packed with a separate mask pointer
    dict(flags=4, ptrs=(0x1000, 0x2002, 0, 0x4000), dtype=1),   # packed tensor on a 2-byte boundary
    dict(flags=4, ptrs=(0x1000, 0, 0, 0x4000)),  # packed without the tensor
    dict(flags=0, ptrs=(0x1000, 0x2000, 0, 0x4000)),            # split layout without a mask
    dict(flags=2, dtype=5), dict(flags=2, N=-1),
]


@pytest.mark.parametrize("kw", INVALID_EX)
def test_forward_ex_rejects_invalid_arguments_on_host(kw):
    assert fwd_ex(dcn.load_library(), **kw) == INVALID


def test_forward_ex_empty_batch_and_old_entry_points():
    lib = dcn.load_library()
    assert fwd_ex(lib, N=0, flags=2 | 4, ptrs=(0, 0, 0, 0)) == OK
    assert fwd_ex(lib, N=0, flags=0, ptrs=(0, 0, 0, 0)) == OK
    # the entry points without flags keep their checks: no mask is invalid
    assert fwd(lib, ptrs=(0x1000, 0x2000, 0, 0x4000)) == INVALID
    assert bwd_ex(lib, flags=4) == INVALID                   # packed with separate mask pointers
    assert bwd_ex(lib, flags=4, ptrs=(0x1000, 0x2000, 0, 0x4000, 0x5000, 0x6000, 0x7000)) == INVALID
    assert bwd_ex(lib, flags=2, K=4) == INVALID
    assert bwd_ex(lib, flags=16) == INVALID
    assert bwd_ex(lib, flags=4, N=0, ptrs=(0,) * 7) == OK


def gate(lib, fn="forward", M=10, G=2, Cg=8, dtype=0, ptrs=None):
    n = 4 if fn == "forward" else 7
    ptrs = ptrs if ptrs is not None else tuple(0x1000 * (i + 1) for i in range(n))
    vp = [ctypes.c_void_p(x) if x else None for x in ptrs]
    f = lib.dcn_center_gate_forward if fn == "forward" else lib.dcn_center_gate_backward
    return f(*vp, M, G, Cg, dtype, None)


@pytest.mark.parametrize("fn", ["forward", "backward"])
def test_gate_validation(fn):
    lib = dcn.load_library()
    n = 4 if fn == "forward" else 7
    assert gate(lib, fn, M=-1) == INVALID
    assert gate(lib, fn, G=0) == INVALID
    assert gate(lib, fn, Cg=0) == INVALID
    assert gate(lib, fn, dtype=3) == INVALID
    assert gate(lib, fn, M=0, ptrs=(0,) * n) == OK
    for k in range(n):
        ptrs = [0x1000 * (i + 1) for i in range(n)]
        ptrs[k] = 0
        assert gate(lib, fn, ptrs=tuple(ptrs)) == INVALID          # a NULL pointer
        ptrs[k] = 0x1001
        assert gate(lib, fn, dtype=1, ptrs=tuple(ptrs)) == INVALID  # not element aligned
    assert gate(lib, fn, Cg=1 << 29) == UNSUPPORTED                # a row of 2^31 bytes
    assert gate(lib, fn, M=1 << 39, G=4) == UNSUPPORTED             # 2^41 rows


def test_linear_validation():
    lib = dcn.load_library()
    vp = ctypes.c_void_p

    def lin(x=0x1000, w=0x2000, b=None, y=0x3000, M=10, N=8, K=64, dtype=0):
        return lib.dcn_linear_forward(vp(x) if x else None, vp(w) if w else None, vp(b) if b else None,
                                      vp(y) if y else None, M, N, K, dtype, None)
    assert lin(M=-1) == INVALID and lin(N=0) == INVALID and lin(K=0) == INVALID and lin(dtype=7) == INVALID
    assert lin(x=0) == INVALID and lin(w=0) == INVALID and lin(y=0) == INVALID
    assert lin(x=0x1001, dtype=1) == INVALID                   # not element aligned
    assert lin(b=0x4001) == INVALID
    assert lin(M=0, x=0, w=0, y=0) == OK
    assert lin(K=6) == UNSUPPORTED                              # K not a multiple of 4
    assert lin(x=0x1004) == UNSUPPORTED                         # not 16-byte aligned
    assert lin(K=640) == UNSUPPORTED and lin(K=1212, dtype=1) == UNSUPPORTED   # w rows exceed on-chip memory


def test_layer_rejects_grid_changing_geometry():
    from deformable_convolution_core_amd.layer import DCNv4
    with pytest.raises(ValueError):
        DCNv4(64, kernel_size=4, group=4)          # even K cannot keep the grid
    with pytest.raises(ValueError):
        DCNv4(64, kernel_size=3, stride=2, group=4)
    with pytest.raises(ValueError):
        DCNv4(64, kernel_size=3, pad=0, group=4)
    with pytest.raises(ValueError):
        DCNv4(60, kernel_size=3, group=8)          # channels not divisible
    layer = DCNv4(64, kernel_size=3, group=4, remove_center=True, center_feature_scale=True)
    assert layer.offset_mask.out_features == 4 * 3 * 8
    assert layer.center_feature_scale_proj.out_features == 4


def test_static_scratch_backward_rejects_on_the_host():
    """dcn_core_backward_static validates before any HIP call: invalid
    arguments, and half-precision calls whose binary32 image of grad_input
    exceeds the static scratch (64 MiB), come back without a launch."""
    lib = dcn.load_library()
    vp = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(7)]
    f = ctypes.c_float(1.0)
    # 64 x 56 x 56 x 128 half elements need 102.8 MB of binary32 accumulators
    assert lib.dcn_core_backward_static(*vp, 64, 56, 56, 8, 16, 3, 1, 1, 1, f, 0, 1, None) == 4
    assert lib.dcn_core_backward_static(*vp, 64, 56, 56, 8, 16, 3, 1, 1, 1, f, 0, 2, None) == 4
    assert dcn.STATIC_SCRATCH_BYTES == 64 << 20
    assert lib.dcn_core_backward_static(*vp, 1, 8, 8, 2, 8, 0, 1, 1, 1, f, 0, 1, None) == INVALID   # K = 0
    assert lib.dcn_core_backward_static(*vp, 1, 8, 8, 2, 8, 3, 1, 1, 1, f, 8, 1, None) == INVALID   # bad flag
    assert lib.dcn_core_backward_static(*vp, 0, 8, 8, 2, 8, 3, 1, 1, 1, f, 0, 1, None) == OK        # empty batch


def test_status_strings():
    lib = dcn.load_library()
    for code, prefix in ((0, b"DCN_OK"), (1, b"DCN_ERR_INVALID_ARG"), (2, b"DCN_ERR_UNSUPPORTED"),
                         (3, b"DCN_ERR_HIP"), (4, b"DCN_ERR_SCRATCH_LIMIT"), (99, b"unknown")):
        assert lib.dcn_status_string(code).startswith(prefix)


def test_binding_rejects_bad_tensors_before_calling():
    x = torch.zeros(1, 8, 8, 16)
    off = torch.zeros(1, 8, 8, 2 * 9 * 2)
    m = torch.zeros(1, 8, 8, 2 * 9)
    with pytest.raises(ValueError):
        dcn.forward(x, off, m, group=2)                 # CPU tensors
    with pytest.raises(ValueError):
        dcn.forward(x, off[..., :-1], m, group=2)        # wrong offset shape
    with pytest.raises(ValueError):
        dcn.forward(x, off, m, group=3)                  # channels not divisible
    with pytest.raises(ValueError):
        dcn.forward(x, off, m, group=2, kernel_size=9, pad=0)   # empty grid


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        dcn.load_library(str(tmp_path / "nope.so"))


@pytest.mark.parametrize("shape", [(5000, 64, 64), (4096, 108, 64), (4097, 4, 64), (100, 8, 8)])
def test_layer_weight_grad_chunking(shape):
    """The layer's chunked weight gradient equals the float64 sum over rows
    (CPU tensors: the function is plain torch)."""
    from deformable_convolution_core_amd.layer import weight_grad
    M, O, I = shape
    gen = torch.Generator().manual_seed(M + O)
    g, x = torch.randn(M, O, generator=gen), torch.randn(M, I, generator=gen)
    want = g.double().t() @ x.double()
    got = weight_grad(g, x).double()
    assert (got - want).abs().max().item() <= 1e-5 * want.abs().max().item()
