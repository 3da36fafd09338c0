"""MI355X (gfx950) deformable sampling core of DCNv3 / DCNv4.

A thin ctypes binding over the C ABI of ``libdcn_core.so`` (declared in
``include/dcn_core.h``): it checks tensor shapes, dtypes and devices, allocates
outputs with torch, and passes raw device pointers plus torch's current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
there is no other implementation behind these functions, and they raise if
the library is not built.

The operation (pages: "没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读",
trdm.cn, section 4 steps 1-5; "DCNv4高效实践指南", seekfood.cn, core-architecture
section): for every output pixel and channel group, sample the group's
channels bilinearly (zero outside the map) at K*K offset positions around the
pixel and sum them weighted by the per-point mask, softmax-normalised for
DCNv3 and raw for DCNv4.  Tensors are channels-last:
input (N,H,W,G*Cg), offset (N,Ho,Wo,G*P*2) as (dx,dy) pixel pairs,
mask (N,Ho,Wo,G*P), output (N,Ho,Wo,G*Cg), with P = K*K points, or K*K - 1
with ``remove_center`` (odd K; the centre tap is left out).  DCNv4's single
offset-and-weight tensor is (N,Ho,Wo,G*3P): per (pixel, group) the 2P
offsets, then the P mask values (``forward_packed`` / ``backward_packed``).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["forward", "backward", "forward_packed", "backward_packed", "out_size", "dcn_core",
           "dcnv4_core", "center_gate_forward", "center_gate_backward", "center_gate", "linear",
           "linear_weight_grad",
           "DCNCoreFunction", "DCNv4CoreFunction", "CenterGateFunction", "DCNv4GatedFunction",
           "forward_packed_gated", "DCNError", "library_path",
           "load_library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libdcn_core.so")
_lib = None

DCN_F32, DCN_F16, DCN_BF16 = 0, 1, 2
_DTYPE = {torch.float32: DCN_F32, torch.float16: DCN_F16, torch.bfloat16: DCN_BF16}
EXPORTED = ("dcn_core_out_size", "dcn_core_forward", "dcn_core_backward", "dcn_core_forward_ex",
            "dcn_core_backward_ex", "dcn_core_backward_workspace_size", "dcn_core_backward_ws",
            "dcn_center_gate_forward", "dcn_center_gate_backward", "dcn_linear_forward", "dcn_linear_weight_grad", "dcn_linear_weight_grad_workspace_size",
            "dcn_core_forward_gated", "dcn_core_backward_static",
            "dcn_status_string")
FLAG_SOFTMAX, FLAG_REMOVE_CENTER, FLAG_PACKED = 1, 2, 4
STATIC_SCRATCH_BYTES = 64 << 20   # DCN_STATIC_SCRATCH_BYTES of the C header


class DCNError(RuntimeError):
    """A dcn_core call returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: str | None = None):
    """Load libdcn_core.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path
    if not os.path.exists(p):
        raise RuntimeError(
            f"HIP library not built: {p} is missing; build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` at the repository root")
    lib = ctypes.CDLL(p)
    i, f, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.dcn_core_out_size.argtypes = [i] * 5
    lib.dcn_core_out_size.restype = i
    lib.dcn_core_forward.argtypes = [vp] * 4 + [i] * 9 + [f, i, i, vp]
    lib.dcn_core_forward.restype = i
    lib.dcn_core_backward.argtypes = [vp] * 7 + [i] * 9 + [f, i, i, vp]
    lib.dcn_core_backward.restype = i
    lib.dcn_core_forward_ex.argtypes = [vp] * 4 + [i] * 9 + [f, i, i, vp]
    lib.dcn_core_forward_ex.restype = i
    lib.dcn_core_backward_ex.argtypes = [vp] * 7 + [i] * 9 + [f, i, i, vp]
    lib.dcn_core_backward_ex.restype = i
    ll = ctypes.c_longlong
    lib.dcn_core_backward_workspace_size.argtypes = [vp] * 3 + [i] * 9 + [f, i, i]
    lib.dcn_core_backward_workspace_size.restype = ll
    lib.dcn_core_backward_ws.argtypes = [vp] * 7 + [i] * 9 + [f, i, i, vp, ll, vp]
    lib.dcn_core_backward_ws.restype = i
    lib.dcn_center_gate_forward.argtypes = [vp] * 4 + [ll, i, i, i, vp]
    lib.dcn_center_gate_forward.restype = i
    lib.dcn_center_gate_backward.argtypes = [vp] * 7 + [ll, i, i, i, vp]
    lib.dcn_center_gate_backward.restype = i
    lib.dcn_linear_forward.argtypes = [vp] * 4 + [ll, i, i, i, vp]
    lib.dcn_linear_forward.restype = i
    lib.dcn_core_forward_gated.argtypes = [vp] * 6 + [i] * 9 + [f, i, i, vp]
    lib.dcn_core_forward_gated.restype = i
    lib.dcn_linear_weight_grad.argtypes = [vp] * 4 + [ll, i, i, i, i, vp, ll, vp]
    lib.dcn_linear_weight_grad.restype = i
    lib.dcn_linear_weight_grad_workspace_size.argtypes = [ll, i, i]
    lib.dcn_linear_weight_grad_workspace_size.restype = ll
    lib.dcn_core_backward_static.argtypes = [vp] * 7 + [i] * 9 + [f, i, i, vp]
    lib.dcn_core_backward_static.restype = i
    lib.dcn_status_string.argtypes = [i]
    lib.dcn_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load_library().dcn_status_string(rc).decode()
        raise DCNError(rc, f"{what}: {msg}")


def out_size(n: int, kernel_size: int, stride: int, pad: int, dilation: int) -> int:
    """Output extent along one axis (<= 0 if invalid), from the library."""
    return int(load_library().dcn_core_out_size(n, kernel_size, stride, pad, dilation))


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else ctypes.c_void_p(0)


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def points(kernel_size: int, remove_center: bool = False) -> int:
    """Sampling points per (pixel, group): K*K, less the centre tap if removed."""
    return kernel_size * kernel_size - (1 if remove_center else 0)


def _flags(softmax, remove_center, packed):
    return ((FLAG_SOFTMAX if softmax else 0) | (FLAG_REMOVE_CENTER if remove_center else 0)
            | (FLAG_PACKED if packed else 0))


def _check_tensor(name, t, ref):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (channels-last NHWC)")
    if t.dtype != ref.dtype or t.device != ref.device:
        raise ValueError(f"{name} must share input's dtype and device")


def _geometry(input, offset, mask, kernel_size, stride, pad, dilation, group, remove_center=False):
    """Shapes of a call; mask None means the packed layout (offset holds the records)."""
    if input.dim() != 4:
        raise ValueError("input must be (N, H, W, G*Cg)")
    N, H, W, C = input.shape
    if group < 1 or C % group:
        raise ValueError(f"channels {C} not divisible by group {group}")
    if remove_center and (kernel_size % 2 == 0 or kernel_size < 3):
        raise ValueError("remove_center needs an odd kernel_size >= 3")
    Ho = out_size(H, kernel_size, stride, pad, dilation)
    Wo = out_size(W, kernel_size, stride, pad, dilation)
    if Ho <= 0 or Wo <= 0:
        raise ValueError("empty output grid for this geometry")
    P = points(kernel_size, remove_center)
    if mask is None:
        if tuple(offset.shape) != (N, Ho, Wo, group * P * 3):
            raise ValueError(f"offset_mask must be {(N, Ho, Wo, group * P * 3)}, got {tuple(offset.shape)}")
        tensors = (("input", input), ("offset_mask", offset))
    else:
        if tuple(offset.shape) != (N, Ho, Wo, group * P * 2):
            raise ValueError(f"offset must be {(N, Ho, Wo, group * P * 2)}, got {tuple(offset.shape)}")
        if tuple(mask.shape) != (N, Ho, Wo, group * P):
            raise ValueError(f"mask must be {(N, Ho, Wo, group * P)}, got {tuple(mask.shape)}")
        tensors = (("input", input), ("offset", offset), ("mask", mask))
    for name, t in tensors:
        _check_tensor(name, t, input)
    if input.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {input.dtype}")
    return N, H, W, C, C // group, Ho, Wo


def _forward(input, offset, mask, kernel_size, stride, pad, dilation, offset_scale, softmax, group,
             remove_center, out):
    N, H, W, C, Cg, Ho, Wo = _geometry(input, offset, mask, kernel_size, stride, pad, dilation, group,
                                       remove_center)
    if out is None:
        out = torch.empty((N, Ho, Wo, C), dtype=input.dtype, device=input.device)
    elif tuple(out.shape) != (N, Ho, Wo, C) or out.dtype != input.dtype or not out.is_contiguous() \
            or out.device != input.device:
        raise ValueError("out has the wrong shape, dtype, device or layout")
    flags = _flags(softmax, remove_center, mask is None)
    with torch.cuda.device(input.device):
        rc = load_library().dcn_core_forward_ex(
            _ptr(input), _ptr(offset), None if mask is None else _ptr(mask), _ptr(out), N, H, W, group,
            Cg, kernel_size, stride, pad, dilation, float(offset_scale), flags, _DTYPE[input.dtype],
            _stream(input.device))
    _check(rc, "dcn_core_forward_ex")
    return out


def _backward(input, offset, mask, grad_output, kernel_size, stride, pad, dilation, offset_scale, softmax,
              group, remove_center):
    N, H, W, C, Cg, Ho, Wo = _geometry(input, offset, mask, kernel_size, stride, pad, dilation, group,
                                       remove_center)
    if tuple(grad_output.shape) != (N, Ho, Wo, C) or grad_output.dtype != input.dtype \
            or not grad_output.is_contiguous() or grad_output.device != input.device:
        raise ValueError("grad_output has the wrong shape, dtype, device or layout")
    gi = torch.empty_like(input)
    goff = torch.empty_like(offset)
    gm = None if mask is None else torch.empty_like(mask)
    flags = _flags(softmax, remove_center, mask is None)
    lib = load_library()
    geo = (N, H, W, group, Cg, kernel_size, stride, pad, dilation, float(offset_scale), flags, _DTYPE[input.dtype])
    # half precision outside the tiled shapes accumulates grad_input in a
    # binary32 workspace, allocated here only when the library asks for one
    need = lib.dcn_core_backward_workspace_size(_ptr(input), _ptr(grad_output), _ptr(gi), *geo)
    if need < 0:
        _check(int(-need), "dcn_core_backward_workspace_size")
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=input.device) if need > 0 else None
    with torch.cuda.device(input.device):
        rc = lib.dcn_core_backward_ws(
            _ptr(input), _ptr(offset), None if mask is None else _ptr(mask), _ptr(grad_output), _ptr(gi),
            _ptr(goff), None if gm is None else _ptr(gm), *geo, None if ws is None else _ptr(ws),
            0 if ws is None else ws.numel() * 4, _stream(input.device))
    _check(rc, "dcn_core_backward_ws")
    return gi, goff, gm


def forward(input, offset, mask, *, kernel_size=3, stride=1, pad=1, dilation=1,
            offset_scale=1.0, softmax=False, group=1, remove_center=False, out=None) -> torch.Tensor:
    """Forward sampling core on input.device, on torch's current stream."""
    if mask is None:
        raise ValueError("mask is required (forward_packed takes the packed layout)")
    return _forward(input, offset, mask, kernel_size, stride, pad, dilation, offset_scale, softmax, group,
                    remove_center, out)


def backward(input, offset, mask, grad_output, *, kernel_size=3, stride=1, pad=1, dilation=1,
             offset_scale=1.0, softmax=False, group=1, remove_center=False):
    """Gradients (grad_input, grad_offset, grad_mask) for grad_output."""
    if mask is None:
        raise ValueError("mask is required (backward_packed takes the packed layout)")
    return _backward(input, offset, mask, grad_output, kernel_size, stride, pad, dilation, offset_scale,
                     softmax, group, remove_center)


def forward_packed(input, offset_mask, *, kernel_size=3, stride=1, pad=1, dilation=1,
                   offset_scale=1.0, softmax=False, group=1, remove_center=False, out=None) -> torch.Tensor:
    """Forward with DCNv4's single offset-and-mask tensor (N, Ho, Wo, G*3P)."""
    return _forward(input, offset_mask, None, kernel_size, stride, pad, dilation, offset_scale, softmax,
                    group, remove_center, out)


def forward_packed_gated(input, offset_mask, gate_logits, *, kernel_size=3, dilation=1, offset_scale=1.0,
                         group=1, remove_center=False, keep_core_output=False):
    """DCNv4 forward (packed records, raw mask) with the layer's centre-feature
    gate fused in: returns (output, core_output or None), output = y (1 - s) +
    input s with s = sigmoid(gate_logits) per (pixel, group) and y the sampled
    result (returned rounded to the dtype if keep_core_output).  Stride 1 and
    pad = dilation (K - 1) / 2 with an odd K.  Raises DCNError with status
    DCN_ERR_UNSUPPORTED (2) for shapes the fused kernel does not take."""
    pad = dilation * (kernel_size - 1) // 2
    N, H, W, C, Cg, Ho, Wo = _geometry(input, offset_mask, None, kernel_size, 1, pad, dilation, group,
                                       remove_center)
    if tuple(gate_logits.shape) != (N, Ho, Wo, group):
        raise ValueError("gate_logits must be (N, H, W, group)")
    _check_tensor("gate_logits", gate_logits, input)
    out = torch.empty((N, Ho, Wo, C), dtype=input.dtype, device=input.device)
    core = torch.empty_like(out) if keep_core_output else None
    with torch.cuda.device(input.device):
        rc = load_library().dcn_core_forward_gated(
            _ptr(input), _ptr(offset_mask), None, _ptr(gate_logits), _ptr(out), None if core is None else _ptr(core),
            N, H, W, group, Cg, kernel_size, 1, pad, dilation, float(offset_scale),
            _flags(False, remove_center, True), _DTYPE[input.dtype], _stream(input.device))
    _check(rc, "dcn_core_forward_gated")
    return out, core


def backward_packed(input, offset_mask, grad_output, *, kernel_size=3, stride=1, pad=1, dilation=1,
                    offset_scale=1.0, softmax=False, group=1, remove_center=False):
    """Gradients (grad_input, grad_offset_mask) of forward_packed; the second
    has the packed record layout of offset_mask."""
    gi, gom, _ = _backward(input, offset_mask, None, grad_output, kernel_size, stride, pad, dilation,
                           offset_scale, softmax, group, remove_center)
    return gi, gom


def _gate_check(y, v, z, group):
    if y.dim() < 1 or y.shape[-1] % group:
        raise ValueError("y's last axis must hold group * Cg channels")
    if tuple(v.shape) != tuple(y.shape) or tuple(z.shape) != tuple(y.shape[:-1]) + (group,):
        raise ValueError(f"v must be shaped like y and z like y[..., :{group}]")
    for name, t in (("y", y), ("v", v), ("z", z)):
        _check_tensor(name, t, y)
    if y.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {y.dtype}")
    M = y.numel() // y.shape[-1] if y.numel() else 0
    return M, y.shape[-1] // group


def center_gate_forward(y, v, z, *, group, out=None) -> torch.Tensor:
    """y * (1 - s) + v * s with s = sigmoid(z) per (pixel, group), in HIP.
    y, v: (..., G*Cg); z: (..., G).  out may be y or v."""
    M, Cg = _gate_check(y, v, z, group)
    if out is None:
        out = torch.empty_like(y)
    elif out.shape != y.shape or out.dtype != y.dtype or not out.is_contiguous() or out.device != y.device:
        raise ValueError("out has the wrong shape, dtype, device or layout")
    with torch.cuda.device(y.device):
        rc = load_library().dcn_center_gate_forward(_ptr(y), _ptr(v), _ptr(z), _ptr(out), M, group, Cg,
                                                    _DTYPE[y.dtype], _stream(y.device))
    _check(rc, "dcn_center_gate_forward")
    return out


def center_gate_backward(y, v, z, grad_output, *, group):
    """Gradients (grad_y, grad_v, grad_z) of center_gate_forward."""
    M, Cg = _gate_check(y, v, z, group)
    if grad_output.shape != y.shape or grad_output.dtype != y.dtype or not grad_output.is_contiguous() \
            or grad_output.device != y.device:
        raise ValueError("grad_output has the wrong shape, dtype, device or layout")
    gy, gv, gz = torch.empty_like(y), torch.empty_like(v), torch.empty_like(z)
    with torch.cuda.device(y.device):
        rc = load_library().dcn_center_gate_backward(_ptr(y), _ptr(v), _ptr(z), _ptr(grad_output), _ptr(gy),
                                                     _ptr(gv), _ptr(gz), M, group, Cg, _DTYPE[y.dtype],
                                                     _stream(y.device))
    _check(rc, "dcn_center_gate_backward")
    return gy, gv, gz


def linear(x, weight, bias=None, *, out=None) -> torch.Tensor:
    """x @ weight.T + bias over the last axis of x, on the matrix cores (HIP).
    x (..., K), weight (N, K), bias (N) or None.  Raises DCNError with status
    DCN_ERR_UNSUPPORTED (2) for shapes the kernel does not take (K not a
    multiple of 4, misaligned or too wide), so a caller can use another GEMM."""
    if weight.dim() != 2 or x.shape[-1] != weight.shape[1]:
        raise ValueError("x (..., K) and weight (N, K) must agree on K")
    N, K = weight.shape
    for name, t in (("x", x), ("weight", weight)) + ((("bias", bias),) if bias is not None else ()):
        _check_tensor(name, t, x)
    if bias is not None and tuple(bias.shape) != (N,):
        raise ValueError("bias must be (N,)")
    if x.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {x.dtype}")
    M = x.numel() // K if K else 0
    if out is None:
        out = torch.empty(*x.shape[:-1], N, dtype=x.dtype, device=x.device)
    with torch.cuda.device(x.device):
        rc = load_library().dcn_linear_forward(_ptr(x), _ptr(weight), None if bias is None else _ptr(bias),
                                               _ptr(out), M, N, K, _DTYPE[x.dtype], _stream(x.device))
    _check(rc, "dcn_linear_forward")
    return out


def linear_weight_grad(g, x, *, bias: bool = True, out_dtype=torch.float32):
    """Weight and bias gradients of y = x @ weight.T + bias on the matrix cores
    (HIP): g (..., O) the gradient of y, x (..., I) the input.  Returns
    (dw (O, I), db (O,) or None) in out_dtype: binary32 sums over rows,
    deterministic (fixed-order chunk partials, kept in a workspace allocated
    here), rounded once to out_dtype."""
    if g.shape[:-1] != x.shape[:-1]:
        raise ValueError("g (..., O) and x (..., I) must share their leading dimensions")
    _check_tensor("g", g, g)
    _check_tensor("x", x, g)
    if g.dtype not in _DTYPE or out_dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {g.dtype} / {out_dtype}")
    O, I = g.shape[-1], x.shape[-1]
    M = g.numel() // O if O else 0
    lib = load_library()
    need = lib.dcn_linear_weight_grad_workspace_size(M, O, I)
    if need < 0:
        _check(int(-need), "dcn_linear_weight_grad_workspace_size")
    dw = torch.empty(O, I, dtype=out_dtype, device=g.device)
    db = torch.empty(O, dtype=out_dtype, device=g.device) if bias else None
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=g.device) if need > 0 else None
    with torch.cuda.device(g.device):
        rc = lib.dcn_linear_weight_grad(_ptr(g), _ptr(x), _ptr(dw), None if db is None else _ptr(db), M, O, I,
                                        _DTYPE[g.dtype], _DTYPE[out_dtype], None if ws is None else _ptr(ws),
                                        0 if ws is None else ws.numel() * 4, _stream(g.device))
    _check(rc, "dcn_linear_weight_grad")
    return dw, db


class CenterGateFunction(torch.autograd.Function):
    """Autograd wrapper of the centre-feature gate."""

    @staticmethod
    def forward(ctx, y, v, z, group):
        ctx.save_for_backward(y, v, z)
        ctx.group = group
        return center_gate_forward(y, v, z, group=group)

    @staticmethod
    def backward(ctx, grad_out):
        y, v, z = ctx.saved_tensors
        gy, gv, gz = center_gate_backward(y, v, z, grad_out.contiguous(), group=ctx.group)
        return gy, gv, gz, None


def center_gate(y, v, z, group):
    """Differentiable centre-feature gate."""
    return CenterGateFunction.apply(y, v, z, group)


class DCNCoreFunction(torch.autograd.Function):
    """Autograd wrapper: the backward recomputes the sampling from the saved
    input, offset and mask (nothing else is kept between the passes)."""

    @staticmethod
    def forward(ctx, input, offset, mask, kernel_size, stride, pad, dilation, offset_scale,
                softmax, group, remove_center=False):
        ctx.save_for_backward(input, offset, mask)
        ctx.cfg = dict(kernel_size=kernel_size, stride=stride, pad=pad, dilation=dilation,
                       offset_scale=offset_scale, softmax=softmax, group=group,
                       remove_center=remove_center)
        return forward(input, offset, mask, **ctx.cfg)

    @staticmethod
    def backward(ctx, grad_out):
        input, offset, mask = ctx.saved_tensors
        gi, goff, gm = backward(input, offset, mask, grad_out.contiguous(), **ctx.cfg)
        return gi, goff, gm, None, None, None, None, None, None, None, None


class DCNv4CoreFunction(torch.autograd.Function):
    """Autograd wrapper of the packed (DCNv4) layout."""

    @staticmethod
    def forward(ctx, input, offset_mask, kernel_size, stride, pad, dilation, offset_scale, group,
                remove_center=False):
        ctx.save_for_backward(input, offset_mask)
        ctx.cfg = dict(kernel_size=kernel_size, stride=stride, pad=pad, dilation=dilation,
                       offset_scale=offset_scale, softmax=False, group=group,
                       remove_center=remove_center)
        return forward_packed(input, offset_mask, **ctx.cfg)

    @staticmethod
    def backward(ctx, grad_out):
        input, offset_mask = ctx.saved_tensors
        gi, gom = backward_packed(input, offset_mask, grad_out.contiguous(), **ctx.cfg)
        return gi, gom, None, None, None, None, None, None, None


class DCNv4GatedFunction(torch.autograd.Function):
    """Autograd wrapper of the fused DCNv4 core + centre-feature gate.  The
    backward is the gate's backward (on the saved pre-gate result) followed
    by the core's, the two gradients of the input added."""

    @staticmethod
    def forward(ctx, input, offset_mask, gate_logits, kernel_size, dilation, offset_scale, group, remove_center):
        ctx.cfg = dict(kernel_size=kernel_size, stride=1, pad=dilation * (kernel_size - 1) // 2,
                       dilation=dilation, offset_scale=offset_scale, softmax=False, group=group,
                       remove_center=remove_center)
        out, core = forward_packed_gated(input, offset_mask, gate_logits, kernel_size=kernel_size,
                                         dilation=dilation, offset_scale=offset_scale, group=group,
                                         remove_center=remove_center, keep_core_output=True)
        ctx.save_for_backward(input, offset_mask, gate_logits, core)
        return out

    @staticmethod
    def backward(ctx, grad_out):
        input, offset_mask, z, core = ctx.saved_tensors
        gy, gv, gz = center_gate_backward(core, input, z, grad_out.contiguous(), group=ctx.cfg["group"])
        gi, gom = backward_packed(input, offset_mask, gy, **ctx.cfg)
        return gi + gv, gom, gz, None, None, None, None, None


def dcn_core(input, offset, mask, kernel_size=3, stride=1, pad=1, dilation=1, offset_scale=1.0,
             softmax=False, group=1, remove_center=False):
    """Differentiable entry point (forward + analytic backward in HIP)."""
    return DCNCoreFunction.apply(input, offset, mask, kernel_size, stride, pad, dilation,
                                 offset_scale, softmax, group, remove_center)


def dcnv4_core(input, offset_mask, kernel_size=3, stride=1, pad=1, dilation=1, offset_scale=1.0,
               group=1, remove_center=False):
    """Differentiable DCNv4 core: raw mask, offsets and mask in one packed tensor."""
    return DCNv4CoreFunction.apply(input, offset_mask, kernel_size, stride, pad, dilation,
                                   offset_scale, group, remove_center)
