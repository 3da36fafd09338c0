"""The DCNv4 layer around the sampling core.

Data flow (page "没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读",
trdm.cn, section 3, with the DCNv4 changes of "告别DCNv3的卡顿：实测DCNv4在A100上3倍提速…",
framerc.cn, section 1 -- one merged offset/weight projection, no LN-GELU, raw
mask; the constructor's arguments follow the DCNv4 module of
"DCNv4高效实践指南", seekfood.cn, programming-interface section):

    v   = x @ Wv.T + bv                      value projection, kept for the gate
    om  = x @ Wom.T + bom                    (N, H, W, G*3P): per (pixel, group)
                                             2P offsets then P raw mask values
    y   = core(v, om)                        HIP sampling core, packed layout
    y   = y * (1 - s) + v * s,  s = sigmoid(x @ Wc.T + bc)
                                             optional centre-feature gate (HIP,
                                             fused into the core's epilogue
                                             where the tiled kernel runs)
    out = y @ Wo.T + bo

The four projections and their input gradients run in this package's
matrix-core GEMM (`linear`: X read once, W in on-chip memory), falling back
to the platform BLAS for shapes it does not take; their weight and bias
gradients run in the package's split-row matrix-core reduction
(`linear_weight_grad`), with a batched BLAS GEMM over row chunks
(weight_grad) as the fallback.  The sampling core and the gate run in this
package's HIP kernels.  Input and output are channels-last (N, H, W, C).  The
offsets are predicted per input pixel, so the layer keeps the grid: stride
1 and pad = dilation * (K - 1) / 2 with an odd K.
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

from . import (DCNError, DCNv4GatedFunction, center_gate, dcnv4_core, forward_packed_gated, linear,
               linear_weight_grad, points)


_WGRAD_ROWS = 2048   # rows per chunk of the weight-gradient reduction


def weight_grad(g2: torch.Tensor, x2: torch.Tensor) -> torch.Tensor:
    """sum over rows m of g2[m, :]^T x2[m, :] -> (out, in), for a row count in
    the hundreds of thousands and a few dozen columns.  One GEMM with that
    long reduction runs on a handful of tiles; chunks of _WGRAD_ROWS rows as
    one batched GEMM spread it over the chip, and the per-chunk partials are
    summed in binary32.  The narrower operand is the one transposed, and both
    GEMM operands are contiguous."""
    M, O = g2.shape
    I = x2.shape[1]
    S = M // _WGRAD_ROWS
    out = torch.zeros(O, I, dtype=torch.float32, device=g2.device)
    if S > 0:
        n = S * _WGRAD_ROWS
        gc = g2[:n].view(S, _WGRAD_ROWS, O)
        xc = x2[:n].view(S, _WGRAD_ROWS, I)
        if O <= I:
            part = torch.bmm(gc.transpose(1, 2).contiguous(), xc)              # (S, O, I)
            out += part.sum(0, dtype=torch.float32)
        else:
            part = torch.bmm(xc.transpose(1, 2).contiguous(), gc)              # (S, I, O)
            out += part.sum(0, dtype=torch.float32).t()
    if S * _WGRAD_ROWS < M:
        r = S * _WGRAD_ROWS
        out += (g2[r:].t().float() @ x2[r:].float())
    return out.to(g2.dtype)


def _matmul_t(x, W, b=None):
    """x @ W.T + b: the package's matrix-core kernel where it takes the shape,
    else the platform BLAS."""
    try:
        return linear(x, W, b)
    except DCNError as e:
        if e.status != 2:        # only "unsupported shape" falls through
            raise
        return F.linear(x, W, b)


class _Projection(torch.autograd.Function):
    """x @ W.T + b; the input gradient g @ W as the same kernel on W.T, the
    weight and bias gradients by _param_grads."""

    @staticmethod
    def forward(ctx, x, W, b):
        ctx.save_for_backward(x, W)
        return _matmul_t(x, W, b)

    @staticmethod
    def backward(ctx, g):
        x, W = ctx.saved_tensors
        g2 = g.reshape(-1, g.shape[-1]).contiguous()
        gx = _matmul_t(g2, W.t().contiguous()).view(x.shape) if ctx.needs_input_grad[0] else None
        gW, gb = _param_grads(g2, x.reshape(-1, x.shape[-1]), ctx.needs_input_grad[1], ctx.needs_input_grad[2])
        return gx, gW, gb


def _param_grads(g2, x2, want_w, want_b):
    """Weight and bias gradients of a projection in the weight's dtype: the
    package's matrix-core reduction, or for shapes it does not take the
    batched BLAS path (weight_grad) and a column sum."""
    if not (want_w or want_b):
        return None, None
    try:
        dw, db = linear_weight_grad(g2, x2, bias=want_b, out_dtype=g2.dtype)
    except DCNError as e:
        if e.status != 2:        # only "unsupported shape" falls through
            raise
        dw = weight_grad(g2, x2) if want_w else None
        db = g2.sum(0, dtype=torch.float32) if want_b else None
    return (dw.to(g2.dtype) if want_w else None), (db.to(g2.dtype) if want_b else None)


def project(x, lin: torch.nn.Linear):
    return _Projection.apply(x, lin.weight, lin.bias)


class DCNv4(torch.nn.Module):
    """DCNv4 layer on channels-last input (N, H, W, channels)."""

    def __init__(self, channels: int, kernel_size: int = 3, stride: int = 1, pad: int | None = None,
                 dilation: int = 1, group: int = 4, offset_scale: float = 1.0,
                 center_feature_scale: bool = False, remove_center: bool = False,
                 device=None, dtype=None):
        super().__init__()
        if channels % group:
            raise ValueError(f"channels {channels} not divisible by group {group}")
        if kernel_size % 2 == 0:
            raise ValueError("the layer keeps the grid, so kernel_size must be odd")
        if pad is None:
            pad = dilation * (kernel_size - 1) // 2
        if stride != 1 or pad != dilation * (kernel_size - 1) // 2:
            raise ValueError("the layer keeps the grid: stride 1 and pad = dilation * (kernel_size - 1) / 2")
        self.channels, self.kernel_size, self.pad, self.dilation = channels, kernel_size, pad, dilation
        self.group, self.offset_scale = group, float(offset_scale)
        self.center_feature_scale, self.remove_center = bool(center_feature_scale), bool(remove_center)
        P = points(kernel_size, remove_center)
        fk = dict(device=device, dtype=dtype)
        self.value_proj = torch.nn.Linear(channels, channels, **fk)
        self.offset_mask = torch.nn.Linear(channels, group * 3 * P, **fk)
        self.output_proj = torch.nn.Linear(channels, channels, **fk)
        self.center_feature_scale_proj = (torch.nn.Linear(channels, group, **fk)
                                          if center_feature_scale else None)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.dim() != 4 or x.shape[-1] != self.channels:
            raise ValueError(f"input must be (N, H, W, {self.channels})")
        x = x.contiguous()
        v = project(x, self.value_proj)
        om = project(x, self.offset_mask)
        if self.center_feature_scale_proj is not None:
            z = project(x, self.center_feature_scale_proj)
            y = self._gated_core(v, om, z)
        else:
            y = dcnv4_core(v, om, self.kernel_size, 1, self.pad, self.dilation, self.offset_scale, self.group,
                           self.remove_center)
        return project(y, self.output_proj)

    def _gated_core(self, v, om, z):
        """The core with the centre-feature gate fused into its epilogue
        (HIP), keeping the pre-gate result only when a backward will need
        it; the core and the gate as two kernels for shapes the fused kernel
        does not take."""
        args = (self.kernel_size, self.dilation, self.offset_scale, self.group, self.remove_center)
        try:
            if torch.is_grad_enabled() and (v.requires_grad or om.requires_grad or z.requires_grad):
                return DCNv4GatedFunction.apply(v, om, z, *args)
            return forward_packed_gated(v, om, z, kernel_size=self.kernel_size, dilation=self.dilation,
                                        offset_scale=self.offset_scale, group=self.group,
                                        remove_center=self.remove_center)[0]
        except DCNError as e:
            if e.status != 2:        # only "unsupported shape" falls through
                raise
        y = dcnv4_core(v, om, self.kernel_size, 1, self.pad, self.dilation, self.offset_scale, self.group,
                       self.remove_center)
        return center_gate(y, v, z, self.group)

    def numpy_params(self) -> dict:
        """The parameters as float64 numpy arrays, keyed Wv, bv, Wom, bom, Wc, bc, Wo, bo."""
        def np64(t):
            return None if t is None else t.detach().double().cpu().numpy()
        c = self.center_feature_scale_proj
        return dict(Wv=np64(self.value_proj.weight), bv=np64(self.value_proj.bias),
                    Wom=np64(self.offset_mask.weight), bom=np64(self.offset_mask.bias),
                    Wc=np64(c.weight) if c is not None else None, bc=np64(c.bias) if c is not None else None,
                    Wo=np64(self.output_proj.weight), bo=np64(self.output_proj.bias))
