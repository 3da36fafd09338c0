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
                                             optional centre-feature gate (HIP)
    out = y @ Wo.T + bo

The four projections are plain GEMMs and run in the platform BLAS through
torch.nn.functional.linear; the sampling core and the gate run in this
package's HIP kernels.  Input and output are channels-last (N, H, W, C).  The
offsets are predicted per input pixel, so the layer keeps the grid: stride
1 and pad = dilation * (K - 1) / 2 with an odd K.
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

from . import center_gate, dcnv4_core, points


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
        v = F.linear(x, self.value_proj.weight, self.value_proj.bias)
        om = F.linear(x, self.offset_mask.weight, self.offset_mask.bias)
        y = dcnv4_core(v, om, self.kernel_size, 1, self.pad, self.dilation, self.offset_scale, self.group,
                       self.remove_center)
        if self.center_feature_scale_proj is not None:
            z = F.linear(x, self.center_feature_scale_proj.weight, self.center_feature_scale_proj.bias)
            y = center_gate(y, v, z, self.group)
        return F.linear(y, self.output_proj.weight, self.output_proj.bias)

    def numpy_params(self) -> dict:
        """The parameters as float64 numpy arrays, keyed Wv, bv, Wom, bom, Wc, bc, Wo, bo."""
        def np64(t):
            return None if t is None else t.detach().double().cpu().numpy()
        c = self.center_feature_scale_proj
        return dict(Wv=np64(self.value_proj.weight), bv=np64(self.value_proj.bias),
                    Wom=np64(self.offset_mask.weight), bom=np64(self.offset_mask.bias),
                    Wc=np64(c.weight) if c is not None else None, bc=np64(c.bias) if c is not None else None,
                    Wo=np64(self.output_proj.weight), bo=np64(self.output_proj.bias))
