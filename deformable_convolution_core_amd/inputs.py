"""Seeded synthetic inputs for the deformable sampling core.

This module only draws random tensors of stated shapes and distributions; it
holds none of the sampling arithmetic, so the CPU oracle and the HIP path can
both be fed from it without sharing any computation.  Output extents (Ho, Wo)
are part of each workload's description and are passed in, never derived here.

The workloads stand in for FlashInternImage-T feature maps at 224 px (four
stages of 56/28/14/7 px, 64 base channels, groups [4, 8, 16, 32], i.e. 16
channels per group, offset_scale 1.0; the T config printed on the page
"DCNv4高效实践指南：掌握可变形卷积的3倍速度提升技术", classification config
section) and an InternImage-G-like large-channel stage (32 channels per group).
No dataset or trained weights are involved: inputs ~ N(0,1), offsets are
i.i.d. normal pixel offsets, masks are normal logits (softmax) or raw weights.

Random values are float32 normals from numpy's PCG64 generator scaled by the
stated sigma, then rounded once (round-to-nearest-even) to the workload dtype;
both sides read the identical rounded tensors.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}

# tensor ids used in the seed: seed = 1000*config + 100*subshape + id
T_INPUT, T_OFFSET, T_MASK, T_GRAD_OUT = 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    W: int
    G: int
    Cg: int
    Ho: int
    Wo: int
    K: int = 3
    stride: int = 1
    pad: int = 1
    dilation: int = 1
    offset_scale: float = 1.0
    softmax: bool = False
    dtype: str = "f32"
    offset_sigma: float = 1.5
    mask_sigma: float = 0.3
    seed_base: int = 0
    backward: bool = False
    remove_center: bool = False   # odd K: the centre tap is left out

    @property
    def C(self) -> int:
        return self.G * self.Cg

    @property
    def P(self) -> int:
        return self.K * self.K - (1 if self.remove_center else 0)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def shapes(self):
        return dict(input=(self.N, self.H, self.W, self.C),
                    offset=(self.N, self.Ho, self.Wo, self.G * self.P * 2),
                    mask=(self.N, self.Ho, self.Wo, self.G * self.P),
                    output=(self.N, self.Ho, self.Wo, self.C))

    def min_bytes_forward(self) -> int:
        """input + offset + mask + output, each touched once."""
        return self.elem_bytes * sum(int(np.prod(s)) for s in self.shapes().values())

    def min_bytes_backward(self) -> int:
        """read input, offset, mask, grad_out; write grad_input, grad_offset, grad_mask."""
        s = self.shapes()
        n = 2 * int(np.prod(s["input"])) + 2 * int(np.prod(s["offset"])) \
            + 2 * int(np.prod(s["mask"])) + int(np.prod(s["output"]))
        return self.elem_bytes * n

    def samples(self) -> int:
        """bilinear reads of one (pixel, group, point) channel row per call."""
        return self.N * self.Ho * self.Wo * self.G * self.P


def _w(name, cfg, sub, **kw):
    return Workload(name=name, seed_base=1000 * cfg + 100 * sub, **kw)


# The five workload families; each is a parity case, config 2 is the headline.
WORKLOADS = {
    "c1_dcnv3_f32_8x8": _w("c1_dcnv3_f32_8x8", 1, 0, N=1, H=8, W=8, G=2, Cg=8, Ho=8, Wo=8,
                           softmax=True, dtype="f32", offset_sigma=1.5, mask_sigma=1.0),
    "c2_dcnv4_f16_56": _w("c2_dcnv4_f16_56", 2, 0, N=64, H=56, W=56, G=4, Cg=16, Ho=56, Wo=56,
                          dtype="f16", offset_sigma=1.5, mask_sigma=0.3),
    "c3a_dcnv4_bf16_56": _w("c3a_dcnv4_bf16_56", 3, 0, N=64, H=56, W=56, G=4, Cg=16, Ho=56, Wo=56,
                            dtype="bf16", offset_sigma=2.0, mask_sigma=0.3),
    "c3b_dcnv4_bf16_28": _w("c3b_dcnv4_bf16_28", 3, 1, N=64, H=28, W=28, G=8, Cg=16, Ho=28, Wo=28,
                            dtype="bf16", offset_sigma=2.0, mask_sigma=0.3),
    "c3c_dcnv4_bf16_14": _w("c3c_dcnv4_bf16_14", 3, 2, N=64, H=14, W=14, G=16, Cg=16, Ho=14, Wo=14,
                            dtype="bf16", offset_sigma=2.0, mask_sigma=0.3),
    "c3d_dcnv4_bf16_7": _w("c3d_dcnv4_bf16_7", 3, 3, N=64, H=7, W=7, G=32, Cg=16, Ho=7, Wo=7,
                           dtype="bf16", offset_sigma=2.0, mask_sigma=0.3),
    "c4s1_dcnv3_bf16_128": _w("c4s1_dcnv3_bf16_128", 4, 1, N=8, H=128, W=128, G=16, Cg=32,
                              Ho=128, Wo=128, softmax=True, dtype="bf16",
                              offset_sigma=1.5, mask_sigma=1.0),
    "c4s2_dcnv3_bf16_128": _w("c4s2_dcnv3_bf16_128", 4, 2, N=8, H=128, W=128, G=16, Cg=32,
                              Ho=64, Wo=64, stride=2, softmax=True, dtype="bf16",
                              offset_sigma=1.5, mask_sigma=1.0),
    "c5_dcnv4_f32_56_fwdbwd": _w("c5_dcnv4_f32_56_fwdbwd", 5, 0, N=32, H=56, W=56, G=4, Cg=16,
                                 Ho=56, Wo=56, dtype="f32", offset_sigma=1.5, mask_sigma=0.3,
                                 backward=True),
}

# The headline is the DCNv4 bf16 forward at the first FlashInternImage-T
# stage (the bar is set on the DCNv4 bf16 forward); the four-stage bf16
# sweep's byte-weighted aggregate is reported beside it.
HEADLINE = "c3a_dcnv4_bf16_56"
BF16_SWEEP = ["c3a_dcnv4_bf16_56", "c3b_dcnv4_bf16_28", "c3c_dcnv4_bf16_14", "c3d_dcnv4_bf16_7"]


def normal(shape, seed: int, sigma: float, dtype: str) -> torch.Tensor:
    """float32 N(0, sigma^2) from PCG64(seed), rounded once to dtype (CPU tensor)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return torch.from_numpy(a).to(DTYPES[dtype])


def make(w: Workload, with_grad: bool | None = None) -> dict:
    """CPU tensors input, offset, mask (and grad_out) for workload w."""
    s = w.shapes()
    t = dict(input=normal(s["input"], w.seed_base + T_INPUT, 1.0, w.dtype),
             offset=normal(s["offset"], w.seed_base + T_OFFSET, w.offset_sigma, w.dtype),
             mask=normal(s["mask"], w.seed_base + T_MASK, w.mask_sigma, w.dtype))
    if with_grad or (with_grad is None and w.backward):
        t["grad_out"] = normal(s["output"], w.seed_base + T_GRAD_OUT, 1.0, w.dtype)
    return t


def pack_offset_mask(offset: torch.Tensor, mask: torch.Tensor, G: int, P: int) -> torch.Tensor:
    """DCNv4's single tensor (N, Ho, Wo, G*3P): per (pixel, group) the 2P
    offset values followed by the P mask values.  A copy, no arithmetic."""
    N, Ho, Wo = offset.shape[:3]
    return torch.cat([offset.reshape(N, Ho, Wo, G, 2 * P), mask.reshape(N, Ho, Wo, G, P)],
                     dim=-1).reshape(N, Ho, Wo, G * 3 * P).contiguous()


def unpack_offset_mask(om: torch.Tensor, G: int, P: int):
    """Inverse of pack_offset_mask: (offset (N,Ho,Wo,G*2P), mask (N,Ho,Wo,G*P))."""
    N, Ho, Wo = om.shape[:3]
    r = om.reshape(N, Ho, Wo, G, 3 * P)
    return (r[..., :2 * P].reshape(N, Ho, Wo, G * 2 * P).contiguous(),
            r[..., 2 * P:].reshape(N, Ho, Wo, G * P).contiguous())


def scaled(w: Workload, **changes) -> Workload:
    """A copy of w with some fields changed (e.g. a smaller N for a parity run)."""
    return replace(w, **changes)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (possibly half-precision) CPU tensor to float64."""
    return t.detach().cpu().to(torch.float64).numpy()
