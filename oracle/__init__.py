"""CPU oracle for the DCNv3/DCNv4 deformable sampling core.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``deformable_convolution_core_amd``; it wraps the
plain C loops of ``dcn_oracle.c`` (binary64 throughout, coordinates optionally
in the binary32 order the library documents) with ctypes and numpy.

The computation follows the five steps of the DCNv3 pure-PyTorch fallback as
read on the page "没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读"
(trdm.cn), section 4, with the mask softmax of section 3 item 3 for DCNv3 and
the raw (unnormalised) mask of DCNv4 ("DCNv4高效实践指南", seekfood.cn, core
architecture section).  The header of ``dcn_oracle.c`` states the formula.

Every function here is pinned by ``tests/test_oracle_*.py`` against things
other than itself: a float64 brute-force written from the normalised-grid form,
the page's grid_sample construction rebuilt on torch CPU, the depthwise conv2d
special case, hand-worked golden values and exact invariants.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dcn_oracle.c")
_LIB = os.path.join(_HERE, "libdcn_oracle.so")
_lib = None

COORD_EXACT = 0     # sampling coordinates in binary64
COORD_BINARY32 = 1  # sampling coordinates in the library's binary32 order


def build(force: bool = True) -> str:
    """Compile dcn_oracle.c with gcc (-O2, OpenMP, no fp contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-std=c99", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _open(path):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i, d = ctypes.c_int, ctypes.c_double
    lib.oracle_out_size.argtypes = [i, i, i, i, i]
    lib.oracle_out_size.restype = i
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i
    lib.oracle_forward.argtypes = [dp, dp, dp, dp, dp] + [i] * 9 + [d, i, i, i]
    lib.oracle_forward.restype = i
    lib.oracle_backward.argtypes = [dp] * 11 + [i] * 9 + [d, i, i, i]
    lib.oracle_backward.restype = i
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _open(_LIB)
    return _lib


@contextlib.contextmanager
def library_override(path):
    """Route the wrappers to another build of dcn_oracle.c (used by the
    mutation tests, which compile deliberately broken copies)."""
    global _lib
    saved = _lib
    _lib = _open(path)
    try:
        yield
    finally:
        _lib = saved


def _f64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    """Threads the oracle's OpenMP loops run on."""
    return int(_load().oracle_max_threads())


def out_size(n: int, K: int, stride: int, pad: int, dilation: int) -> int:
    """Output extent along one axis (0 if the geometry is invalid)."""
    return int(_load().oracle_out_size(n, K, stride, pad, dilation))


def _geometry(input, K, stride, pad, dilation):
    N, H, W, C = input.shape
    Ho, Wo = out_size(H, K, stride, pad, dilation), out_size(W, K, stride, pad, dilation)
    if Ho <= 0 or Wo <= 0:
        raise ValueError("empty output for this geometry")
    return N, H, W, C, Ho, Wo


def forward(input, offset, mask, *, K, stride, pad, dilation, offset_scale,
            softmax, group, coord_mode=COORD_BINARY32, with_absum=True, remove_center=False):
    """Reference forward.

    input (N,H,W,G*Cg); offset (N,Ho,Wo,G*P*2) or (N,Ho,Wo,G,P,2) as (dx,dy)
    pixel offsets; mask (N,Ho,Wo,G*P).  P = K*K, or K*K - 1 with
    remove_center (odd K; the centre tap is left out, the other taps keep
    their order).  Values are read as float64 (pass the already dtype-rounded
    tensors).  Returns (out, absum) as float64 arrays of shape
    (N,Ho,Wo,G*Cg); absum is None unless with_absum.
    """
    x = _f64(input)
    N, H, W, C, Ho, Wo = _geometry(x, K, stride, pad, dilation)
    G = int(group)
    if C % G:
        raise ValueError("channels not divisible by group")
    Cg, P = C // G, K * K - (1 if remove_center else 0)
    off = _f64(offset).reshape(N, Ho, Wo, G * P * 2)
    msk = _f64(mask).reshape(N, Ho, Wo, G * P)
    out = np.empty((N, Ho, Wo, C), np.float64)
    absum = np.empty_like(out) if with_absum else None
    rc = _load().oracle_forward(_ptr(x), _ptr(off), _ptr(msk), _ptr(out), _ptr(absum),
                                N, H, W, G, Cg, K, stride, pad, dilation,
                                float(offset_scale), int(bool(softmax)), int(coord_mode),
                                int(bool(remove_center)))
    if rc != 0:
        raise ValueError("oracle_forward rejected the sizes")
    return out, absum


def backward(input, offset, mask, grad_out, *, K, stride, pad, dilation, offset_scale,
             softmax, group, coord_mode=COORD_BINARY32, with_scales=True, remove_center=False):
    """Reference backward.  Returns a dict with grad_input, grad_offset,
    grad_mask (float64, shaped like input / offset / mask as passed) and, when
    with_scales, gi_abs, gi_cnt, goff_abs, gmask_abs error scales."""
    x = _f64(input)
    N, H, W, C, Ho, Wo = _geometry(x, K, stride, pad, dilation)
    G = int(group)
    Cg, P = C // G, K * K - (1 if remove_center else 0)
    off_shape, msk_shape = np.shape(offset), np.shape(mask)
    off = _f64(offset).reshape(N, Ho, Wo, G * P * 2)
    msk = _f64(mask).reshape(N, Ho, Wo, G * P)
    go = _f64(grad_out).reshape(N, Ho, Wo, C)
    gi = np.empty_like(x)
    goff = np.empty_like(off)
    gm = np.empty_like(msk)
    sc = {}
    if with_scales:
        sc = dict(gi_abs=np.empty_like(x), gi_cnt=np.empty_like(x),
                  goff_abs=np.empty_like(off), gmask_abs=np.empty_like(msk))
    rc = _load().oracle_backward(
        _ptr(x), _ptr(off), _ptr(msk), _ptr(go), _ptr(gi), _ptr(goff), _ptr(gm),
        _ptr(sc.get("gi_abs")), _ptr(sc.get("gi_cnt")), _ptr(sc.get("goff_abs")),
        _ptr(sc.get("gmask_abs")),
        N, H, W, G, Cg, K, stride, pad, dilation,
        float(offset_scale), int(bool(softmax)), int(coord_mode), int(bool(remove_center)))
    if rc != 0:
        raise ValueError("oracle_backward rejected the sizes")
    res = dict(grad_input=gi, grad_offset=goff.reshape(off_shape),
               grad_mask=gm.reshape(msk_shape))
    if with_scales:
        res.update(gi_abs=sc["gi_abs"], gi_cnt=sc["gi_cnt"],
                   goff_abs=sc["goff_abs"].reshape(off_shape),
                   gmask_abs=sc["gmask_abs"].reshape(msk_shape))
    return res
