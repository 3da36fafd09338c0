"""Independent constructions of the sampling core, used only to pin the oracle.

None of these shares code with ``oracle/`` or the HIP library.  They start from
a different description of the same operation:

* ``brute_force``: pure-Python float64 loops over the *normalised* coordinate
  form that the DCNv3 fallback walkthrough describes (page
  "没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读", trdm.cn,
  section 4 steps 1-5): an explicitly zero-padded map, reference points at
  padded pixel centres normalised by the padded size, the dilation grid
  scaled by offset_scale, offsets scaled by offset_scale / spatial size, and
  the bilinear rule of a sampler with align_corners=False (normalised u maps
  to padded pixel coordinate u*size - 0.5) with zeros outside the padded map.
* ``grid_sample_construction``: the same five steps on torch CPU in float64,
  with torch.nn.functional.grid_sample doing step 4.
* ``depthwise_conv``: the zero-offset special case, which is a grouped
  depthwise convolution (torch conv2d in float64).
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def conv_out(n, K, s, p, d):
    return (n + 2 * p - d * (K - 1) - 1) // s + 1


def _bilinear_padded(img, u_pix, v_pix):
    """img (Hp, Wp) array; (u_pix, v_pix) pixel coordinates (x, y) on it;
    zero outside.  Plain textbook bilinear interpolation."""
    Hp, Wp = img.shape
    x0 = math.floor(u_pix)
    y0 = math.floor(v_pix)
    ax = u_pix - x0
    ay = v_pix - y0
    val = 0.0
    for yy, wy in ((y0, 1.0 - ay), (y0 + 1, ay)):
        for xx, wx in ((x0, 1.0 - ax), (x0 + 1, ax)):
            if 0 <= yy < Hp and 0 <= xx < Wp:
                val += wy * wx * img[yy, xx]
    return val


def brute_force(inp, off, mask, K, s, pad, d, alpha, softmax, G, remove_center=False):
    """inp (N,H,W,C) float64; off (N,Ho,Wo,G*P*2); mask (N,Ho,Wo,G*P).
    remove_center: the K*K taps without the middle one, in the same order."""
    inp = np.asarray(inp, np.float64)
    N, H, W, C = inp.shape
    Cg = C // G
    taps = [(i, j) for i in range(K) for j in range(K)]      # kernel column i -> x, row j -> y
    if remove_center:
        taps.remove(((K - 1) // 2, (K - 1) // 2))
    P = len(taps)
    Ho, Wo = conv_out(H, K, s, pad, d), conv_out(W, K, s, pad, d)
    off = np.asarray(off, np.float64).reshape(N, Ho, Wo, G, P, 2)
    mask = np.asarray(mask, np.float64).reshape(N, Ho, Wo, G, P)
    padded = np.pad(inp, ((0, 0), (pad, pad), (pad, pad), (0, 0)))
    Hp, Wp = H + 2 * pad, W + 2 * pad
    half = (d * (K - 1)) // 2
    out = np.zeros((N, Ho, Wo, C))
    for n in range(N):
        for ho in range(Ho):
            for wo in range(Wo):
                ref_x = (half + 0.5 + wo * s) / Wp
                ref_y = (half + 0.5 + ho * s) / Hp
                for g in range(G):
                    m = mask[n, ho, wo, g].copy()
                    if softmax:
                        e = [math.exp(v - max(m)) for v in m]
                        m = np.array(e) / sum(e)
                    for p, (i, j) in enumerate(taps):
                        gx = (-half + i * d) / Wp
                        gy = (-half + j * d) / Hp
                        lx = ref_x + gx * alpha + off[n, ho, wo, g, p, 0] * alpha / Wp
                        ly = ref_y + gy * alpha + off[n, ho, wo, g, p, 1] * alpha / Hp
                        u = 2.0 * lx - 1.0
                        v = 2.0 * ly - 1.0
                        u_pix = ((u + 1.0) * Wp - 1.0) / 2.0
                        v_pix = ((v + 1.0) * Hp - 1.0) / 2.0
                        for c in range(Cg):
                            ch = g * Cg + c
                            out[n, ho, wo, ch] += m[p] * _bilinear_padded(
                                padded[n, :, :, ch], u_pix, v_pix)
    return out


def grid_sample_construction(inp, off, mask, K, s, pad, d, alpha, softmax, G):
    """The fallback's five steps with torch CPU float64 and F.grid_sample."""
    x = torch.as_tensor(np.asarray(inp, np.float64))
    N, H, W, C = x.shape
    Cg, P = C // G, K * K
    Ho, Wo = conv_out(H, K, s, pad, d), conv_out(W, K, s, pad, d)
    off = torch.as_tensor(np.asarray(off, np.float64)).reshape(N, Ho, Wo, G * P * 2)
    msk = torch.as_tensor(np.asarray(mask, np.float64)).reshape(N, Ho, Wo, G, P)
    # step 1: zero pad (N,H,W,C) on H and W
    x = F.pad(x, [0, 0, pad, pad, pad, pad])
    Hp, Wp = x.shape[1], x.shape[2]
    half = (d * (K - 1)) // 2
    # step 2: reference points at padded pixel centres, normalised; dilation grid
    ry, rx = torch.meshgrid(
        torch.linspace(half + 0.5, half + 0.5 + (Ho - 1) * s, Ho, dtype=torch.float64),
        torch.linspace(half + 0.5, half + 0.5 + (Wo - 1) * s, Wo, dtype=torch.float64),
        indexing="ij")
    ref = torch.stack((rx / Wp, ry / Hp), -1).reshape(1, Ho, Wo, 1, 2)
    gxs, gys = torch.meshgrid(
        torch.arange(K, dtype=torch.float64) * d - half,
        torch.arange(K, dtype=torch.float64) * d - half, indexing="ij")   # [i, j]
    grid = torch.stack((gxs / Wp, gys / Hp), -1).reshape(1, 1, 1, P, 2)   # p = i*K + j
    grid = grid.repeat(1, 1, 1, G, 1)                                    # (.., G*P, 2)
    loc = ref + grid * alpha
    # step 3: add offsets scaled by offset_scale / spatial size
    norm = torch.tensor([Wp, Hp], dtype=torch.float64)
    loc = loc + off.reshape(N, Ho, Wo, G * P, 2) * alpha / norm
    grids = 2 * loc - 1                                                  # (N,Ho,Wo,G*P,2)
    # step 4: fold groups into the batch and sample
    x_ = x.reshape(N, Hp * Wp, G * Cg).transpose(1, 2).reshape(N * G, Cg, Hp, Wp)
    g_ = grids.reshape(N, Ho * Wo, G, P, 2).transpose(1, 2).reshape(N * G, Ho * Wo, P, 2)
    sampled = F.grid_sample(x_, g_, mode="bilinear", padding_mode="zeros",
                            align_corners=False)                          # (N*G, Cg, Ho*Wo, P)
    # step 5: mask-weighted sum over P, back to channels-last
    if softmax:
        msk = torch.softmax(msk, -1)
    m_ = msk.reshape(N, Ho * Wo, G, P).transpose(1, 2).reshape(N * G, 1, Ho * Wo, P)
    out = (sampled * m_).sum(-1)                                         # (N*G, Cg, Ho*Wo)
    out = out.reshape(N, G * Cg, Ho * Wo).transpose(1, 2).reshape(N, Ho, Wo, G * Cg)
    return out.numpy()


def depthwise_conv(inp, m_gp, K, s, pad, d, G):
    """Zero offsets and a pixel-invariant mask m_gp (G, P) reduce the core to a
    depthwise conv whose tap at kernel row j, column i carries m[g, i*K + j]."""
    x = torch.as_tensor(np.asarray(inp, np.float64)).permute(0, 3, 1, 2)   # NCHW
    C = x.shape[1]
    Cg = C // G
    wt = torch.zeros(C, 1, K, K, dtype=torch.float64)
    for c in range(C):
        g = c // Cg
        for i in range(K):
            for j in range(K):
                wt[c, 0, j, i] = float(m_gp[g, i * K + j])
    y = F.conv2d(x, wt, stride=s, padding=pad, dilation=d, groups=C)
    return y.permute(0, 2, 3, 1).numpy()
