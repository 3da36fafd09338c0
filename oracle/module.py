"""CPU oracle of the DCNv4 layer around the sampling core, in float64.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares
no code with the HIP library or its Python binding; the sampling core itself
is the C oracle of this package.

The layer, as the pages describe it (our plainest reading where they are
brief):

* "没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读" (trdm.cn),
  section 3: the module first projects its input linearly and keeps that
  projection (x_proj); a separate branch predicts the offsets and the mask
  with fully connected layers; the core samples the projection; an optional
  sigmoid gate (center_feature_scale) blends the centre pixel's projected
  features with the sampled result; an output projection keeps the shape
  (N, H, W, C).
* "告别DCNv3的卡顿：实测DCNv4在A100上3倍提速…" (framerc.cn), section 1: DCNv4
  merges the offset and weight layers into one and removes the LN-GELU of the
  offset branch, and its core takes one offset+weight tensor with a raw mask.

So, for input x (N, H, W, C), C = G*Cg, linear(a, W, b) = a @ W.T + b:

    v   = linear(x, Wv, bv)                    (N, H, W, C)
    om  = linear(x, Wom, bom)                  (N, H, W, G*3P): per (pixel,
          group) 2P offsets as (dx, dy) pairs, then P raw mask values
    y   = core(v, om)                          stride 1, output grid = input grid
    s   = sigmoid(linear(x, Wc, bc))           (N, H, W, G), only with
          center_feature_scale; y = y * (1 - s) + v * s, s repeated over the
          group's Cg channels
    out = linear(y, Wo, bo)

Every function is pinned in tests/test_oracle_module.py against closed forms
and float64 central finite differences of the whole layer.
"""
from __future__ import annotations

import numpy as np

import oracle

PARAMS = ("Wv", "bv", "Wom", "bom", "Wc", "bc", "Wo", "bo")


def linear(a, W, b):
    """a @ W.T + b over the last axis of a."""
    return a @ W.T + b


def linear_backward(a, W, gy):
    """Gradients (ga, gW, gb) of linear(a, W, b) for upstream gy."""
    a2 = a.reshape(-1, a.shape[-1])
    g2 = gy.reshape(-1, gy.shape[-1])
    return gy @ W, g2.T @ a2, g2.sum(axis=0)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def gate_forward(y, v, z, G):
    """y * (1 - s) + v * s with s = sigmoid(z), z (..., G), y and v (..., G*Cg).
    1 - s is evaluated as sigmoid(-z), the same number without the
    cancellation of 1 - s when s is close to 1."""
    sh = y.shape
    Cg = sh[-1] // G
    s = sigmoid(z)[..., None]
    t = sigmoid(-z)[..., None]
    yg = y.reshape(*sh[:-1], G, Cg)
    vg = v.reshape(*sh[:-1], G, Cg)
    return (yg * t + vg * s).reshape(sh)


def gate_backward(y, v, z, gout, G):
    """Gradients (gy, gv, gz) of gate_forward (ds/dz = s * (1 - s))."""
    sh = y.shape
    Cg = sh[-1] // G
    s = sigmoid(z)[..., None]
    t = sigmoid(-z)[..., None]
    yg = y.reshape(*sh[:-1], G, Cg)
    vg = v.reshape(*sh[:-1], G, Cg)
    go = gout.reshape(*sh[:-1], G, Cg)
    gy = (go * t).reshape(sh)
    gv = (go * s).reshape(sh)
    gz = (go * (vg - yg)).sum(axis=-1) * (s[..., 0] * t[..., 0])
    return gy, gv, gz


def split_records(om, G, P):
    """Packed (N, H, W, G*3P) -> offset (N, H, W, G*2P), mask (N, H, W, G*P)."""
    N, H, W = om.shape[:3]
    r = om.reshape(N, H, W, G, 3 * P)
    return (np.ascontiguousarray(r[..., :2 * P]).reshape(N, H, W, G * 2 * P),
            np.ascontiguousarray(r[..., 2 * P:]).reshape(N, H, W, G * P))


def join_records(off, mask, G, P):
    """Inverse of split_records."""
    N, H, W = off.shape[:3]
    return np.concatenate([off.reshape(N, H, W, G, 2 * P), mask.reshape(N, H, W, G, P)],
                          axis=-1).reshape(N, H, W, G * 3 * P)


def _core_kw(cfg):
    K, d = cfg["kernel_size"], cfg.get("dilation", 1)
    return dict(K=K, stride=1, pad=cfg.get("pad", d * (K - 1) // 2), dilation=d,
                offset_scale=cfg.get("offset_scale", 1.0), softmax=False, group=cfg["group"],
                remove_center=cfg.get("remove_center", False),
                coord_mode=cfg.get("coord_mode", oracle.COORD_BINARY32))


def points(cfg):
    K = cfg["kernel_size"]
    return K * K - (1 if cfg.get("remove_center", False) else 0)


def module_forward(x, p, cfg):
    """The layer's output and its intermediates (dict), all float64.

    x: (N, H, W, C); p: dict of the parameters in PARAMS (Wc, bc may be None
    when cfg["center_feature_scale"] is false); cfg: kernel_size, group,
    dilation, pad (default: the one keeping the grid), offset_scale,
    remove_center, center_feature_scale, coord_mode."""
    x = np.asarray(x, np.float64)
    G, P = cfg["group"], points(cfg)
    v = linear(x, p["Wv"], p["bv"])
    om = linear(x, p["Wom"], p["bom"])
    off, mask = split_records(om, G, P)
    y, _ = oracle.forward(v, off, mask, with_absum=False, **_core_kw(cfg))
    if y.shape != x.shape:
        raise ValueError("the layer needs a geometry that keeps the grid (Ho = H, Wo = W)")
    z = None
    yg = y
    if cfg.get("center_feature_scale", False):
        z = linear(x, p["Wc"], p["bc"])
        yg = gate_forward(y, v, z, G)
    out = linear(yg, p["Wo"], p["bo"])
    return dict(out=out, v=v, om=om, y=y, z=z, yg=yg)


def module_backward(x, p, cfg, gout):
    """Gradients of the layer for upstream gout: dict with 'x' and one entry
    per parameter (float64)."""
    x = np.asarray(x, np.float64)
    G, P = cfg["group"], points(cfg)
    f = module_forward(x, p, cfg)
    g = {}
    gyg, g["Wo"], g["bo"] = linear_backward(f["yg"], p["Wo"], gout)
    gx = np.zeros_like(x)
    if cfg.get("center_feature_scale", False):
        gy, gv, gz = gate_backward(f["y"], f["v"], f["z"], gyg, G)
        gxz, g["Wc"], g["bc"] = linear_backward(x, p["Wc"], gz)
        gx += gxz
    else:
        gy, gv = gyg, np.zeros_like(f["v"])
    off, mask = split_records(f["om"], G, P)
    r = oracle.backward(f["v"], off, mask, gy, with_scales=False, **_core_kw(cfg))
    gv = gv + r["grad_input"]
    gom = join_records(r["grad_offset"], r["grad_mask"], G, P)
    gxo, g["Wom"], g["bom"] = linear_backward(x, p["Wom"], gom)
    gxv, g["Wv"], g["bv"] = linear_backward(x, p["Wv"], gv)
    g["x"] = gx + gxo + gxv
    return g
