"""Pins of the DCNv4-layer oracle (oracle/module.py) against things other
than itself: closed forms of the gate, the identity layer, the layer as a
depthwise convolution between two projections (torch conv2d in float64), and
float64 central finite differences of the whole layer for the input and every
parameter.  A few planted mistakes in the layer's backward must each fail
the finite-difference pin."""
import contextlib

import numpy as np
import pytest
import torch

import oracle
from oracle import module as om_oracle


def params(C, G, P, cfs, seed, scale=0.3):
    rng = np.random.default_rng(seed)
    p = dict(Wv=rng.standard_normal((C, C)) * scale, bv=rng.standard_normal(C) * 0.1,
             Wom=rng.standard_normal((G * 3 * P, C)) * 0.2, bom=rng.standard_normal(G * 3 * P) * 0.5,
             Wo=rng.standard_normal((C, C)) * scale, bo=rng.standard_normal(C) * 0.1,
             Wc=None, bc=None)
    if cfs:
        p["Wc"] = rng.standard_normal((G, C)) * 0.3
        p["bc"] = rng.standard_normal(G) * 0.3
    return p


# ------------------------------------------------------------------ gate
def test_gate_closed_forms():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((2, 3, 4, 12))
    v = rng.standard_normal((2, 3, 4, 12))
    G = 3
    big = np.full((2, 3, 4, G), 40.0)
    # s = 1 - 4.2e-18: the result is v to within one rounding
    np.testing.assert_allclose(om_oracle.gate_forward(y, v, big, G), v, rtol=0, atol=1e-16)
    np.testing.assert_allclose(om_oracle.gate_forward(y, v, -big, G), y, rtol=0, atol=1e-16)
    np.testing.assert_allclose(om_oracle.gate_forward(y, v, np.zeros_like(big), G), (y + v) / 2,
                               rtol=1e-15, atol=0)
    # one group gated open, the others closed: the channel blocks follow their group
    z = -big.copy()
    z[..., 1] = 40.0
    out = om_oracle.gate_forward(y, v, z, G)
    np.testing.assert_allclose(out[..., 4:8], v[..., 4:8], atol=1e-16)
    np.testing.assert_allclose(out[..., :4], y[..., :4], atol=1e-16)
    np.testing.assert_allclose(out[..., 8:], y[..., 8:], atol=1e-16)


def test_gate_backward_finite_difference():
    rng = np.random.default_rng(6)
    G, shape = 2, (1, 2, 3, 8)
    y, v = rng.standard_normal(shape), rng.standard_normal(shape)
    z = rng.standard_normal(shape[:-1] + (G,))
    go = rng.standard_normal(shape)
    gy, gv, gz = om_oracle.gate_backward(y, v, z, go, G)
    h = 1e-6

    def loss(yy, vv, zz):
        return float((om_oracle.gate_forward(yy, vv, zz, G) * go).sum())

    for arr, grad in ((y, gy), (v, gv), (z, gz)):
        for idx in [tuple(rng.integers(0, s) for s in arr.shape) for _ in range(6)]:
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            args_p = [plus if a is arr else a for a in (y, v, z)]
            args_m = [minus if a is arr else a for a in (y, v, z)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * (1 + abs(fd)), (idx, fd, grad[idx])


# ------------------------------------------------------------------ layer
def identity_params(C, G, K, rc):
    """Projections = identity, offset branch = constant record: zero offsets,
    mask one at the centre tap (zero elsewhere); without remove_center the
    core is then the identity."""
    P = K * K - (1 if rc else 0)
    rec = np.zeros((G, 3 * P))
    rec[:, 2 * P + (K * K - 1) // 2] = 1.0
    return dict(Wv=np.eye(C), bv=np.zeros(C), Wom=np.zeros((G * 3 * P, C)), bom=rec.reshape(-1),
                Wo=np.eye(C), bo=np.zeros(C), Wc=np.zeros((G, C)), bc=np.zeros(G))


@pytest.mark.parametrize("cfs", [False, True])
def test_identity_layer(cfs):
    rng = np.random.default_rng(7)
    N, H, W, G, Cg, K = 2, 5, 6, 2, 4, 3
    x = rng.standard_normal((N, H, W, G * Cg))
    cfg = dict(kernel_size=K, group=G, center_feature_scale=cfs)
    out = om_oracle.module_forward(x, identity_params(G * Cg, G, K, False), cfg)["out"]
    # with the gate: s = sigmoid(0) = 1/2 blends the core output (= v = x) with v
    np.testing.assert_array_equal(out, x)


@pytest.mark.parametrize("rc", [False, True])
def test_layer_is_projected_depthwise_conv(rc):
    """Constant records (zero offsets, pixel-invariant mask) turn the core into
    a depthwise convolution; with random projections the layer is then
    Wo . dwconv(Wv x + bv) + bo, computed independently with torch conv2d.
    remove_center: the centre weight of the kernel is zero."""
    rng = np.random.default_rng(8 + rc)
    N, H, W, G, Cg, K, d = 2, 7, 6, 2, 3, 3, 2
    C = G * Cg
    P = K * K - (1 if rc else 0)
    p = params(C, G, P, False, 11)
    p["Wom"][:] = 0.0
    mw = rng.standard_normal((G, P))
    rec = np.concatenate([np.zeros((G, 2 * P)), mw], axis=1)
    p["bom"] = rec.reshape(-1)
    cfg = dict(kernel_size=K, group=G, dilation=d, remove_center=rc, coord_mode=oracle.COORD_EXACT)
    x = rng.standard_normal((N, H, W, C))
    out = om_oracle.module_forward(x, p, cfg)["out"]

    v = torch.from_numpy(x @ p["Wv"].T + p["bv"]).permute(0, 3, 1, 2)
    taps = [(i, j) for i in range(K) for j in range(K) if not (rc and i == j == (K - 1) // 2)]
    ker = torch.zeros(C, 1, K, K, dtype=torch.float64)
    for g in range(G):
        for q, (i, j) in enumerate(taps):
            ker[g * Cg:(g + 1) * Cg, 0, j, i] = mw[g, q]     # i: kernel column (x), j: row (y)
    y = torch.nn.functional.conv2d(v, ker, padding=d * (K - 1) // 2, dilation=d, groups=C)
    want = y.permute(0, 2, 3, 1).numpy() @ p["Wo"].T + p["bo"]
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


LAYERS = [  # N, H, W, G, Cg, K, remove_center, center_feature_scale, offset_scale
    (1, 5, 6, 2, 3, 3, False, True, 1.0),
    (2, 4, 5, 1, 4, 3, True, False, 0.7),
    (1, 4, 4, 2, 2, 5, False, True, 1.3),
]


def fd_check(x, p, cfg, gout, g, rng, n_per=5, h=1e-6):
    """Central differences of <layer(x), gout> against g for x and every parameter."""
    def loss(xx, pp):
        return float((om_oracle.module_forward(xx, pp, cfg)["out"] * gout).sum())

    worst = 0.0
    targets = [("x", x)] + [(k, p[k]) for k in om_oracle.PARAMS if p[k] is not None]
    for name, arr in targets:
        for _ in range(n_per):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            keep = arr[idx]
            arr[idx] = keep + h
            lp = loss(x, p)
            arr[idx] = keep - h
            lm = loss(x, p)
            arr[idx] = keep
            fd = (lp - lm) / (2 * h)
            err = abs(fd - g[name][idx]) / (1e-3 + abs(fd))
            worst = max(worst, err)
            if err > 1e-5:
                return False, (name, idx, fd, g[name][idx])
    return True, worst


@pytest.mark.parametrize("case", LAYERS)
def test_layer_backward_finite_difference(case):
    N, H, W, G, Cg, K, rc, cfs, alpha = case
    C, P = G * Cg, K * K - (1 if rc else 0)
    rng = np.random.default_rng(100 + K + 2 * rc + 4 * cfs)
    p = params(C, G, P, cfs, 12 + K)
    x = rng.standard_normal((N, H, W, C))
    cfg = dict(kernel_size=K, group=G, remove_center=rc, center_feature_scale=cfs, offset_scale=alpha,
               coord_mode=oracle.COORD_EXACT)
    gout = rng.standard_normal((N, H, W, C))
    g = om_oracle.module_backward(x, p, cfg, gout)
    ok, info = fd_check(x, p, cfg, gout, g, rng)
    assert ok, info


# Planted mistakes in the layer's backward, each of which the finite-difference
# pin must catch.
@contextlib.contextmanager
def patched(name, fn):
    saved = getattr(om_oracle, name)
    setattr(om_oracle, name, fn)
    try:
        yield
    finally:
        setattr(om_oracle, name, saved)


def _orig(name):
    return getattr(om_oracle, name)


MUTANTS = {
    "weight_grad_transposed": ("linear_backward",
                               lambda f: (lambda a, W, gy: (lambda r: (r[0], r[1].T if r[1].shape[0] == r[1].shape[1]
                                                                       else r[1] * 1.01, r[2]))(f(a, W, gy)))),
    "bias_grad_dropped": ("linear_backward",
                          lambda f: (lambda a, W, gy: (lambda r: (r[0], r[1], 0 * r[2]))(f(a, W, gy)))),
    "gate_grad_sign": ("gate_backward",
                       lambda f: (lambda y, v, z, go, G: (lambda r: (r[0], r[1], -r[2]))(f(y, v, z, go, G)))),
    "gate_value_path_dropped": ("gate_backward",
                                lambda f: (lambda y, v, z, go, G: (lambda r: (r[0], 0 * r[1], r[2]))(f(y, v, z, go, G)))),
    "records_swapped": ("join_records",
                        lambda f: (lambda off, mask, G, P: f(off, mask, G, P)[..., ::-1].copy())),
}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_backward_mistakes_are_caught(mutant):
    name, make = MUTANTS[mutant]
    N, H, W, G, Cg, K, rc, cfs, alpha = LAYERS[0]
    C, P = G * Cg, K * K
    rng = np.random.default_rng(300)
    p = params(C, G, P, cfs, 301)
    x = rng.standard_normal((N, H, W, C))
    cfg = dict(kernel_size=K, group=G, center_feature_scale=cfs, coord_mode=oracle.COORD_EXACT)
    gout = rng.standard_normal((N, H, W, C))
    with patched(name, make(_orig(name))):
        g = om_oracle.module_backward(x, p, cfg, gout)
    ok, _ = fd_check(x, p, cfg, gout, g, rng, n_per=8)
    assert not ok, mutant
