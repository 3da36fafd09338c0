"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it pins.  Together they are meant to catch a plausible
mistake anywhere in the oracle: a dropped corner or term, a wrong sign, x and
y swapped, the wrong point order, the wrong centre (c0) or pixel-centre
convention, offset_scale applied to the wrong term, softmax applied wrongly,
or a wrong boundary rule.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import independent as ind

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def rand_case(rng, N, H, W, G, Cg, K, s, p, d, off_sigma=1.5, mask_sigma=1.0, dyadic=False, rc=False):
    Ho, Wo = ind.conv_out(H, K, s, p, d), ind.conv_out(W, K, s, p, d)
    P = K * K - (1 if rc else 0)
    x = rng.standard_normal((N, H, W, G * Cg))
    off = rng.standard_normal((N, Ho, Wo, G * P * 2)) * off_sigma
    if dyadic:  # exactly representable in binary32 -> binary32 coordinates are exact
        off = np.round(off * 256) / 256
    m = rng.standard_normal((N, Ho, Wo, G * P)) * mask_sigma
    return x, off, m


def fwd(x, off, m, K, s, p, d, a, sm, G, mode=oracle.COORD_EXACT, rc=False):
    out, _ = oracle.forward(x, off, m, K=K, stride=s, pad=p, dilation=d, offset_scale=a,
                            softmax=sm, group=G, coord_mode=mode, with_absum=False, remove_center=rc)
    return out


GEOMS = [  # N, H, W, G, Cg, K, s, pad, d, alpha, softmax
    (1, 5, 6, 1, 2, 3, 1, 1, 1, 1.0, True),
    (2, 6, 5, 2, 3, 3, 2, 1, 1, 0.75, False),
    (1, 7, 7, 2, 1, 3, 1, 2, 2, 1.25, True),
    (1, 6, 7, 1, 2, 5, 1, 2, 1, 0.5, False),
    (1, 4, 5, 3, 1, 1, 1, 0, 1, 1.0, False),
    (1, 7, 6, 1, 2, 2, 1, 1, 1, 1.0, True),   # even K
    (1, 6, 6, 2, 2, 3, 3, 0, 1, 1.0, True),   # stride 3, no padding
]


@pytest.mark.parametrize("geom", GEOMS)
def test_bruteforce_normalised_form_exact_coords(geom):
    """Oracle (binary64 coordinates) == brute force written from the
    normalised-grid form of the fallback, on tiny shapes."""
    N, H, W, G, Cg, K, s, p, d, a, sm = geom
    rng = np.random.default_rng(11 + K + 7 * s)
    x, off, m = rand_case(rng, N, H, W, G, Cg, K, s, p, d)
    ref = ind.brute_force(x, off, m, K, s, p, d, a, sm, G)
    got = fwd(x, off, m, K, s, p, d, a, sm, G)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("geom", GEOMS)
def test_bruteforce_binary32_coords_dyadic(geom):
    """With dyadic offsets and offset_scale the binary32 coordinate order is
    exact, so the oracle's kernel-order mode must also hit the brute force."""
    N, H, W, G, Cg, K, s, p, d, a, sm = geom
    rng = np.random.default_rng(23 + K)
    x, off, m = rand_case(rng, N, H, W, G, Cg, K, s, p, d, dyadic=True)
    ref = ind.brute_force(x, off, m, K, s, p, d, a, sm, G)
    got = fwd(x, off, m, K, s, p, d, a, sm, G, mode=oracle.COORD_BINARY32)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


RC_GEOMS = [  # N, H, W, G, Cg, K, s, pad, d, alpha, softmax  (odd K: remove_center)
    (1, 6, 7, 2, 2, 3, 1, 1, 1, 1.0, True),
    (2, 7, 6, 1, 3, 3, 2, 1, 1, 0.75, False),
    (1, 8, 7, 1, 2, 5, 1, 2, 1, 1.25, False),
    (1, 9, 8, 2, 1, 3, 1, 2, 2, 1.0, True),
]


@pytest.mark.parametrize("geom", RC_GEOMS)
def test_bruteforce_remove_center(geom):
    """remove_center (DCNv4 option): the oracle against the brute force
    written from the normalised-grid form with the middle tap left out."""
    N, H, W, G, Cg, K, s, p, d, a, sm = geom
    rng = np.random.default_rng(31 + K + 5 * s)
    x, off, m = rand_case(rng, N, H, W, G, Cg, K, s, p, d, rc=True)
    ref = ind.brute_force(x, off, m, K, s, p, d, a, sm, G, remove_center=True)
    got = fwd(x, off, m, K, s, p, d, a, sm, G, rc=True)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("geom", RC_GEOMS)
def test_remove_center_is_full_grid_without_centre(geom):
    """Leaving the centre tap out equals the full grid with the centre's
    weight at zero: a raw mask of 0 there, or a softmax logit of -inf (whose
    exponential is 0, so the other taps normalise over the same P - 1)."""
    N, H, W, G, Cg, K, s, p, d, a, sm = geom
    rng = np.random.default_rng(37 + K)
    x, off, m = rand_case(rng, N, H, W, G, Cg, K, s, p, d, rc=True)
    Ho, Wo = off.shape[1], off.shape[2]
    P, c = K * K - 1, (K * K - 1) // 2
    off_full = np.insert(off.reshape(N, Ho, Wo, G, P, 2), c, 0.0, axis=4).reshape(N, Ho, Wo, -1)
    m_full = np.insert(m.reshape(N, Ho, Wo, G, P), c, -np.inf if sm else 0.0, axis=4).reshape(N, Ho, Wo, -1)
    got = fwd(x, off, m, K, s, p, d, a, sm, G, rc=True)
    full = fwd(x, off_full, m_full, K, s, p, d, a, sm, G)
    assert np.max(np.abs(got - full)) <= 1e-13 * max(1.0, np.max(np.abs(full)))


def test_binary32_coords_close_for_general_offsets():
    """Non-dyadic offsets and offset_scale 0.7: binary32 coordinates differ
    from exact ones by about |x| * 2^-24, so outputs differ by at most that
    times the local slope of the map."""
    rng = np.random.default_rng(5)
    N, H, W, G, Cg, K, s, p, d = 2, 9, 8, 2, 3, 3, 1, 1, 1
    x, off, m = rand_case(rng, N, H, W, G, Cg, K, s, p, d)
    ref = fwd(x, off, m, K, s, p, d, 0.7, True, G)
    got = fwd(x, off, m, K, s, p, d, 0.7, True, G, mode=oracle.COORD_BINARY32)
    slope = 2 * np.max(np.abs(x))
    assert np.max(np.abs(got - ref)) <= 4 * 12 * 2.0 ** -24 * slope * K * K


@pytest.mark.parametrize("geom", GEOMS)
def test_grid_sample_construction(geom):
    """Oracle == the page's five steps rebuilt on torch CPU float64 with
    F.grid_sample (align_corners=False, zeros padding)."""
    N, H, W, G, Cg, K, s, p, d, a, sm = geom
    rng = np.random.default_rng(101 + K)
    x, off, m = rand_case(rng, N, H, W, G, Cg, K, s, p, d, off_sigma=2.0)
    ref = ind.grid_sample_construction(x, off, m, K, s, p, d, a, sm, G)
    got = fwd(x, off, m, K, s, p, d, a, sm, G)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("geom", [(2, 9, 7, 2, 3, 3, 1, 1, 1), (1, 10, 11, 3, 2, 3, 2, 1, 1),
                                  (1, 9, 9, 1, 4, 3, 1, 2, 2), (1, 8, 9, 2, 2, 5, 2, 2, 1),
                                  (1, 7, 7, 1, 3, 1, 1, 0, 1)])
def test_zero_offsets_is_depthwise_conv(geom):
    """Zero offsets + pixel-invariant raw mask == grouped depthwise conv2d
    with the tap at (row j, column i) weighted by mask[g, i*K + j].  Pins
    stride, padding, dilation, c0 and the point order."""
    N, H, W, G, Cg, K, s, p, d = geom
    rng = np.random.default_rng(7)
    Ho, Wo, P = ind.conv_out(H, K, s, p, d), ind.conv_out(W, K, s, p, d), K * K
    x = rng.standard_normal((N, H, W, G * Cg))
    m_gp = rng.standard_normal((G, P))
    mask = np.broadcast_to(m_gp.reshape(1, 1, 1, G * P), (N, Ho, Wo, G * P))
    off = np.zeros((N, Ho, Wo, G * P * 2))
    ref = ind.depthwise_conv(x, m_gp, K, s, p, d, G)
    for mode in (oracle.COORD_EXACT, oracle.COORD_BINARY32):
        got = fwd(x, off, mask, K, s, p, d, 1.0, False, G, mode=mode)
        assert got.shape == ref.shape
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_out_size_matches_conv2d():
    for (n, K, s, p, d) in [(8, 3, 1, 1, 1), (128, 3, 2, 1, 1), (7, 3, 1, 1, 1), (9, 5, 2, 2, 1),
                            (10, 3, 3, 0, 2), (5, 1, 1, 0, 1), (6, 4, 1, 1, 1), (2, 3, 1, 0, 1)]:
        assert oracle.out_size(n, K, s, p, d) == max(ind.conv_out(n, K, s, p, d), 0)
    assert oracle.out_size(0, 3, 1, 1, 1) == 0
    assert oracle.out_size(8, 3, 0, 1, 1) == 0


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_golden(case):
    """Values derived by hand (tests/golden/hand_worked.json)."""
    K, s, p, d = case["K"], case["stride"], case["pad"], case["dilation"]
    x = np.array(case["input"], np.float64)[None, :, :, None]
    H, W = x.shape[1:3]
    Ho, Wo, P = ind.conv_out(H, K, s, p, d), ind.conv_out(W, K, s, p, d), K * K
    if case["offset"] == "zeros":
        off = np.zeros((1, Ho, Wo, P * 2))
    else:
        off = np.array(case["offset"], np.float64).reshape(1, Ho, Wo, P * 2)
    if isinstance(case["mask"], str):
        vals = np.array([float(v) for v in case["mask"].split(":")[1].split(",")])
        mask = np.broadcast_to(vals, (1, Ho, Wo, P))
    else:
        mask = np.array(case["mask"], np.float64).reshape(1, Ho, Wo, P)
    exp = np.array(case["expected"], np.float64)
    for mode in (oracle.COORD_EXACT, oracle.COORD_BINARY32):
        got = fwd(x, off, mask, K, s, p, d, case["offset_scale"], case["softmax"], 1, mode)
        np.testing.assert_allclose(got[0, :, :, 0], exp, rtol=0, atol=1e-13)


def identity_case(rng, N, H, W, G, Cg, softmax):
    x = rng.standard_normal((N, H, W, G * Cg))
    off = np.zeros((N, H, W, G * 9 * 2))
    if softmax:
        m = np.full((N, H, W, G, 9), -1e4)
        m[..., 4] = 0.0
    else:
        m = np.zeros((N, H, W, G, 9))
        m[..., 4] = 1.0
    return x, off, m.reshape(N, H, W, G * 9)


@pytest.mark.parametrize("softmax", [False, True])
def test_identity_bit_exact(softmax):
    """Zero offsets and a one-hot centre mask reproduce the input exactly."""
    rng = np.random.default_rng(3)
    x, off, m = identity_case(rng, 2, 6, 7, 3, 2, softmax)
    for mode in (oracle.COORD_EXACT, oracle.COORD_BINARY32):
        got = fwd(x, off, m, 3, 1, 1, 1, 1.0, softmax, 3, mode)
        assert np.array_equal(got, x)


def test_integer_offsets_are_pure_shifts():
    """Integer offsets with a one-hot mask shift the map; beyond the edge is 0."""
    rng = np.random.default_rng(4)
    N, H, W, G, Cg = 1, 7, 8, 2, 2
    x = rng.standard_normal((N, H, W, G * Cg))
    for (p, dx, dy) in [(4, 1, 0), (4, -2, 3), (0, 0, 0), (8, -3, -1), (2, 2, 2)]:
        i, j = divmod(p, 3)
        off = np.zeros((N, H, W, G, 9, 2))
        off[..., p, 0] = dx
        off[..., p, 1] = dy
        m = np.zeros((N, H, W, G, 9))
        m[..., p] = 1.0
        got = fwd(x, off.reshape(N, H, W, -1), m.reshape(N, H, W, -1), 3, 1, 1, 1, 1.0, False, G,
                  oracle.COORD_BINARY32)
        exp = np.zeros_like(x)
        sx, sy = (i - 1) + dx, (j - 1) + dy       # total displacement of the tap
        for yy in range(H):
            for xx in range(W):
                ys, xs = yy + sy, xx + sx
                if 0 <= ys < H and 0 <= xs < W:
                    exp[:, yy, xx] = x[:, ys, xs]
        assert np.array_equal(got, exp), (p, dx, dy)


def test_far_outside_is_zero_and_nonfinite_coords_skip():
    rng = np.random.default_rng(8)
    N, H, W, G, Cg = 1, 5, 5, 1, 3
    x = rng.standard_normal((N, H, W, G * Cg))
    m = rng.standard_normal((N, H, W, G * 9))
    for big in (1e4, -1e4, np.inf, -np.inf, np.nan):
        off = np.full((N, H, W, G * 18), big)
        got = fwd(x, off, m, 3, 1, 1, 1, 1.0, False, G, oracle.COORD_BINARY32)
        assert np.array_equal(got, np.zeros_like(got)), big
    # a single NaN point leaves the other points' contributions untouched
    off = rng.standard_normal((N, H, W, G * 9, 2))
    ref = fwd(x, off.reshape(N, H, W, -1), np.where(np.arange(9) == 3, 0.0, m.reshape(N, H, W, 9)),
              3, 1, 1, 1, 1.0, False, G)
    off[..., 3, 0] = np.nan
    got = fwd(x, off.reshape(N, H, W, -1), m, 3, 1, 1, 1, 1.0, False, G)
    assert np.allclose(got, ref, rtol=0, atol=1e-13)


def coverage(t, n):
    """In-map weight of a 1-D linear read at t on [0, n): a clamped tent."""
    return min(max(min(t + 1.0, n - t), 0.0), 1.0)


def test_constant_input_softmax_closed_form():
    """Constant input k under DCNv3 softmax: interior samples return k exactly
    (the weights sum to 1); every output equals k * sum_p m_p cov(x_p) cov(y_p)
    with cov the clamped tent (a different closed form from the bilinear rule)."""
    rng = np.random.default_rng(9)
    N, H, W, G, Cg, K = 1, 9, 10, 2, 2, 3
    k = 1.7
    x = np.full((N, H, W, G * Cg), k)
    off = rng.uniform(-0.9, 0.9, (N, H, W, G, 9, 2))
    logits = rng.standard_normal((N, H, W, G, 9))
    got = fwd(x, off.reshape(N, H, W, -1), logits.reshape(N, H, W, -1), K, 1, 1, 1, 1.0, True, G)
    for ho in range(H):
        for wo in range(W):
            for g in range(G):
                lg = logits[0, ho, wo, g]
                mt = np.exp(lg - lg.max())
                mt /= mt.sum()
                cov = 0.0
                for i in range(3):
                    for j in range(3):
                        p = i * 3 + j
                        xs = wo - 1 + 1 + (i - 1) + off[0, ho, wo, g, p, 0]
                        ys = ho - 1 + 1 + (j - 1) + off[0, ho, wo, g, p, 1]
                        cov += mt[p] * coverage(xs, W) * coverage(ys, H)
                for c in range(Cg):
                    assert abs(got[0, ho, wo, g * Cg + c] - k * cov) <= 1e-13
                if 1 <= ho < H - 1 and 1 <= wo < W - 1:
                    inner = all(0 <= wo + (i - 1) + off[0, ho, wo, g, i * 3 + j, 0] <= W - 1 and
                                0 <= ho + (j - 1) + off[0, ho, wo, g, i * 3 + j, 1] <= H - 1
                                for i in range(3) for j in range(3))
                    if inner:
                        assert np.allclose(got[0, ho, wo, g * Cg:(g + 1) * Cg], k, rtol=0, atol=1e-14)


def test_linearity_in_input_and_raw_mask():
    rng = np.random.default_rng(10)
    N, H, W, G, Cg, K = 1, 6, 7, 2, 2, 3
    x1, off, m1 = rand_case(rng, N, H, W, G, Cg, K, 1, 1, 1)
    x2, _, m2 = rand_case(rng, N, H, W, G, Cg, K, 1, 1, 1)
    a, b = 0.3, -1.9
    f = lambda x, m: fwd(x, off, m, K, 1, 1, 1, 1.0, False, G)
    assert np.allclose(f(a * x1 + b * x2, m1), a * f(x1, m1) + b * f(x2, m1), rtol=0, atol=1e-12)
    assert np.allclose(f(x1, a * m1 + b * m2), a * f(x1, m1) + b * f(x1, m2), rtol=0, atol=1e-12)


def test_transpose_consistency():
    """Swapping H and W, the offset pair and the point (i, j) -> (j, i)
    transposes the output: catches any x/y or H/W mix-up."""
    rng = np.random.default_rng(12)
    N, H, W, G, Cg, K, s, p, d = 1, 7, 9, 2, 2, 3, 2, 1, 1
    x, off, m = rand_case(rng, N, H, W, G, Cg, K, s, p, d)
    Ho, Wo = ind.conv_out(H, K, s, p, d), ind.conv_out(W, K, s, p, d)
    P = K * K
    perm = [(pp % K) * K + pp // K for pp in range(P)]        # (i,j) -> (j,i)
    offT = off.reshape(N, Ho, Wo, G, P, 2)[:, :, :, :, perm, ::-1].transpose(0, 2, 1, 3, 4, 5)
    mT = m.reshape(N, Ho, Wo, G, P)[:, :, :, :, perm].transpose(0, 2, 1, 3, 4)
    xT = x.transpose(0, 2, 1, 3)
    a = fwd(x, off, m, K, s, p, d, 1.0, True, G)
    b = fwd(np.ascontiguousarray(xT), np.ascontiguousarray(offT).reshape(N, Wo, Ho, -1),
            np.ascontiguousarray(mT).reshape(N, Wo, Ho, -1), K, s, p, d, 1.0, True, G)
    assert np.allclose(b, a.transpose(0, 2, 1, 3), rtol=0, atol=1e-13)


def test_absum_bounds_output():
    rng = np.random.default_rng(13)
    x, off, m = rand_case(rng, 1, 6, 6, 2, 3, 3, 1, 1, 1)
    out, S = oracle.forward(x, off, m, K=3, stride=1, pad=1, dilation=1, offset_scale=1.0,
                            softmax=False, group=2)
    assert np.all(np.abs(out) <= S + 1e-15)
    # with a one-signed integrand the abs-sum equals |out|
    out2, S2 = oracle.forward(np.abs(x), off, np.abs(m), K=3, stride=1, pad=1, dilation=1,
                              offset_scale=1.0, softmax=False, group=2)
    assert np.allclose(out2, S2, rtol=1e-14, atol=0)
