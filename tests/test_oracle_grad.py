"""Pins of the oracle's backward (CPU only).

* grad_input: the forward is linear in the input, so <f(x), g> = <x, grad_input(g)>
  (adjoint identity; a wrong corner, weight or scatter index breaks it).
* grad_mask for a raw mask: the forward is linear in the mask too.
* grad_offset and the softmax grad_mask: central finite differences of the
  forward in binary64, with every coordinate kept at least 0.1 px away from
  integers so no floor() jump lies inside the difference step.
"""
import numpy as np
import pytest

import oracle
from tests import independent as ind


def setup(rng, N, H, W, G, Cg, K, s, p, d, alpha):
    Ho, Wo, P = ind.conv_out(H, K, s, p, d), ind.conv_out(W, K, s, p, d), K * K
    c0 = d * (K - 1) // 2
    x = rng.standard_normal((N, H, W, G * Cg))
    # offsets whose sampling coordinates have fractional parts in [0.1, 0.9]
    off = np.empty((N, Ho, Wo, G, P, 2))
    for pp in range(P):
        i, j = divmod(pp, K)
        for ax, tap in ((0, i * d - c0), (1, j * d - c0)):
            r = rng.integers(-2, 3, size=(N, Ho, Wo, G)).astype(np.float64)
            frac = rng.uniform(0.1, 0.9, size=(N, Ho, Wo, G))
            # alpha * (tap + off) = r + frac  ->  off = (r + frac) / alpha - tap
            off[..., pp, ax] = (r + frac) / alpha - tap
    m = rng.standard_normal((N, Ho, Wo, G * P))
    g = rng.standard_normal((N, Ho, Wo, G * Cg))
    return x, off.reshape(N, Ho, Wo, -1), m, g


def f(x, off, m, K, s, p, d, a, sm, G):
    out, _ = oracle.forward(x, off, m, K=K, stride=s, pad=p, dilation=d, offset_scale=a,
                            softmax=sm, group=G, coord_mode=oracle.COORD_EXACT, with_absum=False)
    return out


def b(x, off, m, go, K, s, p, d, a, sm, G):
    return oracle.backward(x, off, m, go, K=K, stride=s, pad=p, dilation=d, offset_scale=a,
                           softmax=sm, group=G, coord_mode=oracle.COORD_EXACT)


GEOMS = [  # N, H, W, G, Cg, K, s, pad, d, alpha, softmax
    (1, 5, 6, 2, 2, 3, 1, 1, 1, 1.0, False),
    (2, 6, 5, 1, 3, 3, 2, 1, 1, 0.5, True),
    (1, 7, 6, 2, 1, 3, 1, 2, 2, 1.0, True),
    (1, 6, 6, 1, 2, 5, 1, 2, 1, 1.0, False),
]


@pytest.mark.parametrize("geom", GEOMS)
def test_grad_input_adjoint(geom):
    N, H, W, G, Cg, K, s, p, d, a, sm = geom
    rng = np.random.default_rng(31)
    x, off, m, g = setup(rng, N, H, W, G, Cg, K, s, p, d, a)
    off = off + rng.standard_normal(off.shape) * 2.0   # any offsets: linear in x regardless
    lhs = np.sum(f(x, off, m, K, s, p, d, a, sm, G) * g)
    r = b(x, off, m, g, K, s, p, d, a, sm, G)
    rhs = np.sum(x * r["grad_input"])
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # the abs-sum and count scales are consistent with the value
    assert np.all(np.abs(r["grad_input"]) <= r["gi_abs"] + 1e-15)
    assert np.all((r["gi_cnt"] == 0) <= (r["grad_input"] == 0))


def test_grad_mask_raw_adjoint():
    rng = np.random.default_rng(32)
    N, H, W, G, Cg, K = 2, 6, 6, 2, 3, 3
    x, off, m, g = setup(rng, N, H, W, G, Cg, K, 1, 1, 1, 1.0)
    off = off + rng.standard_normal(off.shape)
    lhs = np.sum(f(x, off, m, K, 1, 1, 1, 1.0, False, G) * g)
    r = b(x, off, m, g, K, 1, 1, 1, 1.0, False, G)
    assert abs(lhs - np.sum(m * r["grad_mask"])) <= 1e-12 * max(1.0, abs(lhs))


@pytest.mark.parametrize("geom", GEOMS)
def test_grad_offset_finite_difference(geom):
    N, H, W, G, Cg, K, s, p, d, a, sm = geom
    rng = np.random.default_rng(33)
    x, off, m, g = setup(rng, N, H, W, G, Cg, K, s, p, d, a)
    r = b(x, off, m, g, K, s, p, d, a, sm, G)
    h = 1e-6
    flat = off.reshape(-1)
    idx = rng.choice(flat.size, size=min(60, flat.size), replace=False)
    for k in idx:
        op, om = flat.copy(), flat.copy()
        op[k] += h
        om[k] -= h
        fd = (np.sum(f(x, op.reshape(off.shape), m, K, s, p, d, a, sm, G) * g)
              - np.sum(f(x, om.reshape(off.shape), m, K, s, p, d, a, sm, G) * g)) / (2 * h)
        an = r["grad_offset"].reshape(-1)[k]
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (k, fd, an)


@pytest.mark.parametrize("softmax", [False, True])
def test_grad_mask_finite_difference(softmax):
    rng = np.random.default_rng(34)
    N, H, W, G, Cg, K = 1, 5, 6, 2, 2, 3
    x, off, m, g = setup(rng, N, H, W, G, Cg, K, 1, 1, 1, 1.0)
    r = b(x, off, m, g, K, 1, 1, 1, 1.0, softmax, G)
    h = 1e-6
    flat = m.reshape(-1)
    for k in rng.choice(flat.size, size=40, replace=False):
        mp, mm = flat.copy(), flat.copy()
        mp[k] += h
        mm[k] -= h
        fd = (np.sum(f(x, off, mp.reshape(m.shape), K, 1, 1, 1, 1.0, softmax, G) * g)
              - np.sum(f(x, off, mm.reshape(m.shape), K, 1, 1, 1, 1.0, softmax, G) * g)) / (2 * h)
        an = r["grad_mask"].reshape(-1)[k]
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (k, fd, an)


def test_skipped_samples_have_zero_gradient():
    rng = np.random.default_rng(35)
    N, H, W, G, Cg = 1, 4, 4, 1, 2
    x = rng.standard_normal((N, H, W, Cg))
    off = np.full((N, H, W, 18), 1e4)
    m = rng.standard_normal((N, H, W, 9))
    g = rng.standard_normal((N, H, W, Cg))
    r = oracle.backward(x, off, m, g, K=3, stride=1, pad=1, dilation=1, offset_scale=1.0,
                        softmax=False, group=1)
    assert not np.any(r["grad_input"]) and not np.any(r["grad_offset"]) and not np.any(r["grad_mask"])


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan, 1e300])
def test_skipped_sample_gradients_ignore_its_mask_value(bad):
    """A sample the skip rule drops adds nothing to the output for any mask
    value, and moving its offsets a little keeps it dropped, so the output
    equals the one with that mask value set to 0 (checked on the forward)
    and every gradient equals that call's: grad_input and grad_offset
    unchanged, zero offset and mask gradients at the dropped sample (no
    Inf * 0 from the mask it never multiplies)."""
    rng = np.random.default_rng(37)
    N, H, W, G, Cg, K = 1, 6, 7, 2, 3, 3
    x, off, m, g = setup(rng, N, H, W, G, Cg, K, 1, 1, 1, 1.0)
    off = off.reshape(N, H, W, G, 9, 2)
    m = m.reshape(N, H, W, G, 9)
    drop = rng.random((N, H, W, G, 9)) < 0.3
    off[drop] = np.array([-50.5, 3.25])            # x far left of the map: skipped
    m_bad, m_zero = m.copy(), m.copy()
    m_bad[drop] = bad
    m_zero[drop] = 0.0
    off = off.reshape(N, H, W, -1)
    kw = dict(K=K, stride=1, pad=1, dilation=1, offset_scale=1.0, softmax=False, group=G)
    o_bad, _ = oracle.forward(x, off, m_bad.reshape(N, H, W, -1), **kw)
    o_zero, _ = oracle.forward(x, off, m_zero.reshape(N, H, W, -1), **kw)
    assert np.array_equal(o_bad, o_zero)
    r_bad = oracle.backward(x, off, m_bad.reshape(N, H, W, -1), g, **kw)
    r_zero = oracle.backward(x, off, m_zero.reshape(N, H, W, -1), g, **kw)
    assert np.array_equal(r_bad["grad_input"], r_zero["grad_input"])
    assert np.array_equal(r_bad["grad_offset"], r_zero["grad_offset"])
    assert np.array_equal(r_bad["grad_mask"], r_zero["grad_mask"])
    goff = r_bad["grad_offset"].reshape(N, H, W, G, 9, 2)
    assert not np.any(goff[drop]) and not np.any(r_bad["grad_mask"].reshape(N, H, W, G, 9)[drop])
    assert np.any(goff[~drop])                      # the kept samples do have gradients


def test_binary32_mode_matches_exact_away_from_integers():
    """The binary32 coordinate mode only moves coordinates by ~|x|*2^-24; away
    from integers both modes give nearly the same gradients."""
    rng = np.random.default_rng(36)
    N, H, W, G, Cg, K = 1, 6, 7, 2, 2, 3
    x, off, m, g = setup(rng, N, H, W, G, Cg, K, 1, 1, 1, 1.0)
    kw = dict(K=K, stride=1, pad=1, dilation=1, offset_scale=1.0, softmax=True, group=G)
    r0 = oracle.backward(x, off, m, g, coord_mode=oracle.COORD_EXACT, **kw)
    r1 = oracle.backward(x, off, m, g, coord_mode=oracle.COORD_BINARY32, **kw)
    for key in ("grad_input", "grad_offset", "grad_mask"):
        assert np.allclose(r0[key], r1[key], rtol=0, atol=1e-5), key
