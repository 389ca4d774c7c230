"""Pins of the oracle's real spherical harmonics (CPU only)."""
import math

import numpy as np
from numpy.polynomial import legendre

from oracle import sph


def _unit(n, seed):
    v = np.random.default_rng(seed).normal(size=(n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def test_y00_and_component_normalisation():
    u = _unit(200, 1)
    Y = sph.real_sph(u)
    assert np.allclose(Y[:, 0], 1.0, atol=0, rtol=1e-15)
    L = sph.l_of_index()
    for l in range(4):
        assert np.allclose((Y[:, L == l] ** 2).sum(1), 2 * l + 1, rtol=1e-13)


def test_addition_theorem():
    # sum_m Y_lm(u) Y_lm(v) = (2l+1) P_l(u.v): independent of sign / m conventions
    u, v = _unit(300, 2), _unit(300, 3)
    Yu, Yv = sph.real_sph(u), sph.real_sph(v)
    L = sph.l_of_index()
    c = (u * v).sum(1)
    for l in range(4):
        lhs = (Yu[:, L == l] * Yv[:, L == l]).sum(1)
        coef = np.zeros(l + 1)
        coef[l] = 1.0
        assert np.allclose(lhs, (2 * l + 1) * legendre.legval(c, coef), atol=1e-13)


def test_orthogonality_by_quadrature():
    # Gauss-Legendre in cos(theta) (8 nodes, exact to degree 15) x 16 uniform phi nodes
    xg, wg = legendre.leggauss(8)
    phi = np.arange(16) * (2 * math.pi / 16)
    ct, ph = np.meshgrid(xg, phi, indexing="ij")
    st = np.sqrt(1 - ct**2)
    u = np.stack([st * np.cos(ph), st * np.sin(ph), ct], -1).reshape(-1, 3)
    w = (wg[:, None] * np.full(16, 2 * math.pi / 16)[None, :]).reshape(-1)
    Y = sph.real_sph(u)
    G = (Y * w[:, None]).T @ Y / (4 * math.pi)
    assert np.allclose(G, np.eye(16), atol=1e-13)


def test_on_axis_values():
    Y = sph.real_sph(np.array([[0.0, 0.0, 1.0]]))[0]
    for l in range(4):
        for m in range(-l, l + 1):
            want = math.sqrt(2 * l + 1) if m == 0 else 0.0
            assert abs(Y[sph.lm_index(l, m)] - want) < 1e-14


def test_convention_against_explicit_polynomials():
    # explicit real-harmonic polynomials of the convention chosen (z polar,
    # no Condon-Shortley phase, m = -l..l); an independent closed form of each component
    u = _unit(50, 4)
    x, y, z = u.T
    s = math.sqrt
    want = np.stack([
        np.ones_like(x), s(3) * y, s(3) * z, s(3) * x,
        s(15) * x * y, s(15) * y * z, s(5) / 2 * (3 * z * z - 1), s(15) * x * z, s(15) / 2 * (x * x - y * y),
        s(70) / 4 * y * (3 * x * x - y * y), s(105) * x * y * z, s(42) / 4 * y * (5 * z * z - 1),
        s(7) / 2 * z * (5 * z * z - 3), s(42) / 4 * x * (5 * z * z - 1), s(105) / 2 * z * (x * x - y * y),
        s(70) / 4 * x * (x * x - 3 * y * y),
    ], 1)
    assert np.allclose(sph.real_sph(u), want, atol=1e-13)


def test_tangential_gradient_against_finite_differences():
    # f(d) = Y(d/|d|): grad_d f = (I - u u^T) grad_u Y / r
    rng = np.random.default_rng(5)
    d = rng.normal(size=(20, 3)) * 2.0
    r = np.linalg.norm(d, axis=1)
    u = d / r[:, None]
    _, dY = sph.real_sph(u, grad=True)
    P = np.eye(3)[None] - u[:, :, None] * u[:, None, :]
    ana = np.einsum("eab,ekb->eka", P, dY) / r[:, None, None]
    h = 1e-6
    for a in range(3):
        dp, dm = d.copy(), d.copy()
        dp[:, a] += h
        dm[:, a] -= h
        fp = sph.real_sph(dp / np.linalg.norm(dp, axis=1, keepdims=True))
        fm = sph.real_sph(dm / np.linalg.norm(dm, axis=1, keepdims=True))
        assert np.allclose((fp - fm) / (2 * h), ana[:, :, a], atol=1e-8)
