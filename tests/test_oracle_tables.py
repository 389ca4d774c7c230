"""Pins of the oracle's radial tables (CPU only).

The tables replace the radial chain r -> s2(r) by degree-10 interpolants on
dyadic pieces ("FastMACE rewrite screens", OPT6-T05 radial_tables and OPT6-T04).
Pinned here by what the mathematics fixes: polynomials of degree <= 10 come
back exactly (and degree 11 does not); the coefficients equal NumPy's own
Chebyshev interpolation routine; the power form agrees with the Chebyshev
form; the chain's r-derivative agrees with central differences; the table of
the synthetic model converges to its chain; zero past the cutoff; the
certificate separates a fine table from a coarse one.
"""
import numpy as np
import pytest

import eec_inputs as I
from oracle import tables as TB

RC = 6.0


def _poly_fn(deg, seed=0, units=3):
    """A polynomial of degree deg in r per unit, and its r-derivative."""
    a = np.random.default_rng(seed).normal(size=(deg + 1, units))

    def fn(r):
        x = 2.0 * np.asarray(r)[:, None] / RC - 1.0
        v = sum(a[q] * x**q for q in range(deg + 1))
        d = sum(q * a[q] * x ** (q - 1) for q in range(1, deg + 1)) * (2.0 / RC)
        return v, d

    return fn


def test_polynomials_up_to_degree_10_exact():
    rng = np.random.default_rng(1)
    r = rng.uniform(0.0, RC, 200)
    fn = _poly_fn(10)
    levels, c = TB.build_pair(fn, RC, 3)
    assert np.all(levels == 0)  # exact at the coarsest level already
    v, d = TB.evaluate(levels, c, r, RC, 3)
    ref, dref = fn(r)
    assert np.abs(v - ref).max() <= 1e-11 * np.abs(ref).max()
    assert np.abs(d - dref).max() <= 1e-10 * np.abs(dref).max()
    # one degree more is not reproduced on one piece: the interpolant has degree 10
    fn11 = _poly_fn(11, seed=2)
    l11, c11 = TB.build_pair(fn11, RC, 0, dmax=0)
    v11, _ = TB.evaluate(l11, c11, r, RC, 0)
    assert np.abs(v11 - fn11(r)[0]).max() > 1e-6 * np.abs(fn11(r)[0]).max()


def test_refinement_reaches_the_tolerance():
    # sin(w r) on coarse pieces too wide for degree 10: the levels rise until
    # the interpolants are within TOL, and the table is that accurate
    w = 40.0
    fn = lambda r: (np.sin(w * r)[:, None], (w * np.cos(w * r))[:, None])
    levels, c = TB.build_pair(fn, RC, 3)
    assert levels.min() >= 1 and levels.max() <= TB.DMAX
    r = np.random.default_rng(6).uniform(0.0, RC, 400)
    v, d = TB.evaluate(levels, c, r, RC, 3)
    assert np.abs(v[:, 0] - np.sin(w * r)).max() <= 1e-7
    assert np.abs(d[:, 0] - w * np.cos(w * r)).max() <= 1e-7 * w


def test_coefficients_equal_numpy_chebinterpolate():
    cfg = I.make_config("D64")
    m = cfg.model
    K, k = 5, 19
    h = RC / (1 << K)
    for unit in (0, 17, 63):
        f = lambda x, u=unit: TB.chain((k + 0.5 * (x + 1.0)) * h, m.W1[0], m.W2[0], RC)[0][:, u]
        ref = np.polynomial.chebyshev.chebinterpolate(f, TB.DEG)
        ours = TB.chebyshev_coefficients(TB.chain((k + 0.5 * (TB.nodes() + 1.0)) * h, m.W1[0], m.W2[0], RC)[0])
        np.testing.assert_allclose(ours[:, unit], ref, rtol=0, atol=1e-13 * np.abs(ref).max())


def test_power_form_equals_chebyshev_form():
    c = np.random.default_rng(3).normal(size=(TB.DEG + 1, 5))
    a = TB.power_form(c)
    t = np.linspace(-1, 1, 41)
    np.testing.assert_allclose(np.polynomial.polynomial.polyval(t, a).T,
                               np.polynomial.chebyshev.chebval(t, c).T, rtol=0, atol=1e-12)


def test_chain_derivative_central_differences():
    m = I.make_config("PV2").model
    r = np.random.default_rng(4).uniform(0.8, 5.9, 50)
    for p in (0, 4, 7):
        v, d = TB.chain(r, m.W1[p], m.W2[p], RC)
        eps = 1e-6
        fd = (TB.chain(r + eps, m.W1[p], m.W2[p], RC)[0] - TB.chain(r - eps, m.W1[p], m.W2[p], RC)[0]) / (2 * eps)
        assert np.abs(d - fd).max() <= 1e-7 * np.abs(fd).max()


@pytest.mark.parametrize("name", ["D64", "PV2"])
def test_table_converges_to_chain(name):
    m = I.make_config(name).model
    tabs = TB.build_table(m, 6)
    r = np.random.default_rng(5).uniform(0.05, RC, 300)
    for p in range(m.n_species ** 2):
        levels, coef = tabs[p]
        assert levels[0] > levels[-1]  # the short-range pieces are refined
        v, d = TB.evaluate(levels, coef, r, RC, 6)
        ev, ed = TB.chain(r, m.W1[p], m.W2[p], RC)
        assert np.abs(v - ev).max() <= 1e-7 * np.abs(ev).max()
        assert np.abs(d - ed).max() <= 1e-7 * np.abs(ed).max()


def test_zero_past_cutoff():
    m = I.make_config("D64").model
    levels, coef = TB.build_table(m, 3)[0]
    v, d = TB.evaluate(levels, coef, np.array([RC, RC + 1e-9, RC + 0.3]), RC, 3)
    assert np.all(v == 0.0) and np.all(d == 0.0)


def test_certificate_separates_fine_and_coarse_tables():
    m = I.make_config("D64").model
    fn = TB.pair_chain(m, 0)
    levels, coef = TB.build_pair(fn, RC, 6)
    fine = TB.power_form(coef).astype(np.float32)
    ev, ed = TB.certificate(levels, fine, fn, RC, 6)
    assert ev <= 3e-7 and ed <= 3e-7
    lc, cc = TB.build_pair(fn, RC, 3, dmax=0)
    cv, cd = TB.certificate(lc, TB.power_form(cc).astype(np.float32), fn, RC, 3)
    assert cv > 1e-4 and cd > 1e-4
