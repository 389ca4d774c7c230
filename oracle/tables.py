"""Radial tables: the radial chain r -> s2(r) as piecewise interpolants (float64).

TEST INFRASTRUCTURE ONLY (oracle; never used by the product path).

What the pages fix, and where ("FastMACE rewrite screens"):

* OPT6-T05 radial_tables: per species pair, tables of degree 10 in r on
  dyadic pieces, replacing the radial chain; values and r-derivatives within
  1e-7 of their local scale; a certificate that compares the float32 table's
  error with the float32 network's, both against float64; opt-in, float32;
* OPT6-T04: the accuracy premise (the float32 table is more accurate than the
  float32 network; their ratio 0.13-0.57 on the pages' models).

Readings where the pages leave a step open:

* what is tabulated: the chain up to the last (linear) radial layer, s2(r) =
  silu(silu(b(r) W1) W2), 64 units per ordered species pair.  With the last
  layer folded past the edge sum (the folded call) s2 is the per-edge output
  of the radial chain;
* "dyadic pieces": 2^K coarse pieces [c h0, (c+1) h0) of [0, rc], h0 = rc / 2^K,
  coarse piece c split into 2^d equal sub-pieces, d in [0, DMAX] the smallest
  level at which every binary64 interpolant of c is within TOL of the chain
  (values and r-derivatives, relative to the local scale, at the check
  points); short distances, where the chain is largest and steepest, need
  the finer levels;
* "Chebyshev tables": on each sub-piece the interpolant of degree 10 at the 11
  Chebyshev points of the first kind, x_i = cos(pi (i + 1/2) / 11), in the
  sub-piece variable t in [-1, 1];
* r >= rc: zero (the envelope, and so the chain, vanish there);
* local scale, check points and the certificate: the largest magnitude of a
  unit's value (derivative) over the sub-piece, at its nodes and at the 16
  points t_q = -1 + (2q + 1) / 16; the certificate is the largest error of
  the stored table there against the binary64 chain, values and derivatives
  apart, each relative to that scale.

Pins (tests/test_oracle_tables.py): polynomials of degree <= 10 reproduced
exactly; the coefficients equal NumPy's Chebyshev interpolation routine on a
piece; the chain's r-derivative against central differences; convergence of
the table to the chain at random r; zero past the cutoff.
"""
from __future__ import annotations

import math
import numpy as np

from .model import radial_basis, silu, silu_d

DEG = 10
CHECKS = 16
DMAX = 4  # at most 2^DMAX sub-pieces per coarse piece
TOL = 1e-8  # binary64 interpolation error that fixes a coarse piece's level


def nodes(deg: int = DEG) -> np.ndarray:
    """Chebyshev points of the first kind on [-1, 1]."""
    i = np.arange(deg + 1, dtype=np.float64)
    return np.cos(np.pi * (i + 0.5) / (deg + 1))


def chain(r, W1, W2, rc):
    """s2(r) = silu(silu(b(r) W1) W2) and ds2/dr, float64, rows = r."""
    r = np.asarray(r, np.float64)
    b, db = radial_basis(r, rc, deriv=True)
    W1 = np.asarray(W1, np.float64)
    W2 = np.asarray(W2, np.float64)
    z1 = b @ W1
    dz1 = db @ W1
    s1 = silu(z1)
    ds1 = silu_d(z1) * dz1
    z2 = s1 @ W2
    dz2 = ds1 @ W2
    return silu(z2), silu_d(z2) * dz2


def locate(r, rc, log2_pieces, levels):
    """Slot (c, f) and sub-piece variable t of each r (c = -1 past the cutoff)."""
    r = np.asarray(r, np.float64)
    n = 1 << log2_pieces
    h0 = rc / n
    c = np.floor(r / h0).astype(np.int64)
    ok = (c >= 0) & (c < n)
    cc = np.where(ok, c, 0)
    d = np.asarray(levels)[cc]
    h = h0 / (1 << d)
    f = np.minimum(np.floor((r - cc * h0) / h).astype(np.int64), (1 << d) - 1)
    t = 2.0 * (r - cc * h0 - f * h) / h - 1.0
    return np.where(ok, c, -1), f, t, h


def chebyshev_coefficients(values_at_nodes: np.ndarray) -> np.ndarray:
    """Coefficients c_m (rows) of the interpolant through values at nodes():
    c_m = (2 / n) sum_i f(x_i) T_m(x_i), c_0 halved (discrete orthogonality)."""
    f = np.asarray(values_at_nodes, np.float64)
    n = f.shape[0]
    theta = np.pi * (np.arange(n) + 0.5) / n
    Tm = np.cos(np.outer(np.arange(n), theta))  # T_m(x_i) = cos(m theta_i)
    c = (2.0 / n) * (Tm @ f)
    c[0] *= 0.5
    return c


def sub_piece(fn, r0, h, deg: int = DEG):
    """Chebyshev coefficients [deg + 1][units] of fn on [r0, r0 + h] and the
    interpolant's largest errors (value, derivative) against fn at the check
    points, relative to the local scale.  fn(r) -> (value, r-derivative)."""
    x = nodes(deg)
    vn, dn = fn(r0 + 0.5 * (x + 1.0) * h)
    c = chebyshev_coefficients(vn)
    tq = -1.0 + (2.0 * np.arange(CHECKS) + 1.0) / CHECKS
    vq, dq = fn(r0 + 0.5 * (tq + 1.0) * h)
    C = np.polynomial.chebyshev
    pv = C.chebval(tq, c).T
    pd = C.chebval(tq, C.chebder(c)).T * (2.0 / h)
    sv = np.maximum(np.abs(vn).max(0), np.abs(vq).max(0))
    sd = np.maximum(np.abs(dn).max(0), np.abs(dq).max(0))
    return c, _rel(np.abs(pv - vq).max(0), sv), _rel(np.abs(pd - dq).max(0), sd)


def _rel(err, scale):
    with np.errstate(divide="ignore", invalid="ignore"):
        x = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(np.nan_to_num(x, nan=np.inf).max())


def build_pair(fn, rc, log2_pieces, deg: int = DEG, dmax: int = DMAX, tol: float = TOL):
    """Levels [2^K] and Chebyshev coefficients [2^K][2^dmax][deg + 1][units]
    (unused sub-piece slots zero) of fn(r) -> (value, r-derivative)."""
    n = 1 << log2_pieces
    h0 = rc / n
    levels = np.zeros(n, np.int64)
    coef = None
    for c in range(n):
        for d in range(dmax + 1):
            h = h0 / (1 << d)
            parts = [sub_piece(fn, c * h0 + f * h, h, deg) for f in range(1 << d)]
            worst = max(max(ev, ed) for _, ev, ed in parts)
            if worst <= tol or d == dmax:
                break
        if coef is None:
            coef = np.zeros((n, 1 << dmax, deg + 1, parts[0][0].shape[1]))
        levels[c] = d
        for f, (cf, _, _) in enumerate(parts):
            coef[c, f] = cf
    return levels, coef


def level_errors(fn, rc, log2_pieces, c, d, deg: int = DEG):
    """Largest interpolation error (value or derivative) of coarse piece c at level d."""
    h0 = rc / (1 << log2_pieces)
    h = h0 / (1 << d)
    return max(max(ev, ed) for _, ev, ed in (sub_piece(fn, c * h0 + f * h, h, deg) for f in range(1 << d)))


def pair_chain(model, p):
    return lambda r: chain(r, model.W1[p], model.W2[p], model.cutoff)


def build_table(model, log2_pieces, deg: int = DEG):
    """Per ordered pair: (levels, Chebyshev coefficients) of s2."""
    return [build_pair(pair_chain(model, p), model.cutoff, log2_pieces, deg) for p in range(model.n_species ** 2)]


def evaluate(levels, coef_pair, r, rc, log2_pieces):
    """Value and r-derivative of one pair's table at r (float64; zero past rc)."""
    c, f, t, h = locate(r, rc, log2_pieces, levels)
    C = np.polynomial.chebyshev
    units = coef_pair.shape[-1]
    v = np.zeros((len(c), units))
    d = np.zeros((len(c), units))
    for e in np.nonzero(c >= 0)[0]:
        cf = coef_pair[c[e], f[e]]
        v[e] = C.chebval(t[e], cf)
        d[e] = C.chebval(t[e], C.chebder(cf)) * (2.0 / h[e])
    return v, d


def power_form(coef_cheb: np.ndarray) -> np.ndarray:
    """Chebyshev coefficients [..., m, unit] -> power-form coefficients in t (float64)."""
    deg = coef_cheb.shape[-2] - 1
    M = np.zeros((deg + 1, deg + 1))  # M[q, m] = coefficient of t^q in T_m
    for m in range(deg + 1):
        p = np.polynomial.chebyshev.cheb2poly(np.eye(deg + 1)[m])
        M[: len(p), m] = p
    return np.einsum("qm,...mu->...qu", M, coef_cheb)


def certificate(levels, power_pair: np.ndarray, fn, rc, log2_pieces):
    """Largest error of a stored power-form table [c][f][m][unit] (evaluated in
    float64) against fn (value, derivative) at the check points of every used
    sub-piece: (values, r-derivatives), each relative to the local scale."""
    n = 1 << log2_pieces
    h0 = rc / n
    tq = -1.0 + (2.0 * np.arange(CHECKS) + 1.0) / CHECKS
    x = nodes(power_pair.shape[-2] - 1)
    P = np.polynomial.polynomial
    ev = ed = 0.0
    for c in range(n):
        h = h0 / (1 << int(levels[c]))
        for f in range(1 << int(levels[c])):
            r0 = c * h0 + f * h
            vq, dq = fn(r0 + 0.5 * (tq + 1.0) * h)
            vn, dn = fn(r0 + 0.5 * (x + 1.0) * h)
            a = np.asarray(power_pair[c, f], np.float64)
            pv = P.polyval(tq, a).T
            pd = P.polyval(tq, P.polyder(a)).T * (2.0 / h)
            sv = np.maximum(np.abs(vq).max(0), np.abs(vn).max(0))
            sd = np.maximum(np.abs(dq).max(0), np.abs(dn).max(0))
            ev = max(ev, _rel(np.abs(pv - vq).max(0), sv))
            ed = max(ed, _rel(np.abs(pd - dq).max(0), sd))
    return ev, ed
