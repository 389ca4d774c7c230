"""Real spherical harmonics up to l = 3 and their gradients (float64).

TEST INFRASTRUCTURE ONLY (oracle; never used by the product path).

The pages fix the degree cut-off (lmax 3, "deepmd-kit PR #2", Implementation
and scope: the checked "lmax3" FP32 layout) and the four degrees of the radial
weights ("deepmd-kit PR #6108", What: the (E,4,32) basis).  They do not fix
the normalisation, the sign convention or the m order.  The reading used here:
component-normalised real harmonics (sum_m Y_lm^2 = 2l+1, Y_00 = 1), polar axis
z, no Condon-Shortley phase, m = -l..l, flat index k = l*l + l + m.

Construction (no table): with u = (x, y, z) a unit vector,

    Y_lm(u) = N_lm * Q_l^|m|(z) * T_m(x, y),
    Q_l^m(z) = d^m P_l(z) / dz^m           (derivative of a Legendre polynomial),
    T_m = Re (x + i y)^|m|   for m > 0,
          Im (x + i y)^|m|   for m < 0,   1 for m = 0,
    N_lm = sqrt((2l+1) (l-|m|)! / (l+|m|)!) * (sqrt(2) if m != 0 else 1).

Q_l^m follows the associated-Legendre three-term recurrence
Q_m^m = (2m-1)!!, Q_{m+1}^m = (2m+1) z Q_m^m,
(l-m) Q_l^m = (2l-1) z Q_{l-1}^m - (l+m-1) Q_{l-2}^m,
and d Q_l^m / dz = Q_l^{m+1}.

The gradient returned is that of this polynomial extension off the sphere; it
is only ever used after projection onto the tangent plane (I - u u^T), where
the extension does not matter.

Pins: Y_00 = 1; sum_m Y_lm^2 = 2l+1; the addition theorem
sum_m Y_lm(u) Y_lm(v) = (2l+1) P_l(u.v) (convention-free); orthonormality by
Gauss-Legendre x uniform-phi quadrature; on-axis values; the tangential
gradient against central finite differences on the sphere.
"""
from __future__ import annotations

import math
import numpy as np

LMAX = 3
N_LM = (LMAX + 1) ** 2


def lm_index(l: int, m: int) -> int:
    return l * l + l + m


def _legendre_derivs(z: np.ndarray, lmax: int):
    """Q[l][m] = d^m P_l / dz^m for 0 <= m <= l <= lmax (+ zero for m = l+1)."""
    Q = {}
    for m in range(lmax + 2):
        dfact = 1.0
        for t in range(1, 2 * m, 2):
            dfact *= t
        for l in range(m, lmax + 1):
            if l == m:
                Q[(l, m)] = np.full_like(z, dfact)
            elif l == m + 1:
                Q[(l, m)] = (2 * m + 1) * z * Q[(m, m)]
            else:
                Q[(l, m)] = ((2 * l - 1) * z * Q[(l - 1, m)] - (l + m - 1) * Q[(l - 2, m)]) / (l - m)
    return Q


def _norm(l: int, m: int) -> float:
    am = abs(m)
    n = math.sqrt((2 * l + 1) * math.factorial(l - am) / math.factorial(l + am))
    return n * (math.sqrt(2.0) if m != 0 else 1.0)


def real_sph(u: np.ndarray, lmax: int = LMAX, grad: bool = False):
    """Y [n, (lmax+1)^2] (and dY/du [n, (lmax+1)^2, 3] if grad) for unit vectors u [n, 3]."""
    u = np.asarray(u, np.float64)
    x, y, z = u[:, 0], u[:, 1], u[:, 2]
    Q = _legendre_derivs(z, lmax)
    w = x + 1j * y
    # powers of w and their x / y derivatives
    wp = [np.ones_like(w)]
    for k in range(1, lmax + 1):
        wp.append(wp[-1] * w)
    n = len(u)
    Y = np.zeros((n, (lmax + 1) ** 2))
    dY = np.zeros((n, (lmax + 1) ** 2, 3)) if grad else None
    for l in range(lmax + 1):
        for m in range(-l, l + 1):
            am = abs(m)
            nn = _norm(l, m)
            if m > 0:
                T = wp[am].real
                dTx = am * wp[am - 1].real
                dTy = -am * wp[am - 1].imag
            elif m < 0:
                T = wp[am].imag
                dTx = am * wp[am - 1].imag
                dTy = am * wp[am - 1].real
            else:
                T = np.ones_like(x)
                dTx = np.zeros_like(x)
                dTy = np.zeros_like(x)
            k = lm_index(l, m)
            Y[:, k] = nn * Q[(l, am)] * T
            if grad:
                q1 = Q[(l, am + 1)] if am + 1 <= l else np.zeros_like(z)
                dY[:, k, 0] = nn * Q[(l, am)] * dTx
                dY[:, k, 1] = nn * Q[(l, am)] * dTy
                dY[:, k, 2] = nn * q1 * T
    return (Y, dY) if grad else Y


def l_of_index(lmax: int = LMAX) -> np.ndarray:
    return np.array([l for l in range(lmax + 1) for _ in range(2 * l + 1)], dtype=np.int64)
