"""Real spherical harmonics, fp64.  Test infrastructure (see oracle/__init__).

Convention (a reading: the pages name irreps and L_max but print no basis):
component index of (l, m) is l*l + l + m for m = -l..l, z is the polar axis,
no Condon-Shortley phase, orthonormal on the unit sphere:

    Y_{l,0}      = N_{l,0} P_l(cos t)
    Y_{l,m>0}    = sqrt(2) N_{l,m} P_l^m(cos t) cos(m p)
    Y_{l,m<0}    = sqrt(2) N_{l,|m|} P_l^|m|(cos t) sin(|m| p)
    N_{l,m}      = sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!)
    P_l^m(x)     = (1 - x^2)^(m/2) d^m/dx^m P_l(x)      (no (-1)^m)

so that l = 1 is sqrt(3/(4 pi)) (y, z, x).  The edge-aligned frame of the
E2Former-V2 summary (technical section 2.1, Lemma 4.1: only m = 0 survives
on the aligned axis) is the statement Y_l(z_hat) = sqrt((2l+1)/(4 pi)) e_{m=0},
which holds in this basis and is pinned by the tests.
"""

from functools import lru_cache
from math import factorial, pi, sqrt

import numpy as np
from numpy.polynomial import legendre as npleg


def n_comp(l_max: int) -> int:
    """Number of irreps components up to degree l_max: (L+1)^2."""
    return (l_max + 1) * (l_max + 1)


@lru_cache(maxsize=None)
def _legendre_deriv(l: int, m: int):
    """d^m/dx^m P_l as a Legendre series (a constant of (l, m); kept once)."""
    series = npleg.Legendre.basis(l)
    if m:
        series = series.deriv(m)
    return series


def _assoc_legendre(l: int, m: int, ct: np.ndarray, st: np.ndarray) -> np.ndarray:
    """P_l^m(cos t) without the Condon-Shortley phase, straight from its
    definition: (1-x^2)^(m/2) times the m-th derivative of the Legendre
    polynomial P_l at x = cos t (numpy's Legendre series supplies P_l and
    d/dx).  (1-x^2)^(1/2) = sin t is passed in, taken from the Cartesian
    components, so that it keeps full precision next to the poles."""
    return st**m * _legendre_deriv(l, m)(ct)


def real_sh(l_max: int, v) -> np.ndarray:
    """Y(v) for v of shape [n, 3] (normalised here), returns [n, (L+1)^2]."""
    v = np.asarray(v, dtype=np.float64).reshape(-1, 3)
    r = np.sqrt(np.sum(v * v, axis=1))
    u = v / r[:, None]
    ct = np.clip(u[:, 2], -1.0, 1.0)
    st = np.hypot(u[:, 0], u[:, 1])
    ph = np.arctan2(u[:, 1], u[:, 0])
    out = np.zeros((v.shape[0], n_comp(l_max)), dtype=np.float64)
    for l in range(l_max + 1):
        for m in range(0, l + 1):
            nlm = sqrt((2 * l + 1) / (4.0 * pi) * factorial(l - m) / factorial(l + m))
            plm = _assoc_legendre(l, m, ct, st)
            if m == 0:
                out[:, l * l + l] = nlm * plm
            else:
                out[:, l * l + l + m] = sqrt(2.0) * nlm * plm * np.cos(m * ph)
                out[:, l * l + l - m] = sqrt(2.0) * nlm * plm * np.sin(m * ph)
    return out
