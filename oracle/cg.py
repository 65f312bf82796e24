"""Real Clebsch-Gordan coupling tensors (oracle; test infrastructure only).

The coupling of LunaTP (section 2.1, Eq. 1) and of Sobek's per-path angular
contraction (section 4.2, Eq. 32) uses coefficients c^pi[m1, m2, m3] that the
pages do not print.  The reading taken here:

1. complex <l1 m1 l2 m2 | l3 m3> from the closed-form Racah sum, evaluated in
   exact rational arithmetic with a single square root at the end;
2. change to the real basis of the real spherical harmonics (see ``sh``):
   with Y_real = U Y_complex,
   c[a, b, c] = sum U_l3[c, M] conj(U_l1[a, m1]) conj(U_l2[b, m2]) <l1 m1 l2 m2|l3 M>,
   which is purely real or purely imaginary; the non-zero part is kept;
3. the whole (l1, l2, l3) tensor is multiplied by -1 if needed so that its
   first non-zero entry in row-major (m1, m2, m3) order is positive.

Indices run m = 0 .. 2l over mu = m - l = -l .. l.  The result is unitary:
sum_{m1, m2} c[m1, m2, m3] c[m1, m2, m3'] = delta(m3, m3').
"""

from __future__ import annotations

import functools
import math
from fractions import Fraction

import numpy as np


def _f(n: int) -> int:
    return math.factorial(n)


def complex_cg(l1: int, m1: int, l2: int, m2: int, l3: int, m3: int) -> float:
    """<l1 m1 l2 m2 | l3 m3> by the Racah formula (exact rational, one sqrt)."""
    if m3 != m1 + m2:
        return 0.0
    if not (abs(l1 - l2) <= l3 <= l1 + l2):
        return 0.0
    if abs(m1) > l1 or abs(m2) > l2 or abs(m3) > l3:
        return 0.0
    pre = Fraction((2 * l3 + 1) * _f(l3 + l1 - l2) * _f(l3 - l1 + l2) * _f(l1 + l2 - l3),
                   _f(l1 + l2 + l3 + 1))
    pre *= (_f(l3 + m3) * _f(l3 - m3) * _f(l1 - m1) * _f(l1 + m1) * _f(l2 - m2) * _f(l2 + m2))
    s = Fraction(0)
    for k in range(0, l1 + l2 + l3 + 1):
        d = [k, l1 + l2 - l3 - k, l1 - m1 - k, l2 + m2 - k, l3 - l2 + m1 + k, l3 - l1 - m2 + k]
        if min(d) < 0:
            continue
        den = 1
        for v in d:
            den *= _f(v)
        s += Fraction((-1) ** k, den)
    if s == 0:
        return 0.0
    val2 = s * s * pre  # exact square of the coefficient
    return math.copysign(math.sqrt(val2.numerator) / math.sqrt(val2.denominator)
                         if val2.numerator < 2 ** 1000 else math.sqrt(float(val2)), float(s))


def complex_to_real(l: int) -> np.ndarray:
    """U_l with Y_real[mu] = sum_m U[mu, m] Y_complex[m] (Condon-Shortley complex Y).

    mu > 0: ((-1)^mu Y^mu + Y^-mu)/sqrt2;  mu = 0: Y^0;
    mu < 0: i (Y^mu - (-1)^|mu| Y^|mu|)/sqrt2.
    """
    U = np.zeros((2 * l + 1, 2 * l + 1), dtype=np.complex128)
    r = 1.0 / math.sqrt(2.0)
    for mu in range(-l, l + 1):
        row = mu + l
        if mu > 0:
            U[row, mu + l] = (-1) ** mu * r
            U[row, -mu + l] = r
        elif mu == 0:
            U[row, l] = 1.0
        else:
            a = -mu
            U[row, mu + l] = 1j * r
            U[row, a + l] = -1j * (-1) ** a * r
    return U


@functools.lru_cache(maxsize=None)
def complex_cg_tensor(l1: int, l2: int, l3: int) -> np.ndarray:
    t = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            m3 = m1 + m2
            if abs(m3) <= l3:
                t[m1 + l1, m2 + l2, m3 + l3] = complex_cg(l1, m1, l2, m2, l3, m3)
    return t


@functools.lru_cache(maxsize=None)
def real_cg(l1: int, l2: int, l3: int) -> np.ndarray:
    """Real coupling tensor c[m1, m2, m3] of shape (2l1+1, 2l2+1, 2l3+1); zeros if forbidden."""
    shape = (2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)
    if not (abs(l1 - l2) <= l3 <= l1 + l2):
        return np.zeros(shape)
    C = complex_cg_tensor(l1, l2, l3)
    U1, U2, U3 = complex_to_real(l1), complex_to_real(l2), complex_to_real(l3)
    c = np.einsum("am,bn,cp,mnp->abc", np.conj(U1), np.conj(U2), U3, C)
    re, im = np.abs(c.real).max(), np.abs(c.imag).max()
    if re >= im:
        assert im < 1e-14, (l1, l2, l3, im)
        out = c.real.copy()
    else:
        assert re < 1e-14, (l1, l2, l3, re)
        out = c.imag.copy()
    out[np.abs(out) < 1e-15] = 0.0
    flat = out.reshape(-1)
    first = flat[np.nonzero(flat)[0][0]]
    if first < 0:
        out = -out
    return out


def sparse_terms(l1: int, l2: int, l3: int):
    """Non-zero entries of ``real_cg`` as a list of (m1, m2, m3, value) in row-major order."""
    c = real_cg(l1, l2, l3)
    idx = np.argwhere(c != 0.0)
    return [(int(a), int(b), int(d), float(c[a, b, d])) for a, b, d in idx]
