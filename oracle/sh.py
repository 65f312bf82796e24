"""Real spherical harmonics, component normalised (oracle; test infrastructure only).

Sobek (section 2.4, Eq. 7) feeds the unit edge direction r_hat = r / |r| to
the spherical harmonics Y(r_hat); the pages fix neither basis nor
normalisation.  Reading taken here: the real combination of the complex
Condon-Shortley harmonics (``cg.complex_to_real``), scaled so that
sum_mu Y_l,mu^2 = 2l + 1, with mu = -l..l.  Written as polynomials in the unit
vector n = (x, y, z):

    Y_l,mu(n) = sqrt((2l+1) (l-|mu|)! / (l+|mu|)!) * s_mu * P_l^(|mu|)(z) * t_mu(x, y)

where P_l^(k) is the k-th derivative of the Legendre polynomial P_l,
s_mu = sqrt2 for mu != 0 (1 otherwise), and t_mu = Re (x + i y)^mu for mu > 0,
Im (x + i y)^|mu| for mu < 0, 1 for mu = 0.  So Y_1 = sqrt3 (y, z, x).

Everything is a polynomial in (x, y, z) after the normalisation
n = r / sqrt(x^2 + y^2 + z^2), so the functions accept complex tensors
(complex-step derivatives) and torch autograd (first and second derivatives).
"""

from __future__ import annotations

import math
from typing import List

import torch


def _legendre_coeffs(l: int) -> List[float]:
    """Coefficients a_n of P_l(z) = sum_n a_n z^n (exact rationals as floats)."""
    a = [0.0] * (l + 1)
    for k in range(l // 2 + 1):
        a[l - 2 * k] = ((-1) ** k) * math.comb(l, k) * math.comb(2 * l - 2 * k, l) / 2.0 ** l
    return a


def _deriv(coeffs: List[float], k: int) -> List[float]:
    c = list(coeffs)
    for _ in range(k):
        c = [n * c[n] for n in range(1, len(c))] or [0.0]
    return c


def _poly(c: List[float], z: torch.Tensor) -> torch.Tensor:
    out = torch.zeros_like(z)
    for coef in reversed(c):
        out = out * z + coef
    return out


def _ipow(v: torch.Tensor, k: int) -> torch.Tensor:
    """v**k by repeated products (exact for complex-step arguments, unlike exp-log powers)."""
    out = torch.ones_like(v)
    for _ in range(k):
        out = out * v
    return out


def _xy_power(m: int, x: torch.Tensor, y: torch.Tensor):
    """(Re, Im) of (x + i y)^m expanded as real polynomials (analytic in x, y)."""
    re = torch.zeros_like(x)
    im = torch.zeros_like(x)
    for k in range(m + 1):
        term = math.comb(m, k) * _ipow(x, m - k) * _ipow(y, k)
        if k % 2 == 0:
            re = re + ((-1) ** (k // 2)) * term
        else:
            im = im + ((-1) ** ((k - 1) // 2)) * term
    return re, im


def unit(r: torch.Tensor) -> torch.Tensor:
    """r / |r| with |r| = sqrt(x^2 + y^2 + z^2) (kept analytic for complex steps)."""
    n2 = (r * r).sum(-1, keepdim=True)
    return r / torch.sqrt(n2)


def sh_l(l: int, n: torch.Tensor) -> torch.Tensor:
    """Y_l(n) for unit vectors n (..., 3) -> (..., 2l+1)."""
    x, y, z = n[..., 0], n[..., 1], n[..., 2]
    P = _legendre_coeffs(l)
    cols = [None] * (2 * l + 1)
    for a in range(l + 1):
        norm = math.sqrt((2 * l + 1) * math.factorial(l - a) / math.factorial(l + a))
        d = _poly(_deriv(P, a), z)
        if a == 0:
            cols[l] = norm * d
        else:
            re, im = _xy_power(a, x, y)
            cols[l + a] = math.sqrt(2.0) * norm * d * re
            cols[l - a] = math.sqrt(2.0) * norm * d * im
    return torch.stack(cols, dim=-1)


def sh(lmax: int, r: torch.Tensor) -> torch.Tensor:
    """Concatenated Y_0..Y_lmax of r / |r|; r is (..., 3), result (..., (lmax+1)^2)."""
    n = unit(r)
    return torch.cat([sh_l(l, n) for l in range(lmax + 1)], dim=-1)
