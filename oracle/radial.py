"""Radial basis functions of the edge length and their derivatives (test infrastructure: the CPU
oracle of the fused radial basis; only tests, smoke() and the benchmark's CPU baseline use it).

The pages feed the convolution a radial embedding phi_ij (Sobek section 2.4, Eq. 12: W = phi A)
and name an envelope option (LunaTP, Appendix "Usage") without printing formulas.  The plainest
reading, used by the synthetic workloads as well:

* kind 1, Bessel: phi_n(r) = sqrt(2 / r_c) sin(n pi r / r_c) / r * u(r / r_c), n = 1..K, with the
  polynomial envelope of exponent p = 6, u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 (zero value, slope
  and curvature at d = 1), and phi = 0 for r >= r_c;
* kind 2, Gaussian: phi_k(r) = exp(-(r - mu_k)^2 / (2 D^2)), mu_k = k r_c / (K - 1), k = 0..K-1,
  D = r_c / (K - 1), no envelope.

The derivative enters the position gradient: e-bar += (sum_q phi-bar_q dphi_q/dr) r-hat.  The
double backward of a convolution that computes phi from |r| (the force-training path) also needs
the second derivative (double_backward below).

Pins (tests/test_oracle.py): the envelope's value, slope and curvature at both ends, the
orthonormality of the envelope-free Bessel functions under r^2 dr on [0, r_c], the Gaussian's peak
and width, complex-step first and second derivatives, finite differences of the whole forward in
the positions, and for the double backward torch autograd of the forward taken twice and central
differences of the first-order backward.
"""

from __future__ import annotations

import math

import torch

_F64 = torch.float64
BESSEL, GAUSSIAN = 1, 2


def envelope(d: torch.Tensor) -> torch.Tensor:
    """u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 for d < 1, else 0."""
    u = 1.0 - 28.0 * d ** 6 + 48.0 * d ** 7 - 21.0 * d ** 8
    return torch.where(d < 1.0, u, torch.zeros_like(u))


def basis(kind: int, r, r_cut: float, K: int, envelope_on: bool = True) -> torch.Tensor:
    """(E, K) radial basis values at edge lengths r (complex r allowed for complex-step checks)."""
    r = torch.as_tensor(r)
    if not torch.is_complex(r):
        r = r.to(_F64)
    if kind == BESSEL:
        n = torch.arange(1, K + 1, dtype=_F64)
        v = math.sqrt(2.0 / r_cut) * torch.sin(r[:, None] * n[None, :] * (math.pi / r_cut)) / r[:, None]
        if envelope_on:
            d = r / r_cut
            u = 1.0 - 28.0 * d ** 6 + 48.0 * d ** 7 - 21.0 * d ** 8
            if not torch.is_complex(r):
                u = torch.where(d < 1.0, u, torch.zeros_like(u))
            v = v * u[:, None]
        return v
    if kind == GAUSSIAN:
        mu = torch.arange(K, dtype=_F64) * (r_cut / (K - 1))
        delta = r_cut / (K - 1)
        return torch.exp(-((r[:, None] - mu[None, :]) ** 2) / (2.0 * delta * delta))
    raise ValueError(f"unknown radial kind {kind}")


def basis_derivative(kind: int, r, r_cut: float, K: int) -> torch.Tensor:
    """(E, K) d phi / d r, by the product and chain rules."""
    r = torch.as_tensor(r, dtype=_F64)
    if kind == BESSEL:
        n = torch.arange(1, K + 1, dtype=_F64)
        a = n[None, :] * (math.pi / r_cut)
        s, c = torch.sin(a * r[:, None]), torch.cos(a * r[:, None])
        b = math.sqrt(2.0 / r_cut) * s / r[:, None]
        db = math.sqrt(2.0 / r_cut) * (a * c * r[:, None] - s) / (r[:, None] ** 2)
        d = r / r_cut
        u = 1.0 - 28.0 * d ** 6 + 48.0 * d ** 7 - 21.0 * d ** 8
        du = (-168.0 * d ** 5 + 336.0 * d ** 6 - 168.0 * d ** 7) / r_cut
        inside = (d < 1.0)[:, None]
        return torch.where(inside, db * u[:, None] + b * du[:, None], torch.zeros_like(b))
    if kind == GAUSSIAN:
        mu = torch.arange(K, dtype=_F64) * (r_cut / (K - 1))
        delta = r_cut / (K - 1)
        diff = r[:, None] - mu[None, :]
        return -diff / (delta * delta) * torch.exp(-(diff ** 2) / (2.0 * delta * delta))
    raise ValueError(f"unknown radial kind {kind}")


def edge_lengths(edge_vec) -> torch.Tensor:
    ev = torch.as_tensor(edge_vec, dtype=_F64)
    return torch.sqrt((ev ** 2).sum(1))


def edge_vec_grad(kind: int, edge_vec, r_cut: float, gphi) -> torch.Tensor:
    """The radial part of the edge-vector gradient: (sum_q phi-bar_q dphi_q/dr) r / |r|."""
    ev = torch.as_tensor(edge_vec, dtype=_F64)
    gphi = torch.as_tensor(gphi, dtype=_F64)
    r = edge_lengths(ev)
    s = (gphi * basis_derivative(kind, r, r_cut, gphi.shape[1])).sum(1)
    return (s / r)[:, None] * ev


def basis_second_derivative(kind: int, r, r_cut: float, K: int) -> torch.Tensor:
    """(E, K) d^2 phi / d r^2, by the product rule on basis_derivative's factors."""
    r = torch.as_tensor(r, dtype=_F64)
    if kind == BESSEL:
        n = torch.arange(1, K + 1, dtype=_F64)
        a = n[None, :] * (math.pi / r_cut)
        rr = r[:, None]
        s, c = torch.sin(a * rr), torch.cos(a * rr)
        nrm = math.sqrt(2.0 / r_cut)
        b = nrm * s / rr
        db = nrm * (a * c * rr - s) / rr ** 2
        d2b = nrm * (2.0 * s - 2.0 * a * rr * c - a * a * rr * rr * s) / rr ** 3
        d = r / r_cut
        u = 1.0 - 28.0 * d ** 6 + 48.0 * d ** 7 - 21.0 * d ** 8
        du = (-168.0 * d ** 5 + 336.0 * d ** 6 - 168.0 * d ** 7) / r_cut
        d2u = (-840.0 * d ** 4 + 2016.0 * d ** 5 - 1176.0 * d ** 6) / (r_cut * r_cut)
        inside = (d < 1.0)[:, None]
        v = d2b * u[:, None] + 2.0 * db * du[:, None] + b * d2u[:, None]
        return torch.where(inside, v, torch.zeros_like(v))
    if kind == GAUSSIAN:
        mu = torch.arange(K, dtype=_F64) * (r_cut / (K - 1))
        delta = r_cut / (K - 1)
        diff = r[:, None] - mu[None, :]
        g = torch.exp(-(diff ** 2) / (2.0 * delta * delta))
        return (diff * diff / delta ** 4 - 1.0 / (delta * delta)) * g
    raise ValueError(f"unknown radial kind {kind}")


def double_backward(kind: int, r_cut: float, problem, x, edge_vec, recv, send, A, grad_out, v_x=None, v_e=None,
                    v_A=None, n_nodes=None):
    """Double backward of the convolution whose radial values are phi = basis(|r|) (no phi input).

    The first-order map is (x, r, A, mbar) -> (x-bar, r-bar, A-bar) with r-bar = e-bar + J_phi(r)^T
    phi-bar.  Its second-order pairing along (v_x, v_e, v_A) equals that of the phi-input map with
    the radial direction phidot = J_phi(r) v_e = phi'(|r|) (r-hat . v_e), so every gradient but
    the edge vector's is the phi-input double backward's.  The edge vector's gains, beside the
    direct part, the chain through phi, J_phi^T (gradient of the pairing in phi), and the
    curvature of phi: grad_r [s(|r|) (r-hat . v_e)] with s = sum_q phi-bar_q phi'_q, which is
    s' t r-hat + s (v_e - t r-hat) / |r| for t = r-hat . v_e, s' = sum_q phi-bar_q phi''_q, where
    phi-bar is the first-order gradient of the radial values.
    Returns the phi-input double backward's dictionary with edge_vec and pos replaced; its "phi"
    entry is the gradient of the pairing in the radial values.
    """
    from . import conv
    ev = torch.as_tensor(edge_vec, dtype=_F64)
    E = ev.shape[0]
    K = torch.as_tensor(A).shape[0]
    ve = torch.zeros(E, 3, dtype=_F64) if v_e is None else torch.as_tensor(v_e, dtype=_F64)
    r = edge_lengths(ev)
    n = ev / r[:, None]
    t = (n * ve).sum(1)
    phi = basis(kind, r, r_cut, K)
    dphi = basis_derivative(kind, r, r_cut, K)
    v_phi = dphi * t[:, None]
    gg = conv.double_backward(problem, x, ev, recv, send, phi, A, grad_out, v_x=v_x, v_e=ve, v_phi=v_phi,
                              v_A=v_A, n_nodes=n_nodes)
    phibar = conv.backward(problem, x, ev, recv, send, phi, A, grad_out, n_nodes=n_nodes)["phi"]
    s = (phibar * dphi).sum(1)
    s2 = (phibar * basis_second_derivative(kind, r, r_cut, K)).sum(1)
    chain = (gg["phi"] * dphi).sum(1)[:, None] * n
    curv = (s2 * t)[:, None] * n + (s / r)[:, None] * (ve - t[:, None] * n)
    ge = gg["edge_vec"] + chain + curv
    N = gg["pos"].shape[0]
    gpos = torch.zeros(N, 3, dtype=_F64)
    gpos.index_add_(0, torch.as_tensor(send, dtype=torch.long), ge)
    gpos.index_add_(0, torch.as_tensor(recv, dtype=torch.long), -ge)
    return dict(gg, edge_vec=ge, pos=gpos)
