"""Forward, backward and double backward of the CGTP convolution (oracle).

TEST INFRASTRUCTURE ONLY.  Plain float64 PyTorch CPU code written from:

* Sobek section 2.4, Eq. 7: r_ij = r_j - r_i (here pos[send] - pos[recv] + shift);
* Sobek section 2.4, Eqs. 11-12 and LunaTP Algorithm 1: the conventional
  schedule, m_i = sum_j sum_pi sum_a W_ij,pi,a T_pi,a(x_j, Y_ij) with
  W = phi A materialised per path;
* Sobek section 4.2, Eqs. 32-35: the streamed schedule, receiver state
  S_i,pi,q,u,mo = sum_j phi_ij,q C_pi,u,mo(x_j, Y_ij), then m = S A;
* Sobek section 3.2, Eqs. 18-22: the backward (h, A-bar, phi-bar, x-bar,
  Y-bar), followed by the chain rule through Y(r) for the edge-vector and
  position gradients;
* Sobek section 3.3, Eqs. 23-31: the double backward, assembled as the
  vector-Jacobian product of the backward map.

The per-path angular contraction is LunaTP Eq. 1 with the real coupling
tensors of ``cg``; no path normalisation factor beyond them (alpha_pi = 1).
Loops run over paths (and, where memory demands, over edge or radial slices);
everything inside a path is an einsum over edges and channels.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import cg as _cg
from . import sh as _sh
from .irreps import Problem

_F64 = torch.float64


def _t(a) -> torch.Tensor:
    if isinstance(a, torch.Tensor):
        return a.to(_F64)
    return torch.as_tensor(np.asarray(a), dtype=_F64)


def _idx(a) -> torch.Tensor:
    return torch.as_tensor(np.asarray(a), dtype=torch.long)


def edge_vectors(pos, shift, recv, send) -> torch.Tensor:
    """Sobek Eq. 7: r_ij = r_j - r_i for edge i <- j, plus the periodic image shift."""
    pos, shift = _t(pos), _t(shift)
    recv, send = _idx(recv), _idx(send)
    return pos[send] - pos[recv] + shift


def _block(feat: torch.Tensor, b) -> torch.Tensor:
    """View of block b of an ir_mul feature matrix as (rows, 2l+1, mul)."""
    return feat[:, b.offset:b.offset + b.size].reshape(feat.shape[0], b.dim, b.mul)


def _coupling(p) -> torch.Tensor:
    return torch.as_tensor(_cg.real_cg(p.l1, p.l2, p.l3), dtype=_F64)


def spherical_harmonics(problem: Problem, edge_vec) -> torch.Tensor:
    return _sh.sh(problem.lmax_sh, _t(edge_vec))


def _angular(problem: Problem, p, x: torch.Tensor, Y: torch.Tensor, send: torch.Tensor) -> torch.Tensor:
    """T_pi(x_j, Y_ij)[e, m3, u] = sum_{m1, m2} c[m1, m2, m3] x_j[m1, u] Y[m2] (LunaTP Eq. 1)."""
    bi, bs = problem.irreps_in[p.i_in], problem.irreps_sh[p.i_sh]
    xj = _block(x, bi)[send]                      # (E, d1, C)
    Yb = Y[:, bs.offset:bs.offset + bs.dim]       # (E, d2)
    return torch.einsum("abc,eau,eb->ecu", _coupling(p), xj, Yb)


def forward_conventional(problem: Problem, x, edge_vec, recv, send, phi, A,
                         edge_chunk: int = 1 << 14) -> torch.Tensor:
    """Sobek Eqs. 11-12: materialise W = phi A per path, form each edge message, sum into receivers."""
    Y = spherical_harmonics(problem, edge_vec)
    return forward_from_sh(problem, x, Y, recv, send, phi, A, edge_chunk=edge_chunk)


def forward_from_sh(problem: Problem, x, Y, recv, send, phi, A, n_nodes: Optional[int] = None,
                    edge_chunk: int = 1 << 14) -> torch.Tensor:
    """The conventional forward with the edge operand given: Y (E x sh_dim) holds the angular edge
    values (the real harmonics of the edge directions in forward_conventional; LunaTP Eq. 1 and
    Algorithm 1 take them as the input y)."""
    x, phi, A, Y = _t(x), _t(phi), _t(A), _t(Y)
    recv, send = _idx(recv), _idx(send)
    N = x.shape[0] if n_nodes is None else n_nodes
    E = recv.shape[0]
    out = torch.zeros(N, problem.c_out, dtype=_F64)
    for p in problem.paths:
        bo = problem.irreps_out[p.i_out]
        Ap = A[:, p.weight_offset:p.weight_offset + p.n_weights]
        acc = torch.zeros(N, bo.dim, bo.mul, dtype=_F64)
        for s in range(0, E, edge_chunk):
            sl = slice(s, min(E, s + edge_chunk))
            T = _angular(problem, p, x, Y[sl], send[sl])            # (e, d3, C_in)
            W = phi[sl] @ Ap                                        # materialised edge weights
            if problem.mode == "uvu":
                msg = W[:, None, :] * T
            else:
                W = W.reshape(-1, T.shape[2], bo.mul)               # (e, u, w)
                msg = torch.einsum("euw,ecu->ecw", W, T)
            acc.index_add_(0, recv[sl], msg)
        out[:, bo.offset:bo.offset + bo.size] += acc.reshape(N, -1)
    return out


def receiver_state(problem: Problem, p, x, Y, recv, send, phi, N: int) -> torch.Tensor:
    """Sobek Eq. 33: S[i, q, m3, u] = sum_{j in N(i)} phi_ij,q C_pi,u,m3(x_j, Y_ij)."""
    Cang = _angular(problem, p, x, Y, send)                          # Eq. 32, (E, d3, C_in)
    K = phi.shape[1]
    S = torch.zeros(N, K, Cang.shape[1], Cang.shape[2], dtype=_F64)
    for q in range(K):
        S[:, q].index_add_(0, recv, phi[:, q, None, None] * Cang)
    return S


def forward_streamed(problem: Problem, x, edge_vec, recv, send, phi, A) -> torch.Tensor:
    """Sobek Eqs. 33-35: receiver state S per path, then the channel product m = S A."""
    x, phi, A = _t(x), _t(phi), _t(A)
    recv, send = _idx(recv), _idx(send)
    N, K = x.shape[0], phi.shape[1]
    Y = spherical_harmonics(problem, edge_vec)
    out = torch.zeros(N, problem.c_out, dtype=_F64)
    for p in problem.paths:
        bi, bo = problem.irreps_in[p.i_in], problem.irreps_out[p.i_out]
        S = receiver_state(problem, p, x, Y, recv, send, phi, N)    # (N, K, d3, C_in)
        Ap = A[:, p.weight_offset:p.weight_offset + p.n_weights]
        if problem.mode == "uvu":
            m = torch.einsum("iqcu,qu->icu", S, Ap)
        else:
            m = torch.einsum("iqcu,quw->icw", S, Ap.reshape(K, bi.mul, bo.mul))
        out[:, bo.offset:bo.offset + bo.size] += m.reshape(N, -1)
    return out


def _sh_vjp(problem: Problem, edge_vec, Ybar: torch.Tensor) -> torch.Tensor:
    """Chain rule through Y(r / |r|): returns J_Y(r)^T Ybar per edge."""
    r = _t(edge_vec).clone().requires_grad_(True)
    Y = _sh.sh(problem.lmax_sh, r)
    (g,) = torch.autograd.grad(Y, r, grad_outputs=Ybar)
    return g.detach()


def backward(problem: Problem, x, edge_vec, recv, send, phi, A, grad_out,
             n_nodes: Optional[int] = None, edge_chunk: int = 1 << 14) -> Dict[str, torch.Tensor]:
    """Sobek Eqs. 18-22 plus the chain rule through Y(r) and r = pos[send] - pos[recv] + shift.

    h_ij,pi,a = <mbar_i, T_pi,a(x_j, Y_ij)>;  Abar = sum phi h;  phibar = sum_pi,a A h;
    xbar_j = sum_{i: j in N(i)} sum_pi,a w D_x T* mbar_i;  Ybar_ij = sum_pi,a w D_Y T* mbar_i;
    ebar = J_Y^T Ybar;  posbar = sum_{out-edges} ebar - sum_{in-edges} ebar.
    """
    x, phi, A, gout = _t(x), _t(phi), _t(A), _t(grad_out)
    recv, send = _idx(recv), _idx(send)
    N = x.shape[0] if n_nodes is None else n_nodes
    E, K = recv.shape[0], phi.shape[1]
    Y = spherical_harmonics(problem, edge_vec)
    gx = torch.zeros_like(x)
    gphi = torch.zeros(E, K, dtype=_F64)
    gA = torch.zeros_like(A)
    gY = torch.zeros(E, problem.sh_dim, dtype=_F64)
    for p in problem.paths:
        bi, bs, bo = problem.irreps_in[p.i_in], problem.irreps_sh[p.i_sh], problem.irreps_out[p.i_out]
        c = _coupling(p)
        Ap = A[:, p.weight_offset:p.weight_offset + p.n_weights]
        gAp = torch.zeros_like(Ap)
        gxb = torch.zeros(x.shape[0], bi.dim, bi.mul, dtype=_F64)
        for s in range(0, E, edge_chunk):
            sl = slice(s, min(E, s + edge_chunk))
            rs, ss = recv[sl], send[sl]
            Yb = Y[sl, bs.offset:bs.offset + bs.dim]
            xj = _block(x, bi)[ss]                       # (e, d1, C_in)
            mb = _block(gout, bo)[rs]                    # (e, d3, C_out)
            T = torch.einsum("abc,eau,eb->ecu", c, xj, Yb)
            W = phi[sl] @ Ap
            if problem.mode == "uvu":
                h = (mb * T).sum(1)                                              # Eq. 18
                Bx = torch.einsum("abc,eb,ecu->eau", c, Yb, mb)                  # D_x T* mbar
                gxb.index_add_(0, ss, W[:, None, :] * Bx)                        # Eq. 21
                gY[sl, bs.offset:bs.offset + bs.dim] += torch.einsum(
                    "abc,eau,ecu,eu->eb", c, xj, mb, W)                          # Eq. 22
            else:
                W = W.reshape(-1, bi.mul, bo.mul)
                h = torch.einsum("ecw,ecu->euw", mb, T).reshape(-1, p.n_weights)  # Eq. 18
                Bx = torch.einsum("abc,eb,ecw->eaw", c, Yb, mb)
                gxb.index_add_(0, ss, torch.einsum("euw,eaw->eau", W, Bx))       # Eq. 21
                gY[sl, bs.offset:bs.offset + bs.dim] += torch.einsum(
                    "abc,eau,ecw,euw->eb", c, xj, mb, W)                         # Eq. 22
            gAp += phi[sl].T @ h                                                 # Eq. 19
            gphi[sl] += h @ Ap.T                                                 # Eq. 20
        gA[:, p.weight_offset:p.weight_offset + p.n_weights] = gAp
        gx[:, bi.offset:bi.offset + bi.size] += gxb.reshape(x.shape[0], -1)
    ge = _sh_vjp(problem, edge_vec, gY)
    gpos = torch.zeros(N, 3, dtype=_F64)
    gpos.index_add_(0, send, ge)
    gpos.index_add_(0, recv, -ge)
    return dict(x=gx, edge_vec=ge, pos=gpos, phi=gphi, A=gA, Y=gY)


def grad_A_streamed(problem: Problem, x, edge_vec, recv, send, phi, grad_out, n_nodes: Optional[int] = None,
                    paths=None):
    """Sobek Eq. 36: A-bar = S^T mbar with the receiver state S of Eq. 33 (per path).

    ``paths`` (indices) restricts the result to those paths' columns, concatenated in order.
    """
    x, phi, gout = _t(x), _t(phi), _t(grad_out)
    recv, send = _idx(recv), _idx(send)
    N = x.shape[0] if n_nodes is None else n_nodes
    K = phi.shape[1]
    Y = spherical_harmonics(problem, edge_vec)
    cols = []
    for p in problem.paths:
        if paths is not None and p.index not in paths:
            continue
        bi, bo = problem.irreps_in[p.i_in], problem.irreps_out[p.i_out]
        S = receiver_state(problem, p, x, Y, recv, send, phi, N)     # (N, K, d3, C_in)
        mb = _block(gout, bo)                                         # (N, d3, C_out)
        if problem.mode == "uvu":
            g = torch.einsum("iqcu,icu->qu", S, mb)
        else:
            g = torch.einsum("iqcu,icw->quw", S, mb).reshape(K, -1)
        cols.append(g)
    return torch.cat(cols, dim=1)


def _sh_jvp(problem: Problem, edge_vec, v_e: torch.Tensor) -> torch.Tensor:
    """Ydot = J_Y(r) v_e: directional derivative of the harmonics along v_e (per edge)."""
    r = _t(edge_vec).clone().requires_grad_(True)
    Y = _sh.sh(problem.lmax_sh, r)
    u = torch.zeros_like(Y, requires_grad=True)
    (g,) = torch.autograd.grad(Y, r, grad_outputs=u, create_graph=True)   # J^T u, linear in u
    (jv,) = torch.autograd.grad(g, u, grad_outputs=_t(v_e))               # J v
    return jv.detach()


def _sh_hvp(problem: Problem, edge_vec, v_e: torch.Tensor, Ybar: torch.Tensor) -> torch.Tensor:
    """grad_r < J_Y(r) v_e, Ybar >: the second-derivative term of the edge-vector double backward."""
    r = _t(edge_vec).clone().requires_grad_(True)
    Y = _sh.sh(problem.lmax_sh, r)
    (g,) = torch.autograd.grad(Y, r, grad_outputs=_t(Ybar), create_graph=True)  # J^T Ybar
    (h,) = torch.autograd.grad(g, r, grad_outputs=_t(v_e))                     # d/dr <J^T Ybar, v_e>
    return h.detach()


def double_backward(problem: Problem, x, edge_vec, recv, send, phi, A, grad_out, v_x=None, v_e=None,
                    v_phi=None, v_A=None, n_nodes: Optional[int] = None,
                    edge_chunk: int = 1 << 14) -> Dict[str, torch.Tensor]:
    """Vector-Jacobian product of the backward map (x, r, phi, A, mbar) -> (xbar, ebar, phibar, Abar).

    With the directions xdot = v_x, rdot = v_e, phidot = v_phi, Adot = v_A (Sobek section 3.3):
      wdot = phidot A + phi Adot (Eq. 23), Tdot = D_x T[xdot] + D_Y T[Ydot], Ydot = J_Y(r) rdot (Eq. 24),
      mdot = sum (wdot T + w Tdot) (Eq. 25), hdot = <mbar, Tdot> (+ <mbardot, T>, no mbar direction here),
      Abar-dot = sum phidot h + phi hdot (Eq. 26), phibar-dot = sum Adot h + A hdot (Eq. 27),
      xbar-dot = sum wdot B^x + w Bdot^x with Bdot^x = D_x T(., Ydot)* mbar (Eq. 30),
      Ybar-dot = sum wdot B^Y + w Bdot^Y with Bdot^Y = D_Y T(xdot, .)* mbar (Eq. 31).
    The VJP with respect to mbar is mdot; with respect to r it is J_Y^T Ybar-dot plus the curvature
    term grad_r <J_Y(r) rdot, Ybar> with the first-order Ybar of Eq. 22.
    Missing directions are zero.
    """
    x, phi, A, gout = _t(x), _t(phi), _t(A), _t(grad_out)
    recv, send = _idx(recv), _idx(send)
    N = x.shape[0] if n_nodes is None else n_nodes
    E, K = recv.shape[0], phi.shape[1]
    vx = torch.zeros_like(x) if v_x is None else _t(v_x)
    ve = torch.zeros(E, 3, dtype=_F64) if v_e is None else _t(v_e)
    vphi = torch.zeros_like(phi) if v_phi is None else _t(v_phi)
    vA = torch.zeros_like(A) if v_A is None else _t(v_A)
    Y = spherical_harmonics(problem, edge_vec)
    Yd = _sh_jvp(problem, edge_vec, ve)
    gg = dict(x=torch.zeros_like(x), phi=torch.zeros(E, K, dtype=_F64), A=torch.zeros_like(A),
              grad_out=torch.zeros(N, problem.c_out, dtype=_F64))
    Ybar_d = torch.zeros(E, problem.sh_dim, dtype=_F64)   # Ybar-dot (Eq. 31)
    Ybar_w = torch.zeros(E, problem.sh_dim, dtype=_F64)   # first-order Ybar (Eq. 22)
    for p in problem.paths:
        bi, bs, bo = problem.irreps_in[p.i_in], problem.irreps_sh[p.i_sh], problem.irreps_out[p.i_out]
        c = _coupling(p)
        sl_w = slice(p.weight_offset, p.weight_offset + p.n_weights)
        Ap, vAp = A[:, sl_w], vA[:, sl_w]
        gAp = torch.zeros_like(Ap)
        gxb = torch.zeros(x.shape[0], bi.dim, bi.mul, dtype=_F64)
        mdot = torch.zeros(N, bo.dim, bo.mul, dtype=_F64)
        for s in range(0, E, edge_chunk):
            sl = slice(s, min(E, s + edge_chunk))
            rs, ss = recv[sl], send[sl]
            Yb = Y[sl, bs.offset:bs.offset + bs.dim]
            Ydb = Yd[sl, bs.offset:bs.offset + bs.dim]
            xj = _block(x, bi)[ss]
            vxj = _block(vx, bi)[ss]
            mb = _block(gout, bo)[rs]
            T = torch.einsum("abc,eau,eb->ecu", c, xj, Yb)
            Tdot = torch.einsum("abc,eau,eb->ecu", c, xj, Ydb) + torch.einsum("abc,eau,eb->ecu", c, vxj, Yb)
            W = phi[sl] @ Ap
            Wd = vphi[sl] @ Ap + phi[sl] @ vAp
            if problem.mode == "uvu":
                h = (mb * T).sum(1)
                hd = (mb * Tdot).sum(1)
                mdot.index_add_(0, rs, Wd[:, None, :] * T + W[:, None, :] * Tdot)              # Eq. 25
                Bx = torch.einsum("abc,eb,ecu->eau", c, Yb, mb)
                Bxd = torch.einsum("abc,eb,ecu->eau", c, Ydb, mb)
                gxb.index_add_(0, ss, Wd[:, None, :] * Bx + W[:, None, :] * Bxd)               # Eq. 30
                Ybar_d[sl, bs.offset:bs.offset + bs.dim] += (
                    torch.einsum("abc,eau,ecu,eu->eb", c, xj, mb, Wd)
                    + torch.einsum("abc,eau,ecu,eu->eb", c, vxj, mb, W))                       # Eq. 31
                Ybar_w[sl, bs.offset:bs.offset + bs.dim] += torch.einsum("abc,eau,ecu,eu->eb", c, xj, mb, W)
            else:
                W = W.reshape(-1, bi.mul, bo.mul)
                Wd = Wd.reshape(-1, bi.mul, bo.mul)
                h = torch.einsum("ecw,ecu->euw", mb, T).reshape(-1, p.n_weights)
                hd = torch.einsum("ecw,ecu->euw", mb, Tdot).reshape(-1, p.n_weights)
                mdot.index_add_(0, rs, torch.einsum("euw,ecu->ecw", Wd, T) + torch.einsum("euw,ecu->ecw", W, Tdot))
                Bx = torch.einsum("abc,eb,ecw->eaw", c, Yb, mb)
                Bxd = torch.einsum("abc,eb,ecw->eaw", c, Ydb, mb)
                gxb.index_add_(0, ss, torch.einsum("euw,eaw->eau", Wd, Bx) + torch.einsum("euw,eaw->eau", W, Bxd))
                Ybar_d[sl, bs.offset:bs.offset + bs.dim] += (
                    torch.einsum("abc,eau,ecw,euw->eb", c, xj, mb, Wd)
                    + torch.einsum("abc,eau,ecw,euw->eb", c, vxj, mb, W))
                Ybar_w[sl, bs.offset:bs.offset + bs.dim] += torch.einsum("abc,eau,ecw,euw->eb", c, xj, mb, W)
            gAp += vphi[sl].T @ h + phi[sl].T @ hd                                             # Eq. 26
            gg["phi"][sl] += h @ vAp.T + hd @ Ap.T                                             # Eq. 27
        gg["A"][:, sl_w] = gAp
        gg["x"][:, bi.offset:bi.offset + bi.size] += gxb.reshape(x.shape[0], -1)
        gg["grad_out"][:, bo.offset:bo.offset + bo.size] += mdot.reshape(N, -1)
    ge = _sh_vjp(problem, edge_vec, Ybar_d) + _sh_hvp(problem, edge_vec, ve, Ybar_w)
    gpos = torch.zeros(N, 3, dtype=_F64)
    gpos.index_add_(0, send, ge)
    gpos.index_add_(0, recv, -ge)
    gg["edge_vec"] = ge
    gg["pos"] = gpos
    return gg


# --------------------------------------------------------------------------------------------
# Third-order derivative (LunaTP Appendix F, Algorithm 4), channelwise.
#
# The operands are those of the page's algorithm: node features x, the angular edge operand Y
# (E x sh_dim, the harmonics of the edge directions), the edge weights w = phi A (kept factored:
# phi per edge, A shared) and the output cotangent g.  With these the convolution is the 4-linear
# form Phi(a, b, c, d) = sum_e sum_paths sum_u c_e,u sum C a_send(e),m1,u b_e,m2 d_recv(e),m3,u.
# The first-order outputs are the gradients of Phi(x, Y, w, g); the second-order ones (directions
# v = (v_x, v_Y, v_phi, v_A)) the gradients of
#   S2 = Phi(v_x, Y, w, g) + Phi(x, v_Y, w, g) + Phi(x, Y, wv, g),   wv = v_phi A + phi v_A;
# the third-order ones (cotangents q = (q_x, q_Y, q_phi, q_A, q_g) of the second-order outputs)
# the gradients of S3 = <q, grad S2>, the derivative of S2 along q, with respect to
# x, Y, phi, A, g and the directions v.  With wq = q_phi A + phi q_A and wvq = v_phi q_A + q_phi v_A:
_TRIPLE_TERMS = (
    # (a, b, weight factors (phi-type, A-type), d)
    ("v_x", "q_Y", (("phi", "A"),), "g"),
    ("v_x", "Y", (("q_phi", "A"), ("phi", "q_A")), "g"),
    ("v_x", "Y", (("phi", "A"),), "q_g"),
    ("q_x", "v_Y", (("phi", "A"),), "g"),
    ("x", "v_Y", (("q_phi", "A"), ("phi", "q_A")), "g"),
    ("x", "v_Y", (("phi", "A"),), "q_g"),
    ("q_x", "Y", (("v_phi", "A"), ("phi", "v_A")), "g"),
    ("x", "q_Y", (("v_phi", "A"), ("phi", "v_A")), "g"),
    ("x", "Y", (("v_phi", "q_A"), ("q_phi", "v_A")), "g"),
    ("x", "Y", (("v_phi", "A"), ("phi", "v_A")), "q_g"),
)
# Outputs: the variables of S3 that are not cotangents.
TRIPLE_OUTPUTS = ("x", "Y", "phi", "A", "g", "v_x", "v_Y", "v_phi", "v_A")


def triple_backward(problem: Problem, x, Y, recv, send, phi, A, grad_out, v_x=None, v_Y=None, v_phi=None,
                    v_A=None, q_x=None, q_Y=None, q_phi=None, q_A=None, q_grad_out=None,
                    n_nodes: Optional[int] = None, outputs=None, paths=None) -> Dict[str, torch.Tensor]:
    """Gradients of S3 (above) with respect to x, Y, phi, A, g (key "grad_out") and v_x, v_Y, v_phi, v_A.

    S3 is the sum of the ten terms of _TRIPLE_TERMS.  Each term is linear in each of its four
    slots, so its gradient with respect to the variable in a slot is the form with that slot left
    open; a weight slot c = sum_k phi_k A_k passes H = dPhi/dc on as dc/dphi_k = H A_k^T and
    dc/dA_k = phi_k^T H.  Missing directions and cotangents are zero (their terms vanish).
    ``outputs`` (names) limits what is computed; ``paths`` (indices) limits the sum over paths,
    which leaves the weight-gradient columns of those paths exact (used at large sizes).
    """
    if problem.mode != "uvu":
        raise ValueError("the third-order oracle covers the channelwise mode")
    x, Y, phi, A, g = _t(x), _t(Y), _t(phi), _t(A), _t(grad_out)
    recv, send = _idx(recv), _idx(send)
    N = x.shape[0] if n_nodes is None else n_nodes
    E = recv.shape[0]
    z = dict(x=x, Y=Y, phi=phi, A=A, g=g,
             v_x=None if v_x is None else _t(v_x), v_Y=None if v_Y is None else _t(v_Y),
             v_phi=None if v_phi is None else _t(v_phi), v_A=None if v_A is None else _t(v_A),
             q_x=None if q_x is None else _t(q_x), q_Y=None if q_Y is None else _t(q_Y),
             q_phi=None if q_phi is None else _t(q_phi), q_A=None if q_A is None else _t(q_A),
             q_g=None if q_grad_out is None else _t(q_grad_out))
    shapes = dict(x=x.shape, Y=Y.shape, phi=phi.shape, A=A.shape, g=(N, problem.c_out))
    wanted = set(TRIPLE_OUTPUTS) if outputs is None else {("g" if k == "grad_out" else k) for k in outputs}
    out = {k: torch.zeros(shapes[k.replace("v_", "")], dtype=_F64) for k in TRIPLE_OUTPUTS if k in wanted}
    for a_name, b_name, factors, d_name in _TRIPLE_TERMS:
        factors = tuple(f for f in factors if z[f[0]] is not None and z[f[1]] is not None)
        if z[a_name] is None or z[b_name] is None or z[d_name] is None or not factors:
            continue
        a, b, d = z[a_name], z[b_name], z[d_name]
        for p in problem.paths:
            if paths is not None and p.index not in paths:
                continue
            bi, bs, bo = problem.irreps_in[p.i_in], problem.irreps_sh[p.i_sh], problem.irreps_out[p.i_out]
            c = _coupling(p)
            cols = slice(p.weight_offset, p.weight_offset + p.n_weights)
            ae = _block(a, bi)[send]                      # (E, d1, C)
            be = b[:, bs.offset:bs.offset + bs.dim]       # (E, d2)
            de = _block(d, bo)[recv]                      # (E, d3, C)
            w = sum(z[fp] @ z[fA][:, cols] for fp, fA in factors)   # (E, C)
            if a_name in out:        # slot a open: sum over the sender's out-edges
                ga = torch.zeros(N, bi.dim, bi.mul, dtype=_F64)
                ga.index_add_(0, send, torch.einsum("abc,eb,ecu,eu->eau", c, be, de, w))
                out[a_name][:, bi.offset:bi.offset + bi.size] += ga.reshape(N, -1)[:x.shape[0]]
            if b_name in out:        # slot b open: per edge, summed over channels
                out[b_name][:, bs.offset:bs.offset + bs.dim] += torch.einsum("abc,eau,ecu,eu->eb", c, ae, de, w)
            if d_name in out:        # slot d open: sum over the receiver's in-edges
                gd = torch.zeros(N, bo.dim, bo.mul, dtype=_F64)
                gd.index_add_(0, recv, torch.einsum("abc,eau,eb,eu->ecu", c, ae, be, w))
                out[d_name][:, bo.offset:bo.offset + bo.size] += gd.reshape(N, -1)
            if not any(f in out for fac in factors for f in fac):
                continue
            H = torch.einsum("abc,eau,eb,ecu->eu", c, ae, be, de)   # slot c open: (E, C)
            for fp, fA in factors:
                if fp in out:
                    out[fp] += H @ z[fA][:, cols].T
                if fA in out:
                    out[fA][:, cols] += z[fp].T @ H
    if "g" in out:
        out["grad_out"] = out.pop("g")
    return out
