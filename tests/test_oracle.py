"""Pins of the CPU oracle against facts the pages and the mathematics fix (no GPU).

Each test ties one oracle function to something other than itself: textbook
coefficients, closed forms, SciPy's spherical harmonics, tables printed on the
pages, symmetry (rotation and inversion equivariance), exact identities between
the two schedules, brute force on tiny graphs and finite differences.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import cg, conv, csr, sh
from oracle.irreps import make_problem, parse
from tests.oracle_helpers import (golden_lines, make_case, random_rotation,
                                  rotate_features, wigner_from_sh)

LMAX = 6


def _triples(lmax=LMAX):
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
                yield l1, l2, l3


# --------------------------------------------------------------------------- CG

def test_complex_cg_textbook_values():
    n = 0
    for line in golden_lines("clebsch_gordan_textbook.txt"):
        l1, m1, l2, m2, L, M, expr = line.split(maxsplit=6)
        ref = eval(expr, {"__builtins__": {}})
        got = cg.complex_cg(int(l1), int(m1), int(l2), int(m2), int(L), int(M))
        assert abs(got - ref) < 1e-15, line
        n += 1
    assert n == 15


def test_complex_cg_zero_axial_closed_form():
    # <l1 0 l2 0 | L 0> has a closed form in factorials (zero when l1 + l2 + L is odd).
    for l1, l2, L in _triples():
        s = l1 + l2 + L
        got = cg.complex_cg(l1, 0, l2, 0, L, 0)
        if s % 2:
            assert got == 0.0
            continue
        g = s // 2
        f = math.factorial
        ref = ((-1) ** (g - L) * math.sqrt(2 * L + 1) * f(g) / (f(g - l1) * f(g - l2) * f(g - L))
               * math.sqrt(f(2 * g - 2 * l1) * f(2 * g - 2 * l2) * f(2 * g - 2 * L) / f(2 * g + 1)))
        assert abs(got - ref) < 1e-14


def test_real_cg_orthonormal_columns():
    for l1, l2, l3 in _triples():
        c = cg.real_cg(l1, l2, l3).reshape(-1, 2 * l3 + 1)
        np.testing.assert_allclose(c.T @ c, np.eye(2 * l3 + 1), atol=1e-14)


def test_real_cg_scalar_identities():
    for l in range(LMAX + 1):
        np.testing.assert_allclose(cg.real_cg(0, l, l)[0], np.eye(2 * l + 1), atol=1e-15)
        np.testing.assert_allclose(cg.real_cg(l, 0, l)[:, 0, :], np.eye(2 * l + 1), atol=1e-15)


def test_real_cg_vector_products():
    # (1,1->0) is the dot product / sqrt3; (1,1->1) the cross product / sqrt2 in (y, z, x) order.
    np.testing.assert_allclose(cg.real_cg(1, 1, 0)[:, :, 0], np.eye(3) / math.sqrt(3), atol=1e-15)
    eps = np.zeros((3, 3, 3))
    for (a, b, c), s in {(0, 1, 2): 1, (1, 2, 0): 1, (2, 0, 1): 1,
                         (0, 2, 1): -1, (2, 1, 0): -1, (1, 0, 2): -1}.items():
        eps[a, b, c] = s
    np.testing.assert_allclose(cg.real_cg(1, 1, 1), eps / math.sqrt(2), atol=1e-15)
    g = np.random.default_rng(1)
    u, v = g.normal(size=3), g.normal(size=3)
    yzx = [1, 2, 0]
    cross = np.einsum("abc,a,b->c", cg.real_cg(1, 1, 1), u[yzx], v[yzx]) * math.sqrt(2)
    np.testing.assert_allclose(cross, np.cross(u, v)[yzx], atol=1e-14)


def test_real_cg_rank2_symmetric_traceless():
    c = cg.real_cg(1, 1, 2)
    for m in range(5):
        np.testing.assert_allclose(c[:, :, m], c[:, :, m].T, atol=1e-15)
        assert abs(np.trace(c[:, :, m])) < 1e-15


def test_real_cg_sign_rule():
    for l1, l2, l3 in _triples():
        flat = cg.real_cg(l1, l2, l3).reshape(-1)
        assert flat[np.nonzero(flat)[0][0]] > 0


def test_gaunt_identity_ties_cg_to_sh():
    # sum c Y_l1(n) Y_l2(n) = kappa Y_l3(n), |kappa| = sqrt((2l1+1)(2l2+1)/(2l3+1)) |<l1 0 l2 0|l3 0>|.
    n = sh.unit(torch.as_tensor(np.random.default_rng(2).normal(size=(40, 3))))
    for l1, l2, l3 in _triples():
        c = cg.real_cg(l1, l2, l3)
        lhs = np.einsum("abc,na,nb->nc", c, sh.sh_l(l1, n).numpy(), sh.sh_l(l2, n).numpy())
        k = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * l3 + 1)) * abs(cg.complex_cg(l1, 0, l2, 0, l3, 0))
        y3 = sh.sh_l(l3, n).numpy()
        if k == 0.0:
            assert np.abs(lhs).max() < 1e-12
            continue
        kappa = (lhs * y3).sum() / (y3 * y3).sum()
        assert abs(abs(kappa) - k) < 1e-12, (l1, l2, l3)
        assert np.abs(lhs - kappa * y3).max() < 1e-12


# --------------------------------------------------------------------------- SH

def test_sh_closed_forms():
    r = torch.as_tensor(np.random.default_rng(3).normal(size=(30, 3)))
    n = (r / r.norm(dim=1, keepdim=True)).numpy()
    x, y, z = n.T
    Y = sh.sh(2, r).numpy()
    np.testing.assert_allclose(Y[:, 0], 1.0, atol=1e-15)
    np.testing.assert_allclose(Y[:, 1:4], math.sqrt(3) * np.stack([y, z, x], 1), atol=1e-14)
    s15 = math.sqrt(15)
    y2 = np.stack([s15 * x * y, s15 * y * z, math.sqrt(5) / 2 * (3 * z * z - 1), s15 * x * z,
                   s15 / 2 * (x * x - y * y)], 1)
    np.testing.assert_allclose(Y[:, 4:9], y2, atol=1e-13)


def test_sh_component_norm():
    r = torch.as_tensor(np.random.default_rng(4).normal(size=(30, 3)))
    Y = sh.sh(LMAX, r).numpy()
    for l in range(LMAX + 1):
        np.testing.assert_allclose((Y[:, l * l:(l + 1) ** 2] ** 2).sum(1), 2 * l + 1, rtol=1e-13)


def test_sh_matches_scipy_through_basis_change():
    from scipy.special import sph_harm_y
    r = np.random.default_rng(5).normal(size=(30, 3))
    n = r / np.linalg.norm(r, axis=1, keepdims=True)
    theta, phi = np.arccos(n[:, 2]), np.arctan2(n[:, 1], n[:, 0])
    Y = sh.sh(LMAX, torch.as_tensor(r)).numpy()
    for l in range(LMAX + 1):
        Yc = np.stack([sph_harm_y(l, m, theta, phi) for m in range(-l, l + 1)], -1)
        Yr = math.sqrt(4 * math.pi) * Yc @ cg.complex_to_real(l).T
        assert np.abs(Yr.imag).max() < 1e-13
        np.testing.assert_allclose(Yr.real, Y[:, l * l:(l + 1) ** 2], atol=1e-12)


def test_sh_rotation_matrices_are_orthogonal():
    R = random_rotation(6)
    for l in range(LMAX + 1):
        D = wigner_from_sh(l, R)
        np.testing.assert_allclose(D @ D.T, np.eye(2 * l + 1), atol=1e-10)
    P = np.eye(3)[[1, 2, 0]]
    np.testing.assert_allclose(wigner_from_sh(1, R), P @ R @ P.T, atol=1e-12)


# --------------------------------------------------------------------------- paths

def _alt(muls):
    return "+".join(f"{m}x{l}{'e' if l % 2 == 0 else 'o'}" for l, m in enumerate(muls))


def _sh_str(lmax):
    return _alt([1] * (lmax + 1))


def test_path_counts_sobek_table1():
    n = 0
    for line in golden_lines("sobek_table1_nw.txt"):
        prof, nw, gib = line.split()
        ir = _alt([int(v) for v in prof.split("/")])
        P = make_problem(ir, _sh_str(2), ir, "uvw")
        assert P.n_weights == int(nw)
        # Sobek section 2.5: M_W = b |E| N_w bytes for the materialised edge weights.
        assert round(4 * 1.0e6 * P.n_weights / 2 ** 30, 1) == float(gib)
        n += 1
    assert n == 4


def test_path_counts_sobek_table3():
    n = 0
    for line in golden_lines("sobek_table3_nw.txt"):
        prof, nw = line.split()
        muls = [int(v) for v in prof.split("/")]
        ir = _alt(muls)
        P = make_problem(ir, _sh_str(len(muls) - 1), ir, "uvw")
        assert P.n_weights == int(nw), prof
        n += 1
    assert n == 16


def test_path_selection_lunatp_table1():
    # Count per output (l, parity) the input multiplicity of every admissible path (triangle rule and
    # sigma_out = sigma_in sigma_sh of Sobek Eq. 5); the table lists outputs of the edge irreps' kinds.
    n = 0
    for line in golden_lines("lunatp_table1_irreps.txt"):
        case, nodes, edges, outs = [t.strip() for t in line.split("|")]
        bi, bs = parse(nodes), parse(edges)
        lmax = max(b.l for b in bs)
        targets = {(b.l, b.parity) for b in bs}   # the table's outputs keep the edge (l, parity) set
        counts = {}
        for a in bi:
            for s in bs:
                for l3 in range(abs(a.l - s.l), min(a.l + s.l, lmax) + 1):
                    key = (l3, a.parity * s.parity)
                    if key not in targets:
                        continue
                    counts[key] = counts.get(key, 0) + a.mul
        got = "+".join(f"{counts[k]}x{k[0]}{'e' if k[1] > 0 else 'o'}"
                       for k in sorted(counts, key=lambda t: (t[0], -t[1])))
        assert got == outs, case
        n += 1
    assert n == 10


def test_path_selection_matches_problem_for_lunatp_c2():
    # The channelwise problem of the 1,024-atom workload (LunaTP C2 irreps) has 17 paths:
    # 3 into 0e, 5 into 1o, 5 into 2e, 4 into 3o (384/640/640/512 channels in LunaTP's table).
    P = make_problem(_alt([128] * 3), _sh_str(3), _alt([128] * 4), "uvu")
    per_out = [sum(1 for p in P.paths if p.i_out == k) for k in range(4)]
    assert per_out == [3, 5, 5, 4]
    assert P.n_weights == 17 * 128


# --------------------------------------------------------------------------- CSR

def test_csr_matches_lexsort_and_inverts():
    w = make_case(1).raw
    perm, row_ptr, col = csr.receiver_csr(w.n_nodes, w.recv, w.send, w.image)
    keys = (np.arange(len(w.recv)), w.image[:, 2], w.image[:, 1], w.image[:, 0], w.send, w.recv)
    ref = np.lexsort(keys)
    assert np.array_equal(perm, ref)
    assert np.array_equal(np.diff(row_ptr), np.bincount(w.recv, minlength=w.n_nodes))
    assert np.array_equal(col, w.send[ref])
    sp, se = csr.source_csr(w.n_nodes, col)
    sent = np.zeros(len(col), dtype=bool)
    for j in range(w.n_nodes):
        edges = se[sp[j]:sp[j + 1]]
        assert np.all(np.diff(edges) > 0)
        assert np.all(col[edges] == j)
        sent[edges] = True
    assert sent.all()


# --------------------------------------------------------------------------- conv

def _run(case, fn, **kw):
    return fn(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A, **kw)


def test_schedules_agree_fp64_config1():
    c = make_case(1)
    a = _run(c, conv.forward_conventional)
    b = _run(c, conv.forward_streamed)
    assert (a - b).abs().max().item() <= 1e-13 * a.abs().max().item()


def test_schedules_agree_fp64_uvw_small():
    c = make_case(1, irreps_override=dict(irreps_in="4x0e+3x1o+2x2e", irreps_out="3x0e+2x1o+4x2e", mode="uvw"))
    a = _run(c, conv.forward_conventional)
    b = _run(c, conv.forward_streamed)
    assert (a - b).abs().max().item() <= 1e-13 * a.abs().max().item()


@pytest.mark.parametrize("improper", [False, True])
@pytest.mark.parametrize("mode", ["uvu", "uvw"])
def test_equivariance_rotation_and_inversion(mode, improper):
    ov = dict(irreps_in="3x0e+3x1o+3x2e+3x3o", irreps_out="3x0e+3x1o+3x2e+3x3o+3x1e", mode=mode,
              irreps_sh=_sh_str(3))
    c = make_case(1, irreps_override=ov)
    R = random_rotation(11)
    Rg = -R if improper else R
    m = _run(c, conv.forward_conventional).numpy()
    ev = (c.edge_vec.numpy() @ Rg.T)
    xr = rotate_features(c.problem.irreps_in, c.x, R, improper)
    mr = conv.forward_conventional(c.problem, xr, ev, c.recv, c.send, c.phi, c.A).numpy()
    want = rotate_features(c.problem.irreps_out, m, R, improper)
    np.testing.assert_allclose(mr, want, atol=1e-9 * np.abs(m).max())


def test_linearity_and_relabelling():
    c = make_case(1)
    m = _run(c, conv.forward_conventional)
    m2 = conv.forward_conventional(c.problem, 2.0 * c.x, c.edge_vec, c.recv, c.send, c.phi, -0.5 * c.A)
    np.testing.assert_allclose(m2.numpy(), -m.numpy(), atol=1e-12)
    m3 = conv.forward_conventional(c.problem, c.x, c.edge_vec, c.recv, c.send, 3.0 * c.phi, c.A)
    np.testing.assert_allclose(m3.numpy(), 3.0 * m.numpy(), atol=1e-12)
    g = np.random.default_rng(12).permutation(c.n_nodes)   # new label of node i is g[i]
    inv = np.argsort(g)
    mp = conv.forward_conventional(c.problem, c.x[inv], c.edge_vec, g[c.recv], g[c.send], c.phi, c.A)
    np.testing.assert_allclose(mp.numpy(), m.numpy()[inv], atol=1e-12)


def test_brute_force_scalar_graph():
    # Scalars only: Y_0 = 1 and c(0,0,0) = 1, so m_i = sum_j (phi_ij A) * x_j.
    P = make_problem("2x0e", "1x0e", "2x0e", "uvu")
    pos = np.array([[0.0, 0.0, 0.0], [1.0, 0.2, 0.0], [0.1, 1.3, 0.4]])
    recv = np.array([0, 0, 1, 2]); send = np.array([1, 2, 0, 1])
    phi = np.array([[1.0, 2.0], [0.5, -1.0], [3.0, 0.0], [-2.0, 1.5]])
    A = np.array([[0.3, -0.7], [1.1, 0.4]])
    x = np.array([[1.0, 2.0], [-1.0, 0.5], [0.25, -3.0]])
    ev = conv.edge_vectors(pos, np.zeros((4, 3)), recv, send)
    m = conv.forward_conventional(P, x, ev, recv, send, phi, A).numpy()
    want = np.zeros((3, 2))
    for e in range(4):
        for u in range(2):
            want[recv[e], u] += (phi[e] @ A[:, u]) * x[send[e], u]
    np.testing.assert_allclose(m, want, atol=1e-15)


def test_brute_force_vector_graph_fixes_argument_order():
    """Degree-1 couplings written out by hand on a 3-node graph: the scalar-vector products,
    the dot product (1,1 -> 0) = (x . Y_1) / sqrt(3) and the cross product
    (1,1 -> 1) = (x cross Y_1) / sqrt(2), with x the sender's vector and Y_1 = sqrt(3) (y, z, x) / r
    both in (y, z, x) component order (a cyclic reordering, so np.cross on them is the cross
    product in the same order).  x cross Y and Y cross x differ in sign: this pins which operand
    of the coupling is the feature and which the harmonic."""
    P = make_problem("1x0e+1x1o", "1x0e+1x1o", "1x0e+1x1o+1x1e", "uvu")
    # Paths in enumeration order: (0e,0e->0e), (0e,1o->1o), (1o,0e->1o), (1o,1o->0e), (1o,1o->1e).
    got = [(p.l1, p.l2, p.l3) for p in P.paths]
    assert got == [(0, 0, 0), (0, 1, 1), (1, 0, 1), (1, 1, 0), (1, 1, 1)]
    pos = np.array([[0.0, 0.0, 0.0], [1.0, 0.2, -0.3], [0.1, 1.3, 0.4]])
    recv = np.array([0, 0, 1, 2, 2]); send = np.array([1, 2, 0, 0, 1])
    shift = np.zeros((5, 3)); shift[4] = [0.0, 0.5, -2.0]
    rng = np.random.default_rng(3)
    K = 3
    phi = rng.normal(size=(5, K)); A = rng.normal(size=(K, P.n_weights)); x = rng.normal(size=(3, 4))
    ev = conv.edge_vectors(pos, shift, recv, send).numpy()
    m = conv.forward_conventional(P, x, ev, recv, send, phi, A).numpy()
    want = np.zeros((3, 7))           # out row: [0e | 1o (y,z,x) | 1e (y,z,x)]
    for e in range(5):
        w = phi[e] @ A                # one weight per path (one channel)
        r = ev[e]
        y1 = np.sqrt(3.0) * np.array([r[1], r[2], r[0]]) / np.linalg.norm(r)
        s, v = x[send[e], 0], x[send[e], 1:4]
        want[recv[e], 0] += w[0] * s + w[3] * (v @ y1) / np.sqrt(3.0)
        want[recv[e], 1:4] += w[1] * s * y1 + w[2] * v
        want[recv[e], 4:7] += w[4] * np.cross(v, y1) / np.sqrt(2.0)
    np.testing.assert_allclose(m, want, atol=1e-13)


def test_backward_matches_finite_differences():
    ov = dict(irreps_in="2x0e+2x1o+2x2e", irreps_out="2x0e+2x1o+2x2e", irreps_sh=_sh_str(2))
    for mode in ("uvu", "uvw"):
        ov["mode"] = mode
        c = make_case(1, irreps_override=ov, n_nodes=12)
        g = c.grad_out
        b = conv.backward(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.A, g)

        def L(x=c.x, pos=c.pos, phi=c.phi, A=c.A):
            ev = conv.edge_vectors(pos, c.shift, c.recv, c.send)
            return float((conv.forward_conventional(c.problem, x, ev, c.recv, c.send, phi, A) * torch.as_tensor(g)).sum())

        rng = np.random.default_rng(13)
        h = 1e-6
        for name, arr in (("x", c.x), ("pos", c.pos), ("phi", c.phi), ("A", c.A)):
            for _ in range(4):
                idx = tuple(int(rng.integers(s)) for s in arr.shape)
                ap, am = arr.copy(), arr.copy()
                ap[idx] += h
                am[idx] -= h
                fd = (L(**{name: ap}) - L(**{name: am})) / (2 * h)
                got = float(b[name][idx])
                assert abs(fd - got) <= 1e-6 * max(1.0, abs(got)), (mode, name, idx, fd, got)


def test_backward_matches_autograd_config1():
    c = make_case(1)
    pos = torch.tensor(c.pos, requires_grad=True)
    x = torch.tensor(c.x, requires_grad=True)
    phi = torch.tensor(c.phi, requires_grad=True)
    A = torch.tensor(c.A, requires_grad=True)
    ev = conv.edge_vectors(pos, c.shift, c.recv, c.send)
    m = conv.forward_conventional(c.problem, x, ev, c.recv, c.send, phi, A)
    (m * torch.as_tensor(c.grad_out)).sum().backward()
    b = conv.backward(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.A, c.grad_out)
    for k, ref in (("x", x.grad), ("pos", pos.grad), ("phi", phi.grad), ("A", A.grad)):
        np.testing.assert_allclose(b[k].numpy(), ref.numpy(), atol=1e-12 * ref.abs().max().item())


def test_sh_gradient_complex_step():
    # J_Y^T v from autograd against complex-step derivatives of the analytic polynomial form.
    r = np.random.default_rng(14).normal(size=(5, 3))
    v = np.random.default_rng(15).normal(size=(5, (LMAX + 1) ** 2))
    P = make_problem("1x0e", _sh_str(LMAX), "1x0e", "uvu")
    got = conv._sh_vjp(P, r, torch.as_tensor(v)).numpy()
    h = 1e-30
    for d in range(3):
        rc = r.astype(np.complex128)
        rc[:, d] += 1j * h
        dY = sh.sh(LMAX, torch.as_tensor(rc)).numpy().imag / h
        np.testing.assert_allclose((dY * v).sum(1), got[:, d], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["uvu", "uvw"])
def test_grad_A_streamed_equals_edge_form(mode):
    # Sobek Eq. 36 (A-bar = S^T mbar) and Eq. 19 (A-bar = sum_e phi h) agree.
    ov = dict(irreps_in="3x0e+2x1o+2x2e", irreps_out="3x0e+2x1o+2x2e", mode=mode)
    if mode == "uvw":
        ov["irreps_out"] = "2x0e+3x1o+1x2e"
    c = make_case(1, irreps_override=ov)
    a = conv.backward(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.A, c.grad_out)["A"]
    b = conv.grad_A_streamed(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.grad_out)
    assert (a - b).abs().max().item() <= 1e-12 * a.abs().max().item()


def _dbl_case(mode, n_nodes=10):
    ov = dict(irreps_in="2x0e+2x1o+2x2e", irreps_out="2x0e+2x1o+2x2e", irreps_sh=_sh_str(2), mode=mode)
    c = make_case(1, irreps_override=ov, n_nodes=n_nodes)
    g = np.random.default_rng(31)
    v = dict(v_x=g.normal(size=c.x.shape), v_e=g.normal(size=(len(c.recv), 3)), v_phi=g.normal(size=c.phi.shape),
             v_A=g.normal(size=c.A.shape))
    return c, v


@pytest.mark.parametrize("mode", ["uvu", "uvw"])
def test_double_backward_matches_autograd(mode):
    # Independent route: torch autograd of the oracle forward, differentiated twice.
    c, v = _dbl_case(mode)
    x = torch.tensor(c.x, requires_grad=True)
    pos = torch.tensor(c.pos, requires_grad=True)
    phi = torch.tensor(c.phi, requires_grad=True)
    A = torch.tensor(c.A, requires_grad=True)
    mbar = torch.tensor(c.grad_out, requires_grad=True)
    ev = conv.edge_vectors(pos, c.shift, c.recv, c.send)
    m = conv.forward_conventional(c.problem, x, ev, c.recv, c.send, phi, A)
    gx, gev, gphi, gA = torch.autograd.grad((m * mbar).sum(), (x, ev, phi, A), create_graph=True)
    s = ((gx * torch.as_tensor(v["v_x"])).sum() + (gev * torch.as_tensor(v["v_e"])).sum()
         + (gphi * torch.as_tensor(v["v_phi"])).sum() + (gA * torch.as_tensor(v["v_A"])).sum())
    rx, rpos, rphi, rA, rm = torch.autograd.grad(s, (x, pos, phi, A, mbar))
    got = conv.double_backward(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.A, c.grad_out, **v)
    for k, ref in (("x", rx), ("pos", rpos), ("phi", rphi), ("A", rA), ("grad_out", rm)):
        np.testing.assert_allclose(got[k].numpy(), ref.numpy(), atol=1e-11 * max(1.0, ref.abs().max().item()))


def test_double_backward_matches_finite_differences_of_backward():
    # <gg_theta, d> = d/dt <v, B(theta + t d)> at t = 0, by central differences of the oracle backward.
    c, v = _dbl_case("uvu")
    gg = conv.double_backward(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.A, c.grad_out, **v)
    rng = np.random.default_rng(32)
    d = dict(x=rng.normal(size=c.x.shape), pos=rng.normal(size=c.pos.shape), phi=rng.normal(size=c.phi.shape),
             A=rng.normal(size=c.A.shape), mbar=rng.normal(size=c.grad_out.shape))

    def pairing(t):
        x = c.x + t * d["x"]
        pos = c.pos + t * d["pos"]
        phi = c.phi + t * d["phi"]
        A = c.A + t * d["A"]
        mb = c.grad_out + t * d["mbar"]
        ev = conv.edge_vectors(pos, c.shift, c.recv, c.send)
        b = conv.backward(c.problem, x, ev, c.recv, c.send, phi, A, mb)
        return float((b["x"].numpy() * v["v_x"]).sum() + (b["edge_vec"].numpy() * v["v_e"]).sum()
                     + (b["phi"].numpy() * v["v_phi"]).sum() + (b["A"].numpy() * v["v_A"]).sum())

    h = 1e-5
    fd = (pairing(h) - pairing(-h)) / (2 * h)
    an = float((gg["x"].numpy() * d["x"]).sum() + (gg["pos"].numpy() * d["pos"]).sum()
               + (gg["phi"].numpy() * d["phi"]).sum() + (gg["A"].numpy() * d["A"]).sum()
               + (gg["grad_out"].numpy() * d["mbar"]).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


def test_double_backward_second_order_symmetry():
    # With mbar fixed, gg_theta = H v for the Hessian H of L = <mbar, m>: <H v1, v2> = <H v2, v1>.
    c, v1 = _dbl_case("uvu")
    rng = np.random.default_rng(33)
    v2 = dict(v_x=rng.normal(size=c.x.shape), v_e=rng.normal(size=(len(c.recv), 3)),
              v_phi=rng.normal(size=c.phi.shape), v_A=rng.normal(size=c.A.shape))
    g1 = conv.double_backward(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.A, c.grad_out, **v1)
    g2 = conv.double_backward(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.A, c.grad_out, **v2)

    def pair(g, v):
        return float((g["x"].numpy() * v["v_x"]).sum() + (g["edge_vec"].numpy() * v["v_e"]).sum()
                     + (g["phi"].numpy() * v["v_phi"]).sum() + (g["A"].numpy() * v["v_A"]).sum())

    a, b = pair(g1, v2), pair(g2, v1)
    assert abs(a - b) <= 1e-10 * max(1.0, abs(a))


# ---------------------------------------------------------------- fused radial basis (oracle)

def test_envelope_is_smooth_at_the_cutoff():
    from oracle import radial
    d = torch.tensor([0.0, 1.0 - 1e-300], dtype=torch.float64, requires_grad=True)
    u = (1.0 - 28.0 * d ** 6 + 48.0 * d ** 7 - 21.0 * d ** 8)
    assert abs(float(radial.envelope(torch.tensor([0.0], dtype=torch.float64))[0]) - 1.0) == 0.0
    assert float(radial.envelope(torch.tensor([1.0, 1.5], dtype=torch.float64)).abs().max()) == 0.0
    g1, = torch.autograd.grad(u.sum(), d, create_graph=True)
    g2, = torch.autograd.grad(g1.sum(), d)
    # u(1) = u'(1) = u''(1) = 0: the basis and its first two derivatives vanish at r_c.
    assert abs(float(u[1].detach())) < 1e-12 and abs(float(g1[1].detach())) < 1e-9 and abs(float(g2[1])) < 1e-8
    assert abs(float(g1[0].detach())) == 0.0


def test_bessel_basis_is_orthonormal_without_envelope():
    # sqrt(2/r_c) sin(n pi r / r_c) / r are orthonormal under r^2 dr on [0, r_c].
    from oracle import radial
    rc, K = 5.0, 8
    xg, wg = np.polynomial.legendre.leggauss(400)
    r = torch.tensor(0.5 * rc * (xg + 1.0))
    w = torch.tensor(0.5 * rc * wg)
    B = radial.basis(radial.BESSEL, r, rc, K, envelope_on=False)
    gram = (B * (w * r ** 2)[:, None]).T @ B
    assert float((gram - torch.eye(K, dtype=torch.float64)).abs().max()) < 1e-12


def test_gaussian_basis_peak_and_width():
    from oracle import radial
    rc, K = 6.0, 16
    D = rc / (K - 1)
    mu = torch.arange(K, dtype=torch.float64) * D
    at_mu = radial.basis(radial.GAUSSIAN, mu, rc, K)
    assert float((torch.diagonal(at_mu) - 1.0).abs().max()) == 0.0
    off = radial.basis(radial.GAUSSIAN, mu[3:4] + D, rc, K)
    assert abs(float(off[0, 3]) - math.exp(-0.5)) < 1e-15


@pytest.mark.parametrize("kind", [1, 2])
def test_radial_derivative_complex_step(kind):
    from oracle import radial
    rc, K = 5.0, 8
    r = torch.tensor([0.7, 1.9, 3.3, 4.6, 4.99], dtype=torch.float64)
    h = 1e-30
    cs = radial.basis(kind, r.to(torch.complex128) + 1j * h, rc, K).imag / h
    d = radial.basis_derivative(kind, r, rc, K)
    assert float((cs - d).abs().max()) <= 1e-12 * max(1.0, float(d.abs().max()))


@pytest.mark.parametrize("kind", [1, 2])
def test_position_gradient_through_the_radial_basis(kind):
    # Finite differences of <grad_out, m(pos)> with phi computed from |r|: the oracle backward
    # (through Y) plus the radial term (sum_q phi-bar_q dphi_q/dr) r-hat, mapped to positions.
    from oracle import radial
    ov = dict(irreps_in="2x0e+2x1o+2x2e", irreps_out="2x0e+2x1o+2x2e", irreps_sh=_sh_str(2), mode="uvu")
    c = make_case(1, irreps_override=ov, n_nodes=12)
    rc, K = 3.0, c.phi.shape[1]

    def L(pos):
        ev = conv.edge_vectors(pos, c.shift, c.recv, c.send)
        phi = radial.basis(kind, radial.edge_lengths(ev), rc, K)
        return float((conv.forward_conventional(c.problem, c.x, ev, c.recv, c.send, phi, c.A)
                      * torch.as_tensor(c.grad_out)).sum())

    ev = c.edge_vec
    phi = radial.basis(kind, radial.edge_lengths(ev), rc, K)
    b = conv.backward(c.problem, c.x, ev, c.recv, c.send, phi, c.A, c.grad_out, n_nodes=c.n_nodes)
    ge = b["edge_vec"] + radial.edge_vec_grad(kind, ev, rc, b["phi"])
    gpos = torch.zeros(c.n_nodes, 3, dtype=torch.float64)
    gpos.index_add_(0, torch.as_tensor(c.send, dtype=torch.long), ge)
    gpos.index_add_(0, torch.as_tensor(c.recv, dtype=torch.long), -ge)
    rng = np.random.default_rng(21)
    h = 1e-6
    for _ in range(6):
        idx = (int(rng.integers(c.n_nodes)), int(rng.integers(3)))
        pp, pm = c.pos.copy(), c.pos.copy()
        pp[idx] += h
        pm[idx] -= h
        fd = (L(pp) - L(pm)) / (2 * h)
        got = float(gpos[idx])
        assert abs(fd - got) <= 1e-6 * max(1.0, abs(got)), (kind, idx, fd, got)


@pytest.mark.parametrize("kind", [1, 2])
def test_radial_second_derivative_complex_step(kind):
    from oracle import radial
    rc, K = 5.0, 8
    r = torch.tensor([0.7, 1.9, 3.3, 4.6, 4.99], dtype=torch.float64)
    h = 1e-30
    # Complex step of the first derivative written with complex-safe operations (the oracle's
    # basis_derivative clips at the cutoff with torch.where on real inputs only).
    def dphi(z):
        if kind == radial.BESSEL:
            n = torch.arange(1, K + 1, dtype=torch.float64)
            a = n[None, :] * (math.pi / rc)
            zz = z[:, None]
            s, c = torch.sin(a * zz), torch.cos(a * zz)
            b = math.sqrt(2.0 / rc) * s / zz
            db = math.sqrt(2.0 / rc) * (a * c * zz - s) / zz ** 2
            d = z / rc
            u = 1.0 - 28.0 * d ** 6 + 48.0 * d ** 7 - 21.0 * d ** 8
            du = (-168.0 * d ** 5 + 336.0 * d ** 6 - 168.0 * d ** 7) / rc
            return db * u[:, None] + b * du[:, None]
        D = rc / (K - 1)
        diff = z[:, None] - torch.arange(K, dtype=torch.float64) * D
        return -diff / (D * D) * torch.exp(-(diff ** 2) / (2.0 * D * D))
    assert float((dphi(r.to(torch.complex128)).real - radial.basis_derivative(kind, r, rc, K)).abs().max()) < 1e-13
    cs = dphi(r.to(torch.complex128) + 1j * h).imag / h
    d2 = radial.basis_second_derivative(kind, r, rc, K)
    assert float((cs - d2).abs().max()) <= 1e-12 * max(1.0, float(d2.abs().max()))
    # Beyond the cutoff the Bessel basis and its derivatives are zero.
    if kind == radial.BESSEL:
        assert float(radial.basis_second_derivative(kind, torch.tensor([5.0, 6.0]), rc, K).abs().max()) == 0.0


def _radial_dbl_case(kind, mode="uvu"):
    ov = dict(irreps_in="2x0e+2x1o+2x2e", irreps_out="2x0e+2x1o+2x2e", irreps_sh=_sh_str(2), mode=mode)
    c = make_case(1, irreps_override=ov, n_nodes=10)
    g = np.random.default_rng(61 + kind)
    v = dict(v_x=g.normal(size=c.x.shape), v_e=g.normal(size=(len(c.recv), 3)), v_A=g.normal(size=c.A.shape))
    return c, v, 3.0


@pytest.mark.parametrize("kind,mode", [(1, "uvu"), (2, "uvu"), (1, "uvw"), (2, "uvw")])
def test_radial_double_backward_matches_autograd(kind, mode):
    # Independent route: torch autograd of the forward with phi = basis(|r|), taken twice.
    from oracle import radial
    c, v, rc = _radial_dbl_case(kind, mode)
    K = c.phi.shape[1]
    x = torch.tensor(c.x, requires_grad=True)
    pos = torch.tensor(c.pos, requires_grad=True)
    A = torch.tensor(c.A, requires_grad=True)
    mbar = torch.tensor(c.grad_out, requires_grad=True)
    ev = conv.edge_vectors(pos, c.shift, c.recv, c.send)
    phi = radial.basis(kind, torch.sqrt((ev ** 2).sum(1)), rc, K)
    m = conv.forward_conventional(c.problem, x, ev, c.recv, c.send, phi, A)
    gx, gev, gA = torch.autograd.grad((m * mbar).sum(), (x, ev, A), create_graph=True)
    s = ((gx * torch.as_tensor(v["v_x"])).sum() + (gev * torch.as_tensor(v["v_e"])).sum()
         + (gA * torch.as_tensor(v["v_A"])).sum())
    rx, rpos, rA, rm = torch.autograd.grad(s, (x, pos, A, mbar))
    got = radial.double_backward(kind, rc, c.problem, c.x, c.edge_vec, c.recv, c.send, c.A, c.grad_out, **v,
                                 n_nodes=c.n_nodes)
    for k, ref in (("x", rx), ("pos", rpos), ("A", rA), ("grad_out", rm)):
        np.testing.assert_allclose(got[k].numpy(), ref.numpy(), atol=1e-11 * max(1.0, ref.abs().max().item()))


@pytest.mark.parametrize("kind", [1, 2])
def test_radial_double_backward_matches_finite_differences(kind):
    # <gg_theta, d> = d/dt <v, B(theta + t d)> with the first-order radial backward B (e-bar
    # through Y plus the radial term), by central differences.
    from oracle import radial
    c, v, rc = _radial_dbl_case(kind)
    K = c.phi.shape[1]
    gg = radial.double_backward(kind, rc, c.problem, c.x, c.edge_vec, c.recv, c.send, c.A, c.grad_out, **v,
                                n_nodes=c.n_nodes)
    rng = np.random.default_rng(62)
    d = dict(x=rng.normal(size=c.x.shape), pos=rng.normal(size=c.pos.shape), A=rng.normal(size=c.A.shape),
             mbar=rng.normal(size=c.grad_out.shape))

    def pairing(t):
        x, pos, A, mb = (c.x + t * d["x"], c.pos + t * d["pos"], c.A + t * d["A"], c.grad_out + t * d["mbar"])
        ev = conv.edge_vectors(pos, c.shift, c.recv, c.send)
        phi = radial.basis(kind, radial.edge_lengths(ev), rc, K)
        b = conv.backward(c.problem, x, ev, c.recv, c.send, phi, A, mb, n_nodes=c.n_nodes)
        ge = b["edge_vec"] + radial.edge_vec_grad(kind, ev, rc, b["phi"])
        return float((b["x"].numpy() * v["v_x"]).sum() + (ge.numpy() * v["v_e"]).sum()
                     + (b["A"].numpy() * v["v_A"]).sum())

    h = 1e-5
    fd = (pairing(h) - pairing(-h)) / (2 * h)
    an = float((gg["x"].numpy() * d["x"]).sum() + (gg["pos"].numpy() * d["pos"]).sum()
               + (gg["A"].numpy() * d["A"]).sum() + (gg["grad_out"].numpy() * d["mbar"]).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


# ------------------------------------------------------------------ third-order derivative

def _triple_case(n_nodes=10, seed=41, with_y_dirs=True):
    """A small channelwise problem with every operand of the third-order derivative: the edge
    operand Y is the harmonics of the edge vectors; directions and cotangents are N(0, 1)."""
    ov = dict(irreps_in="2x0e+2x1o+2x2e", irreps_out="2x0e+2x1o+2x2e", irreps_sh=_sh_str(2))
    c = make_case(1, irreps_override=ov, n_nodes=n_nodes)
    Y = conv.spherical_harmonics(c.problem, c.edge_vec).numpy()
    rng = np.random.default_rng(seed)
    nrm = lambda shape: rng.normal(size=shape)  # noqa: E731
    d = dict(v_x=nrm(c.x.shape), v_Y=nrm(Y.shape) if with_y_dirs else None, v_phi=nrm(c.phi.shape),
             v_A=nrm(c.A.shape), q_x=nrm(c.x.shape), q_Y=nrm(Y.shape) if with_y_dirs else None,
             q_phi=nrm(c.phi.shape), q_A=nrm(c.A.shape), q_grad_out=nrm(c.grad_out.shape))
    return c, Y, d


def test_triple_backward_matches_third_order_autograd():
    """The explicit third-order formulas against autograd taken three times over the oracle
    forward with the edge operand given: f = <g, m(x, Y, phi, A)>, S2 = <v, grad f>,
    S3 = <q, grad S2>, T = grad S3 (LunaTP Appendix F, Algorithms 2-4 in that nesting)."""
    c, Y, d = _triple_case()
    leaf = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64, requires_grad=True)  # noqa: E731
    x, Yt, phi, A, g = leaf(c.x), leaf(Y), leaf(c.phi), leaf(c.A), leaf(c.grad_out)
    vx, vY, vphi, vA = leaf(d["v_x"]), leaf(d["v_Y"]), leaf(d["v_phi"]), leaf(d["v_A"])
    f = (conv.forward_from_sh(c.problem, x, Yt, c.recv, c.send, phi, A) * g).sum()
    gx, gY, gphi, gA = torch.autograd.grad(f, (x, Yt, phi, A), create_graph=True)
    S2 = (vx * gx).sum() + (vY * gY).sum() + (vphi * gphi).sum() + (vA * gA).sum()
    D = torch.autograd.grad(S2, (x, Yt, phi, A, g), create_graph=True)
    qs = [torch.as_tensor(d[k]) for k in ("q_x", "q_Y", "q_phi", "q_A", "q_grad_out")]
    S3 = sum((q * Dk).sum() for q, Dk in zip(qs, D))
    want = torch.autograd.grad(S3, (x, Yt, phi, A, g, vx, vY, vphi, vA))
    got = conv.triple_backward(c.problem, c.x, Y, c.recv, c.send, c.phi, c.A, c.grad_out, **d)
    for k, w in zip(("x", "Y", "phi", "A", "grad_out", "v_x", "v_Y", "v_phi", "v_A"), want):
        ref = w.detach().numpy()
        err = np.abs(got[k].numpy() - ref).max() / np.abs(ref).max()
        assert np.abs(ref).max() > 0, k
        assert err < 1e-12, (k, err)


def test_triple_backward_finite_differences_of_double_backward():
    """With the edge operand held fixed (no Y directions), S3 = <q, second-order outputs> is
    computed by the position-level double backward (its edge-vector direction zero); central
    differences of S3 in x, phi, A, g and the directions pin the third-order outputs."""
    c, Y, d = _triple_case(with_y_dirs=False)

    def S3(x=c.x, phi=c.phi, A=c.A, g=c.grad_out, v_x=d["v_x"], v_phi=d["v_phi"], v_A=d["v_A"]):
        dd = conv.double_backward(c.problem, x, c.edge_vec, c.recv, c.send, phi, A, g, v_x=v_x, v_phi=v_phi, v_A=v_A)
        return float((torch.as_tensor(d["q_x"]) * dd["x"]).sum() + (torch.as_tensor(d["q_phi"]) * dd["phi"]).sum()
                     + (torch.as_tensor(d["q_A"]) * dd["A"]).sum()
                     + (torch.as_tensor(d["q_grad_out"]) * dd["grad_out"]).sum())

    got = conv.triple_backward(c.problem, c.x, Y, c.recv, c.send, c.phi, c.A, c.grad_out, **d)
    rng = np.random.default_rng(43)
    base = dict(x=c.x, phi=c.phi, A=c.A, g=c.grad_out, v_x=d["v_x"], v_phi=d["v_phi"], v_A=d["v_A"])
    keys = dict(x="x", phi="phi", A="A", g="grad_out", v_x="v_x", v_phi="v_phi", v_A="v_A")
    h = 1e-3
    for k, out_key in keys.items():
        delta = rng.normal(size=np.shape(base[k]))
        plus = dict(base, **{k: base[k] + h * delta})
        minus = dict(base, **{k: base[k] - h * delta})
        fd = (S3(**plus) - S3(**minus)) / (2 * h)
        an = float((got[out_key].numpy() * delta).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (k, fd, an)


def test_triple_backward_direction_gradients_are_second_order_outputs():
    """Symmetry of mixed partials: the gradients with respect to the directions v equal the
    second-order outputs along the cotangents q plus the first-order outputs for the output
    cotangent q_g (edge operand fixed: no Y directions)."""
    c, Y, d = _triple_case(with_y_dirs=False)
    got = conv.triple_backward(c.problem, c.x, Y, c.recv, c.send, c.phi, c.A, c.grad_out, **d)
    dd = conv.double_backward(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.A, c.grad_out,
                              v_x=d["q_x"], v_phi=d["q_phi"], v_A=d["q_A"])
    b = conv.backward(c.problem, c.x, c.edge_vec, c.recv, c.send, c.phi, c.A, d["q_grad_out"])
    for k in ("x", "phi", "A"):
        ref = (dd[k] + b[k]).numpy()
        err = np.abs(got["v_" + k].numpy() - ref).max() / np.abs(ref).max()
        assert err < 1e-12, (k, err)
