"""Degenerate inputs on the GPU: zero-length edges, empty edge lists, receivers without edges,
a single atom whose only neighbours are its own periodic images (needs an MI355X)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import conv
from oracle.irreps import make_problem
from tests.oracle_helpers import make_case

pytestmark = pytest.mark.gpu

IRREPS = dict(irreps_in="16x0e+16x1o", irreps_sh="1x0e+1x1o+1x2e", irreps_out="16x0e+16x1o+16x2e")


def _plan(dtype="float64", K=4):
    from clebsch_gordan_tensor_receiver_amd import _lib
    return _lib.Plan(IRREPS["irreps_in"], IRREPS["irreps_sh"], IRREPS["irreps_out"], "uvu", dtype, K)


def _inputs(n, recv, send, shift, K, seed, dtype=torch.float64):
    g = np.random.default_rng(seed)
    prob = make_problem(IRREPS["irreps_in"], IRREPS["irreps_sh"], IRREPS["irreps_out"], "uvu")
    d = dict(x=g.normal(size=(n, prob.c_in)), pos=g.uniform(0, 4, size=(n, 3)),
             phi=g.normal(size=(len(recv), K)), A=g.normal(size=(K, prob.n_weights)) / np.sqrt(K),
             grad_out=g.normal(size=(n, prob.c_out)), shift=np.asarray(shift, dtype=np.float64).reshape(-1, 3))
    return prob, d


def _run(plan, n, recv, send, d, want_bwd=True):
    from clebsch_gordan_tensor_receiver_amd import _lib
    graph = _lib.Graph(n, np.asarray(recv, np.int32), np.asarray(send, np.int32))
    perm = graph.perm
    conv_ = _lib.Convolution(plan, graph)
    dev = dict(dtype=torch.float64, device="cuda")
    t = {k: torch.tensor(v, **dev) for k, v in d.items() if k not in ("phi", "shift")}
    E = len(recv)
    phi = torch.tensor(d["phi"][perm] if E else np.zeros((1, d["phi"].shape[1])), **dev).contiguous()
    shift = torch.tensor(d["shift"][perm] if E else np.zeros((1, 3)), **dev).contiguous()
    out = conv_.forward(t["x"], t["pos"], shift, phi, t["A"])
    grads = conv_.backward(t["x"], t["pos"], shift, phi, t["A"], t["grad_out"]) if want_bwd else None
    return graph, perm, out, grads


def test_check_edges_clean_graph():
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import GpuCase
    case = make_case(1)
    g = GpuCase(case)
    ws = g.conv.workspace(_lib.OP_FORWARD)
    assert _lib.check_edges(g.plan, g.graph, g.pos, g.shift, ws) == -1


def test_check_edges_finds_first_zero_length_edge():
    from clebsch_gordan_tensor_receiver_amd import _lib
    n = 6
    rng = np.random.default_rng(3)
    pos = rng.uniform(0, 5, size=(n, 3))
    pos[4] = pos[1]          # atoms 1 and 4 coincide: edges 1 <- 4 and 4 <- 1 have zero length
    recv, send = zip(*[(i, j) for i in range(n) for j in range(n) if i != j])
    recv, send = np.array(recv, np.int32), np.array(send, np.int32)
    plan = _plan()
    graph = _lib.Graph(n, recv, send)
    perm = graph.perm
    vec = pos[send[perm]] - pos[recv[perm]]
    expect = int(np.nonzero((vec ** 2).sum(1) == 0.0)[0].min())
    dev = dict(dtype=torch.float64, device="cuda")
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    got = _lib.check_edges(plan, graph, torch.tensor(pos, **dev), torch.zeros((len(recv), 3), **dev), ws)
    print(f"first zero-length edge {got} (expected {expect})", flush=True)
    assert got == expect


def test_empty_edge_list():
    K = 4
    n = 5
    prob, d = _inputs(n, [], [], np.zeros((0, 3)), K, seed=4)
    graph, perm, out, grads = _run(_plan(K=K), n, [], [], d)
    assert out.shape == (n, prob.c_out) and float(out.abs().max()) == 0.0
    for k in ("x", "pos", "A"):
        assert float(grads[k].abs().max()) == 0.0, k


def test_receivers_without_edges():
    # A small random graph in which receivers 0, 5 and 9 have no incoming edges and 9 sends none.
    from tests.gpu_helpers import TOL, rel_err
    K, n = 4, 10
    rng = np.random.default_rng(5)
    pairs = [(i, j) for i in range(n) for j in range(n - 1) if i != j and i not in (0, 5, 9) and rng.random() < 0.5]
    recv = np.array([p[0] for p in pairs], np.int32)
    send = np.array([p[1] for p in pairs], np.int32)
    prob, d = _inputs(n, recv, send, np.zeros((len(recv), 3)), K, seed=6)
    graph, perm, out, grads = _run(_plan(K=K), n, recv, send, d)
    ev = conv.edge_vectors(d["pos"], d["shift"][perm], recv[perm], send[perm])
    ref = conv.forward_conventional(prob, d["x"], ev, recv[perm], send[perm], d["phi"][perm], d["A"]).numpy()
    assert rel_err(out.cpu().numpy(), ref) <= TOL["float64"]
    assert float(out[[0, 5, 9]].abs().max()) == 0.0
    b = conv.backward(prob, d["x"], ev, recv[perm], send[perm], d["phi"][perm], d["A"], d["grad_out"], n_nodes=n)
    for k in ("x", "pos", "edge_vec", "phi", "A"):
        err = rel_err(grads[k].cpu().numpy()[:len(b[k])], b[k].numpy())
        print(f"isolated receivers grad {k}: {err:.3e}", flush=True)
        assert err <= TOL["float64"], k
    assert float(grads["x"][9].abs().max()) == 0.0


def test_single_atom_periodic_images():
    # One atom in a 1.5 A periodic cube with cutoff 3 A: every edge joins the atom to one of its
    # own images, so every edge is a self-loop with a non-zero shift.
    from tests.gpu_helpers import GpuCase, TOL, rel_err
    case = make_case(1, n_nodes=1, irreps_override=IRREPS)
    assert case.n_nodes == 1 and len(case.recv) > 0 and np.all(case.recv == case.send)
    g = GpuCase(case)
    out = g.forward().cpu().numpy()
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    assert rel_err(out, ref) <= TOL["float64"]
    got = g.backward()
    b = conv.backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A, case.grad_out)
    for k in ("x", "pos", "edge_vec", "phi", "A"):
        err = rel_err(got[k].cpu().numpy(), b[k].numpy())
        print(f"single atom grad {k}: {err:.3e}", flush=True)
        # pos-bar of a lone atom is the sum of +e-bar and -e-bar over its self-loops: exactly 0
        if k == "pos":
            assert float(np.abs(got[k].cpu().numpy()).max()) <= 1e-12
        else:
            assert err <= TOL["float64"], k


UVW_IRREPS = dict(irreps_in="4x0e+3x1o+2x2e", irreps_sh="1x0e+1x1o+1x2e", irreps_out="3x0e+2x1o+5x2e")


def _dbl_inputs(mode, n, recv, send, K, seed):
    irr = IRREPS if mode == "uvu" else UVW_IRREPS
    g = np.random.default_rng(seed)
    prob = make_problem(irr["irreps_in"], irr["irreps_sh"], irr["irreps_out"], mode)
    E = len(recv)
    d = dict(x=g.normal(size=(n, prob.c_in)), pos=g.uniform(0, 4, size=(n, 3)), phi=g.normal(size=(E, K)),
             A=g.normal(size=(K, prob.n_weights)) / np.sqrt(K), grad_out=g.normal(size=(n, prob.c_out)),
             v_x=g.normal(size=(n, prob.c_in)), v_pos=g.normal(size=(n, 3)), v_edge_vec=g.normal(size=(E, 3)),
             v_phi=g.normal(size=(E, K)), v_A=g.normal(size=(K, prob.n_weights)))
    return irr, prob, d


def _dbl_run(mode, irr, n, recv, send, d, K, radial=0, rc=3.0):
    from clebsch_gordan_tensor_receiver_amd import _lib
    plan = _lib.Plan(irr["irreps_in"], irr["irreps_sh"], irr["irreps_out"], mode, "float64", K)
    if radial:
        plan.set_radial(radial, rc)
    graph = _lib.Graph(n, np.asarray(recv, np.int32), np.asarray(send, np.int32))
    perm = graph.perm
    conv_ = _lib.Convolution(plan, graph)
    dev = dict(dtype=torch.float64, device="cuda")
    E = len(recv)
    edge = lambda a, w: torch.tensor(a[perm] if E else np.zeros((1, w)), **dev).contiguous()  # noqa: E731
    t = {k: torch.tensor(d[k], **dev) for k in ("x", "pos", "A", "grad_out", "v_x", "v_pos", "v_A")}
    phi = None if radial else edge(d["phi"], K)
    v_phi = None if radial else edge(d["v_phi"], K)
    gg = conv_.double_backward(t["x"], t["pos"], torch.zeros((max(E, 1), 3), **dev), phi, t["A"], t["grad_out"],
                               v_x=t["v_x"], v_pos=t["v_pos"], v_edge_vec=edge(d["v_edge_vec"], 3), v_phi=v_phi,
                               v_A=t["v_A"])
    return perm, gg


@pytest.mark.parametrize("mode,radial", [("uvu", 0), ("uvw", 0), ("uvu", 1), ("uvw", 2)])
def test_double_backward_empty_edge_list(mode, radial):
    K, n = 4, 5
    irr, prob, d = _dbl_inputs(mode, n, [], [], K, seed=14)
    _, gg = _dbl_run(mode, irr, n, [], [], d, K, radial)
    for k in ("x", "pos", "A", "grad_out"):
        assert float(gg[k].abs().max()) == 0.0, k


@pytest.mark.parametrize("mode,radial", [("uvu", 0), ("uvw", 0), ("uvw", 1)])
def test_double_backward_receivers_without_edges(mode, radial):
    # Receivers 0, 5 and 9 have no incoming edges and 9 sends none: every output against the oracle.
    from oracle import radial as oradial
    from tests.gpu_helpers import TOL, rel_err
    K, n, rc = 4, 10, 6.0
    rng = np.random.default_rng(15)
    pairs = [(i, j) for i in range(n) for j in range(n - 1) if i != j and i not in (0, 5, 9) and rng.random() < 0.5]
    recv = np.array([p[0] for p in pairs], np.int32)
    send = np.array([p[1] for p in pairs], np.int32)
    irr, prob, d = _dbl_inputs(mode, n, recv, send, K, seed=16)
    perm, gg = _dbl_run(mode, irr, n, recv, send, d, K, radial, rc)
    r, s = recv[perm], send[perm]
    ev = conv.edge_vectors(d["pos"], np.zeros((len(r), 3)), r, s)
    v_e = d["v_edge_vec"][perm] + d["v_pos"][s] - d["v_pos"][r]
    if radial:
        ref = oradial.double_backward(radial, rc, prob, d["x"], ev, r, s, d["A"], d["grad_out"], v_x=d["v_x"],
                                      v_e=v_e, v_A=d["v_A"], n_nodes=n)
    else:
        ref = conv.double_backward(prob, d["x"], ev, r, s, d["phi"][perm], d["A"], d["grad_out"], v_x=d["v_x"],
                                   v_e=v_e, v_phi=d["v_phi"][perm], v_A=d["v_A"], n_nodes=n)
    for k in ("x", "pos", "edge_vec", "phi", "A", "grad_out"):
        err = rel_err(gg[k].cpu().numpy()[:len(ref[k])], ref[k].numpy())
        print(f"{mode} radial {radial} isolated receivers gg {k}: {err:.3e}", flush=True)
        assert err <= TOL["float64"], k
    assert float(gg["grad_out"][[0, 5, 9]].abs().max()) == 0.0


def test_triple_backward_empty_edge_list():
    from clebsch_gordan_tensor_receiver_amd import _lib
    K, n = 4, 5
    plan = _plan(K=K)
    graph = _lib.Graph(n, np.zeros(0, np.int32), np.zeros(0, np.int32))
    conv_ = _lib.Convolution(plan, graph)
    info = plan.info
    g = torch.Generator().manual_seed(17)
    dev = dict(dtype=torch.float64, device="cuda")
    r = lambda *sh: torch.randn(*sh, generator=g, dtype=torch.float64).to("cuda")  # noqa: E731
    inputs = dict(x=r(n, info["c_in"]), Y=torch.zeros((1, info["sh_dim"]), **dev), phi=torch.zeros((1, K), **dev),
                  A=r(K, info["n_weights"]), grad_out=r(n, info["c_out"]), v_x=r(n, info["c_in"]),
                  v_A=r(K, info["n_weights"]), q_x=r(n, info["c_in"]), q_grad_out=r(n, info["c_out"]))
    outs = conv_.triple_backward(inputs)
    for k, v in outs.items():
        if k in ("Y", "phi", "v_Y", "v_phi"):
            continue   # edge-sized outputs of an empty edge list hold nothing
        assert float(v.abs().max()) == 0.0, k
