"""Third-order derivative (LunaTP Appendix F, Algorithm 4) of the HIP path against the oracle
(needs an MI355X).  The edge operand Y is the oracle's harmonics of the edge vectors; directions
v and cotangents q are seeded N(0, 1) draws."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import conv
from tests.oracle_helpers import make_case
from workloads import normal_tensor

pytestmark = pytest.mark.gpu

L2_16 = dict(irreps_in="16x0e+16x1o+16x2e", irreps_sh="1x0e+1x1o+1x2e", irreps_out="16x0e+16x1o+16x2e")
L3_96 = dict(irreps_in="96x0e+96x1o+96x2e", irreps_sh="1x0e+1x1o+1x2e+1x3o",
             irreps_out="96x0e+96x1o+96x2e+96x3o")
OUT_KEYS = ("x", "Y", "phi", "A", "grad_out", "v_x", "v_Y", "v_phi", "v_A")


def _inputs(case, drop=()):
    """Host inputs of the third-order call: primal (Y from the edge vectors) and seeded directions
    (streams 20-28), rounded to the case's dtype; names in `drop` are left out (zero)."""
    Y = conv.spherical_harmonics(case.problem, case.edge_vec).numpy()
    if case.dtype == "float32":
        Y = Y.astype(np.float32).astype(np.float64)
    shapes = dict(x=case.x.shape, Y=Y.shape, phi=case.phi.shape, A=case.A.shape, grad_out=case.grad_out.shape)
    h = dict(x=case.x, Y=Y, phi=case.phi, A=case.A, grad_out=case.grad_out)
    for s, name in enumerate(("v_x", "v_Y", "v_phi", "v_A", "q_x", "q_Y", "q_phi", "q_A", "q_grad_out")):
        if name in drop:
            continue
        base = name[2:]
        h[name] = normal_tensor(case.config, 20 + s, shapes[base], dtype=case.dtype)
    return h


def _oracle(case, h, edges=None, **opt):
    kw = {k: h.get(k) for k in ("v_x", "v_Y", "v_phi", "v_A", "q_x", "q_Y", "q_phi", "q_A", "q_grad_out")}
    kw.update(opt)
    if edges is None:
        return conv.triple_backward(case.problem, h["x"], h["Y"], case.recv, case.send, h["phi"], h["A"],
                                    h["grad_out"], **kw)
    for k in ("v_Y", "v_phi", "q_Y", "q_phi"):
        if kw[k] is not None:
            kw[k] = kw[k][edges]
    return conv.triple_backward(case.problem, h["x"], h["Y"][edges], case.recv[edges], case.send[edges],
                                h["phi"][edges], h["A"], h["grad_out"], n_nodes=case.n_nodes, **kw)


def _gpu_run(case, h, budget=0):
    from tests.gpu_helpers import GpuCase
    g = GpuCase(case)
    if budget:
        g.plan.set_scratch_budget(budget)
    dt = torch.float64 if case.dtype == "float64" else torch.float32
    dev = {k: torch.tensor(np.ascontiguousarray(v), dtype=dt, device="cuda") for k, v in h.items()}
    return g, g.conv.triple_backward(dev)


def _compare(got, ref, dtype, label, keys=OUT_KEYS, rows=None):
    from tests.gpu_helpers import TOL, rel_err
    for k in keys:
        a = got[k].cpu().numpy()
        b = ref[k].numpy()
        if rows is not None and k in rows:
            a, b = a[rows[k]], b[rows[k]]
        err = rel_err(a, b)
        print(f"{label} t_{k}: rel err {err:.3e}", flush=True)
        assert np.abs(b).max() > 0, k
        assert err <= TOL[dtype], (k, err)


@pytest.mark.parametrize("dtype", ["float64", "float32"])
def test_triple_backward_small(dtype):
    case = make_case(1, irreps_override=L2_16, dtype=dtype)
    h = _inputs(case)
    _, got = _gpu_run(case, h)
    _compare(got, _oracle(case, h), dtype, f"l2 16ch {dtype}")


def test_triple_backward_ragged_channels_l3():
    case = make_case(1, irreps_override=L3_96, dtype="float32")
    h = _inputs(case)
    _, got = _gpu_run(case, h)
    _compare(got, _oracle(case, h), "float32", "l3 96ch")


@pytest.mark.parametrize("drop", [("v_Y", "q_Y"), ("q_x", "q_phi", "q_A", "q_Y"), ("v_x", "v_phi", "q_grad_out")])
def test_triple_backward_missing_directions(drop):
    case = make_case(1, irreps_override=L2_16, dtype="float64")
    h = _inputs(case, drop=drop)
    _, got = _gpu_run(case, h)
    ref = _oracle(case, h)
    keys = [k for k in OUT_KEYS if np.abs(ref[k].numpy()).max() > 0]
    _compare(got, ref, "float64", f"without {drop}", keys=keys)
    for k in OUT_KEYS:
        if k not in keys:
            assert torch.count_nonzero(got[k]).item() == 0, k


@pytest.mark.parametrize("budget", [64 << 10, 1 << 20])
def test_triple_backward_chunked_scratch_and_repeatable(budget):
    """Small scratch budgets cut the receivers into chunks of different sizes (per-chunk A-bar
    slots, source bounds and forward rows)."""
    case = make_case(1, irreps_override=L2_16, dtype="float64")
    h = _inputs(case)
    _, got = _gpu_run(case, h, budget=budget)
    _compare(got, _oracle(case, h), "float64", f"chunked {budget}")
    _, again = _gpu_run(case, h, budget=budget)
    for k in OUT_KEYS:
        assert torch.equal(got[k], again[k]), k


def test_triple_backward_config2_full_size_sampled():
    """The 1,024-atom diamond graph with the l <= 3, 128-channel irreps (LunaTP case C2's), fp32:
    per-node and per-edge outputs of sampled nodes and their edges against the oracle on those
    edges, and the A-type outputs (sums over every edge) against the full oracle."""
    case = make_case(2)
    h = _inputs(case)
    _, got = _gpu_run(case, h)
    rng = np.random.default_rng(7)
    nodes = np.unique(np.concatenate([rng.choice(case.n_nodes, 8, replace=False), [0, case.n_nodes - 1]]))
    edges = np.nonzero(np.isin(case.send, nodes) | np.isin(case.recv, nodes))[0]
    sub = _oracle(case, h, edges)
    rows = {k: nodes for k in ("x", "grad_out", "v_x")}
    rows.update({k: edges for k in ("Y", "phi", "v_Y", "v_phi")})
    sub_cmp = {k: (sub[k][nodes] if k in ("x", "grad_out", "v_x") else sub[k]) for k in sub}
    got_sel = {k: (got[k][torch.as_tensor(rows[k], device="cuda")] if k in rows else got[k]) for k in got}
    _compare(got_sel, sub_cmp, "float32", "config 2 sampled", keys=("x", "Y", "phi", "grad_out", "v_x", "v_Y", "v_phi"))
    # A-type outputs sum over every edge: the columns of the first and the last path in full.
    pick = [0, len(case.problem.paths) - 1]
    full = _oracle(case, h, outputs=("A", "v_A"), paths=pick)
    cols = np.concatenate([np.arange(case.problem.paths[k].weight_offset,
                                     case.problem.paths[k].weight_offset + case.problem.paths[k].n_weights)
                           for k in pick])
    sel = {k: got[k][:, torch.as_tensor(cols, device="cuda")] for k in ("A", "v_A")}
    _compare(sel, {k: full[k][:, cols] for k in ("A", "v_A")}, "float32", f"config 2 full, paths {pick}",
             keys=("A", "v_A"))
