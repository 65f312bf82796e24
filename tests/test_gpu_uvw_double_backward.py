"""Fully connected (uvw) double backward against the CPU oracle (needs an MI355X).

The library evaluates it by linearity from the first-order streamed passes (Sobek section 3.3,
Eqs. 37-39): each second-order output is a sum of passes with one operand replaced by its
direction; the oracle differentiates the backward map directly."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.oracle_helpers import make_case, make_directions
from tests.test_gpu_double_backward import KEYS, _compare, _gpu, _oracle

pytestmark = pytest.mark.gpu

RAGGED = dict(irreps_in="4x0e+3x1o+2x2e", irreps_out="3x0e+2x1o+5x2e", mode="uvw")
WIDE = dict(irreps_in="70x0e+66x1o", irreps_out="65x0e+72x1o+3x2e", mode="uvw")


@pytest.mark.parametrize("ov,dtype", [(RAGGED, "float64"), (RAGGED, "float32"), (WIDE, "float32")])
def test_uvw_double_backward_all_outputs(ov, dtype):
    case = make_case(1, irreps_override=ov, dtype=dtype)
    dirs = make_directions(case)
    _compare(_gpu(case).double_backward(dirs), _oracle(case, dirs), dtype, label=f"uvw {dtype}")


@pytest.mark.parametrize("which", [("v_x",), ("v_pos",), ("v_edge_vec",), ("v_phi",), ("v_phi", "v_A"), ("v_A",)])
def test_uvw_double_backward_partial_directions(which):
    case = make_case(1, irreps_override=RAGGED, dtype="float64")
    dirs = {k: v for k, v in make_directions(case).items() if k in which}
    _compare(_gpu(case).double_backward(dirs), _oracle(case, dirs), "float64", label=f"uvw only {'+'.join(which)}")


def test_uvw_double_backward_chunked_scratch():
    # A budget of a few receivers and senders per chunk: several receiver and sender chunks.
    case = make_case(1, irreps_override=RAGGED, dtype="float64")
    dirs = make_directions(case)
    g = _gpu(case)
    g.plan.set_scratch_budget(96 << 10)
    _compare(g.double_backward(dirs), _oracle(case, dirs), "float64", label="uvw chunked")


def test_uvw_double_backward_subset_of_outputs():
    case = make_case(1, irreps_override=RAGGED, dtype="float64")
    dirs = make_directions(case)
    g = _gpu(case)
    ref = _oracle(case, dirs)
    _compare(g.double_backward(dirs, want=("A",)), ref, "float64", keys=("A",), label="uvw A only")
    _compare(g.double_backward(dirs, want=("pos",)), ref, "float64", keys=("pos",), label="uvw pos only")
    _compare(g.double_backward(dirs, want=("phi", "x")), ref, "float64", keys=("phi", "x"), label="uvw phi+x")


def test_uvw_double_backward_repeatable_bitwise():
    case = make_case(1, irreps_override=RAGGED, dtype="float32")
    dirs = make_directions(case)
    g = _gpu(case)
    a = g.double_backward(dirs)
    b = g.double_backward(dirs)
    for k in KEYS:
        assert torch.equal(a[k], b[k]), k


def test_uvw_double_backward_config4_irreps_reduced_graph():
    """64 x (0e, 1o, 2e) -> same, SH l <= 2, 8 radial functions, fp32, 300 atoms: every output."""
    case = make_case(4, n_nodes=300)
    dirs = make_directions(case)
    _compare(_gpu(case).double_backward(dirs), _oracle(case, dirs), "float32", label="uvw config 4 reduced")


def test_uvw_double_backward_config4_full_size_sampled():
    """16,384 atoms, 859k edges: outputs of sampled nodes and their edges against the oracle on the
    subgraph of their in- and out-edges (every sampled output depends on those edges only)."""
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(4)
    dirs = make_directions(case)
    got = {k: v.cpu().numpy() for k, v in _gpu(case).double_backward(dirs).items()}
    for v in got.values():
        assert np.isfinite(v).all()
    rng = np.random.default_rng(54)
    nodes = np.unique(np.concatenate([rng.choice(case.n_nodes, 4, replace=False), [0, case.n_nodes - 1]]))
    keep = np.isin(case.send, nodes) | np.isin(case.recv, nodes)
    sub = _oracle(case, dirs, keep=keep, n_nodes=case.n_nodes)
    idx = np.nonzero(keep)[0]
    checks = {
        "x": (got["x"][nodes], sub["x"].numpy()[nodes]),
        "pos": (got["pos"][nodes], sub["pos"].numpy()[nodes]),
        "grad_out": (got["grad_out"][nodes], sub["grad_out"].numpy()[nodes]),
        "edge_vec": (got["edge_vec"][idx], sub["edge_vec"].numpy()),
        "phi": (got["phi"][idx], sub["phi"].numpy()),
    }
    for k, (a, b) in checks.items():
        err = rel_err(a, b)
        print(f"uvw config 4 sampled gg {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL["float32"], (k, err)
