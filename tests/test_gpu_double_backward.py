"""Double-backward parity of the HIP path against the CPU oracle (needs an MI355X)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import conv
from tests.oracle_helpers import effective_edge_direction, make_case, make_directions

pytestmark = pytest.mark.gpu

SMALL_L3 = dict(irreps_in="96x0e+96x1o+96x2e", irreps_sh="1x0e+1x1o+1x2e+1x3o",
                irreps_out="96x0e+96x1o+96x2e+96x3o")
KEYS = ("x", "pos", "edge_vec", "phi", "A", "grad_out")


def _gpu(case):
    from tests.gpu_helpers import GpuCase
    return GpuCase(case)


def _oracle(case, dirs, keep=None, n_nodes=None):
    v_e = effective_edge_direction(case, dirs.get("v_edge_vec"), dirs.get("v_pos"))
    recv, send, phi, ev = case.recv, case.send, case.phi, case.edge_vec
    v_phi = dirs.get("v_phi")
    if keep is not None:
        idx = torch.as_tensor(np.nonzero(keep)[0])
        recv, send, phi, ev, v_e = recv[keep], send[keep], phi[keep], ev[idx], v_e[keep]
        v_phi = None if v_phi is None else v_phi[keep]
    return conv.double_backward(case.problem, case.x, ev, recv, send, phi, case.A, case.grad_out,
                                v_x=dirs.get("v_x"), v_e=v_e, v_phi=v_phi, v_A=dirs.get("v_A"),
                                n_nodes=n_nodes)


def _compare(got, ref, dtype, keys=KEYS, label=""):
    from tests.gpu_helpers import TOL, rel_err
    for k in keys:
        err = rel_err(got[k].cpu().numpy()[:len(ref[k])], ref[k].numpy())
        print(f"{label} gg {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype], (k, err)


def test_double_backward_config1_full():
    case = make_case(1)
    dirs = make_directions(case)
    _compare(_gpu(case).double_backward(dirs), _oracle(case, dirs), "float64", label="config 1")


@pytest.mark.parametrize("dtype", ["float32", "float64"])
def test_double_backward_l3_ragged_channels(dtype):
    case = make_case(1, irreps_override=SMALL_L3, dtype=dtype)
    dirs = make_directions(case)
    _compare(_gpu(case).double_backward(dirs), _oracle(case, dirs), dtype, label=f"l3 ragged {dtype}")


@pytest.mark.parametrize("mul,dtype", [(16, "float32"), (12, "float64"), (24, "float32")])
def test_double_backward_l3_narrow_blocks(mul, dtype):
    # Blocks of at most 16 (32) channels take four (two) edges per wave step, a ragged tail of
    # lanes past the block's width in each lane group.
    irreps = dict(irreps_in=f"{mul}x0e+{mul}x1o+{mul}x2e", irreps_sh="1x0e+1x1o+1x2e+1x3o",
                  irreps_out=f"{mul}x0e+{mul}x1o+{mul}x2e+{mul}x3o")
    case = make_case(1, irreps_override=irreps, dtype=dtype)
    dirs = make_directions(case)
    _compare(_gpu(case).double_backward(dirs), _oracle(case, dirs), dtype, label=f"l3 {mul}ch {dtype}")


@pytest.mark.parametrize("which", [("v_x",), ("v_pos",), ("v_edge_vec",), ("v_phi", "v_A"), ("v_A",)])
def test_double_backward_partial_directions(which):
    # Missing directions are zero.
    case = make_case(1, irreps_override=SMALL_L3, dtype="float64")
    dirs = {k: v for k, v in make_directions(case).items() if k in which}
    _compare(_gpu(case).double_backward(dirs), _oracle(case, dirs), "float64", label=f"only {'+'.join(which)}")


def test_double_backward_chunked_scratch():
    case = make_case(1, irreps_override=SMALL_L3, dtype="float64")
    dirs = make_directions(case)
    g = _gpu(case)
    g.plan.set_scratch_budget(64 << 10)
    _compare(g.double_backward(dirs), _oracle(case, dirs), "float64", label="chunked")


def test_double_backward_subset_of_outputs():
    case = make_case(1, irreps_override=SMALL_L3, dtype="float64")
    dirs = make_directions(case)
    g = _gpu(case)
    ref = _oracle(case, dirs)
    _compare(g.double_backward(dirs, want=("A",)), ref, "float64", keys=("A",), label="A only")
    _compare(g.double_backward(dirs, want=("pos",)), ref, "float64", keys=("pos",), label="pos only")
    _compare(g.double_backward(dirs, want=("grad_out", "x")), ref, "float64", keys=("grad_out", "x"),
             label="grad_out+x")


def test_double_backward_repeatable_bitwise():
    case = make_case(1, irreps_override=SMALL_L3, dtype="float32")
    dirs = make_directions(case)
    g = _gpu(case)
    a = g.double_backward(dirs)
    b = g.double_backward(dirs)
    for k in KEYS:
        assert torch.equal(a[k], b[k]), k


def test_double_backward_config5_reduced_full():
    """l <= 6, 32 channels, 16 radial functions, 200 atoms: every output in full."""
    case = make_case(5, n_nodes=200)
    dirs = make_directions(case)
    _compare(_gpu(case).double_backward(dirs), _oracle(case, dirs), "float32", label="config 5 reduced")


def test_double_backward_config5_full_size_sampled():
    """4,096 atoms, 60 neighbours: outputs of sampled nodes and their edges against the oracle on the
    subgraph of their in- and out-edges (every sampled output depends on those edges only)."""
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(5)
    dirs = make_directions(case)
    got = {k: v.cpu().numpy() for k, v in _gpu(case).double_backward(dirs).items()}
    for v in got.values():
        assert np.isfinite(v).all()
    rng = np.random.default_rng(52)
    nodes = np.unique(np.concatenate([rng.choice(case.n_nodes, 6, replace=False), [0, case.n_nodes - 1]]))
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
        print(f"config 5 sampled gg {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL["float32"], (k, err)
