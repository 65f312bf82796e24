"""Forward parity of the HIP path against the CPU oracle (needs an MI355X)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import conv
from tests.oracle_helpers import make_case

pytestmark = pytest.mark.gpu

SMALL_L3 = dict(irreps_in="96x0e+96x1o+96x2e", irreps_sh="1x0e+1x1o+1x2e+1x3o",
                irreps_out="96x0e+96x1o+96x2e+96x3o")


def _gpu(case):
    from tests.gpu_helpers import GpuCase
    return GpuCase(case)


def _sample_receivers(case, n, seed=0):
    rng = np.random.default_rng(seed)
    pick = rng.choice(case.n_nodes, size=min(n, case.n_nodes), replace=False)
    return np.unique(np.concatenate([pick, [0, case.n_nodes - 1]]))


def _oracle_rows(case, rows):
    """Oracle output rows for the receivers ``rows`` (their incoming edges only)."""
    keep = np.isin(case.recv, rows)
    ev = case.edge_vec[torch.as_tensor(np.nonzero(keep)[0])]
    m = conv.forward_conventional(case.problem, case.x, ev, case.recv[keep], case.send[keep],
                                  case.phi[keep], case.A)
    return m.numpy()[rows]


@pytest.mark.parametrize("schedule", ["conventional", "streamed"])
def test_forward_config1_full(schedule):
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(1)
    g = _gpu(case)
    assert np.array_equal(g.perm, case.perm)
    sch = _lib.CONVENTIONAL if schedule == "conventional" else _lib.STREAMED
    out = g.forward(sch).cpu().numpy()
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    err = rel_err(out, ref)
    print(f"config 1 {schedule} rel err {err:.3e}", flush=True)
    assert err <= TOL["float64"]


@pytest.mark.parametrize("dtype", ["float32", "float64"])
@pytest.mark.parametrize("schedule", ["conventional", "streamed"])
def test_forward_l3_ragged_channels(dtype, schedule):
    # 96 channels = one full 64-channel block and a ragged 32-channel tail, SH lmax 3.
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(1, irreps_override=SMALL_L3, dtype=dtype)
    g = _gpu(case)
    sch = _lib.CONVENTIONAL if schedule == "conventional" else _lib.STREAMED
    out = g.forward(sch).cpu().numpy()
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    err = rel_err(out, ref)
    print(f"l3 ragged {dtype} {schedule} rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("schedule", ["conventional", "streamed"])
@pytest.mark.parametrize("config", [2, 3])
def test_forward_full_size_sampled(config, schedule):
    """Full-size diamond graph (1,024 atoms, 91k edges), fp32 (config 2) and fp64 (config 3), both
    schedules (Sobek section 3.1, Eqs. 15-16: the streamed S_i = sum phi (x) CG, then m = S A, and
    the conventional per-edge weights): sampled receiver rows against the oracle."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(config)
    g = _gpu(case)
    assert np.array_equal(g.perm, case.perm)
    sch = _lib.CONVENTIONAL if schedule == "conventional" else _lib.STREAMED
    out = g.forward(sch).cpu().numpy()
    rows = _sample_receivers(case, 48, seed=config)
    ref = _oracle_rows(case, rows)
    err = rel_err(out[rows], ref)
    print(f"config {config} {schedule} sampled rel err {err:.3e}", flush=True)
    assert err <= TOL[case.dtype]
    assert np.isfinite(out).all()


def test_forward_repeatable_bitwise():
    case = make_case(1, irreps_override=SMALL_L3, dtype="float32")
    g = _gpu(case)
    a = g.forward().cpu().numpy()
    b = g.forward().cpu().numpy()
    assert np.array_equal(a, b)


def test_forward_isolated_receivers_and_scratch_chunks():
    # A tiny scratch budget forces many receiver chunks; nodes without in-edges give zeros.
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(1, dtype="float64")
    g = _gpu(case)
    g.plan.set_scratch_budget(4096)
    out = g.forward().cpu().numpy()
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    assert rel_err(out, ref) <= TOL["float64"]


def test_forward_empty_graph_gives_zeros():
    from clebsch_gordan_tensor_receiver_amd import _lib
    plan = _lib.Plan("8x0e+8x1o", "1x0e+1x1o", "8x0e+8x1o", "uvu", "float32", 4)
    graph = _lib.Graph(5, np.zeros(0, np.int32), np.zeros(0, np.int32))
    c = _lib.Convolution(plan, graph)
    dev = dict(dtype=torch.float32, device="cuda")
    x = torch.randn(5, plan.info["c_in"], **dev)
    pos = torch.randn(5, 3, **dev)
    phi = torch.zeros(1, 4, **dev)
    A = torch.randn(4, plan.info["n_weights"], **dev)
    out = c.forward(x, pos, None, phi, A)
    assert torch.count_nonzero(out).item() == 0


def test_forward_config5_reduced_full():
    """l <= 6, 32 channels (half-masked waves), 16 Gaussian radial functions, 200 atoms."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(5, n_nodes=200)
    g = _gpu(case)
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    for sch, name in ((_lib.CONVENTIONAL, "conventional"), (_lib.STREAMED, "streamed")):
        out = g.forward(sch).cpu().numpy()
        err = rel_err(out, ref)
        print(f"config 5 reduced {name} rel err {err:.3e}", flush=True)
        assert err <= TOL["float32"]


def test_forward_config5_full_size_sampled():
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(5)
    g = _gpu(case)
    out = g.forward().cpu().numpy()
    rows = _sample_receivers(case, 24, seed=5)
    err = rel_err(out[rows], _oracle_rows(case, rows))
    print(f"config 5 sampled rel err {err:.3e}", flush=True)
    assert err <= TOL["float32"]
