"""Backward parity of the HIP path against the CPU oracle (needs an MI355X)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import conv
from tests.oracle_helpers import make_case

pytestmark = pytest.mark.gpu

SMALL_L3 = dict(irreps_in="96x0e+96x1o+96x2e", irreps_sh="1x0e+1x1o+1x2e+1x3o",
                irreps_out="96x0e+96x1o+96x2e+96x3o")
KEYS = ("x", "pos", "edge_vec", "phi", "A")


def _gpu(case):
    from tests.gpu_helpers import GpuCase
    return GpuCase(case)


def _oracle_full(case):
    return conv.backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A,
                         case.grad_out)


def _compare(got, ref, dtype, keys=KEYS, label=""):
    from tests.gpu_helpers import TOL, rel_err
    for k in keys:
        err = rel_err(got[k].cpu().numpy(), ref[k].numpy())
        print(f"{label} grad {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype], (k, err)


def test_backward_config1_full():
    case = make_case(1)
    g = _gpu(case)
    _compare(g.backward(), _oracle_full(case), "float64", label="config 1")


@pytest.mark.parametrize("dtype", ["float32", "float64"])
def test_backward_l3_ragged_channels(dtype):
    case = make_case(1, irreps_override=SMALL_L3, dtype=dtype)
    g = _gpu(case)
    _compare(g.backward(), _oracle_full(case), dtype, label=f"l3 ragged {dtype}")


@pytest.mark.parametrize("dtype", ["float32", "float64"])
def test_backward_chunked_scratch(dtype):
    # A small scratch budget splits the receivers into many chunks: chunk-local source CSR,
    # accumulated x-bar and A-bar across chunks.
    case = make_case(1, irreps_override=SMALL_L3, dtype=dtype)
    g = _gpu(case)
    g.plan.set_scratch_budget(64 << 10)
    _compare(g.backward(), _oracle_full(case), dtype, label=f"chunked {dtype}")


def test_backward_subset_of_outputs():
    case = make_case(1, irreps_override=SMALL_L3, dtype="float64")
    g = _gpu(case)
    ref = _oracle_full(case)
    _compare(g.backward(want=("A",)), ref, "float64", keys=("A",), label="A only")
    _compare(g.backward(want=("pos",)), ref, "float64", keys=("pos",), label="pos only")
    _compare(g.backward(want=("x", "phi")), ref, "float64", keys=("x", "phi"), label="x+phi")


def test_backward_repeatable_bitwise():
    case = make_case(1, irreps_override=SMALL_L3, dtype="float32")
    g = _gpu(case)
    a = g.backward()
    b = g.backward()
    for k in KEYS:
        assert torch.equal(a[k], b[k]), k


def _check_config2_sampled(case, got, label):
    """Every output of 24 sampled nodes and their edges against the oracle on those edges, and
    A-bar in full (it sums over every edge)."""
    from tests.gpu_helpers import TOL, rel_err
    for v in got.values():
        assert np.isfinite(v).all()
    rng = np.random.default_rng(22)
    nodes = np.unique(np.concatenate([rng.choice(case.n_nodes, 24, replace=False), [0, case.n_nodes - 1]]))
    keep = np.isin(case.send, nodes) | np.isin(case.recv, nodes)
    idx = np.nonzero(keep)[0]
    ev = case.edge_vec[torch.as_tensor(idx)]
    sub = conv.backward(case.problem, case.x, ev, case.recv[keep], case.send[keep], case.phi[keep], case.A,
                        case.grad_out, n_nodes=case.n_nodes)
    out_edges = np.nonzero(np.isin(case.send[keep], nodes))[0]
    checks = {
        "x": (got["x"][nodes], sub["x"].numpy()[nodes]),
        "pos": (got["pos"][nodes], sub["pos"].numpy()[nodes]),
        "edge_vec": (got["edge_vec"][idx], sub["edge_vec"].numpy()),
        "phi": (got["phi"][idx], sub["phi"].numpy()),
    }
    for k, (a, b) in checks.items():
        err = rel_err(a, b)
        print(f"{label} sampled grad {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL["float32"], (k, err)
    assert len(out_edges) > 0
    full = _oracle_full(case)
    err = rel_err(got["A"], full["A"].numpy())
    print(f"{label} grad A (full): rel err {err:.3e}", flush=True)
    assert err <= TOL["float32"]


def test_backward_config2_full_size():
    """1,024-atom diamond graph, fp32: every output of sampled nodes/edges, and A-bar in full."""
    case = make_case(2)
    g = _gpu(case)
    got = {k: v.cpu().numpy() for k, v in g.backward().items()}
    _check_config2_sampled(case, got, "config 2")


def test_backward_config2_full_size_with_kept_edge_rows():
    """The measured step at full size: the conventional forward keeping its per-edge rows, then
    the backward reading them.  The forward rows and all five gradients against the oracle
    (sampled as above), and bitwise equal to the forward and backward that derive the rows."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(2)
    g = _gpu(case)
    state = g.conv.state_buffer()
    out_k = g.conv.forward(g.x, g.pos, g.shift, g.phi, g.A, schedule=_lib.CONVENTIONAL, state=state)
    grads_k = g.conv.backward(g.x, g.pos, g.shift, g.phi, g.A, g.grad_out, state=state)
    out = g.forward()
    grads = g.backward()
    torch.cuda.synchronize()
    assert torch.equal(out, out_k)
    for k in KEYS:
        assert torch.equal(grads[k], grads_k[k]), k
    rng = np.random.default_rng(23)
    rows = np.unique(np.concatenate([rng.choice(case.n_nodes, 32, replace=False), [0, case.n_nodes - 1]]))
    keep = np.isin(case.recv, rows)
    ev = case.edge_vec[torch.as_tensor(np.nonzero(keep)[0])]
    ref = conv.forward_conventional(case.problem, case.x, ev, case.recv[keep], case.send[keep], case.phi[keep],
                                    case.A).numpy()[rows]
    err = rel_err(out_k.cpu().numpy()[rows], ref)
    print(f"config 2 kept rows forward sampled rel err {err:.3e}", flush=True)
    assert err <= TOL["float32"]
    _check_config2_sampled(case, {k: v.cpu().numpy() for k, v in grads_k.items()}, "config 2 kept rows")


def test_backward_allocates_no_device_memory():
    """After the graph upload and the kernels' first load, a backward allocates nothing on the
    device: not with one receiver chunk, and not after a smaller scratch budget splits the
    receivers into many chunks (each chunk's source-CSR bounds are computed on the device into the
    caller's workspace).  Free device memory is compared around the calls."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    case = make_case(1, irreps_override=SMALL_L3, dtype="float32")
    g = _gpu(case)
    g.graph.upload()
    g.plan.set_scratch_budget(64 << 10)       # many chunks
    ref = g.backward()                       # first calls: load the plan's kernels
    g.plan.set_scratch_budget(48 << 10)       # a different chunking from here on
    ws = g.conv.workspace(_lib.OP_BACKWARD)   # allocated by the caller beforehand
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    outs = {k: torch.empty_like(v) for k, v in ref.items()}
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    _lib.conv_backward(g.plan, g.graph, g.x, g.pos, g.shift, g.phi, g.A, g.grad_out, grad_x=outs["x"],
                       grad_pos=outs["pos"], grad_edge_vec=outs["edge_vec"], grad_phi=outs["phi"], grad_A=outs["A"],
                       workspace=ws)
    torch.cuda.synchronize()
    free2, _ = torch.cuda.mem_get_info()
    print(f"free device memory: {free0} -> {free1} (outputs) -> {free2} (chunked backward)", flush=True)
    assert free2 == free1
    _compare(outs, _oracle_full(case), "float32", label="chunked, no allocation")


def test_backward_config5_reduced_full():
    """l <= 6, 32 channels, 16 radial functions, 200 atoms: every gradient in full."""
    case = make_case(5, n_nodes=200)
    g = _gpu(case)
    _compare(g.backward(), _oracle_full(case), "float32", label="config 5 reduced")


@pytest.mark.parametrize("dtype,budget,radial", [("float64", 0, 0), ("float32", 64 << 10, 0),
                                                 ("float32", 0, 1)])
def test_backward_with_kept_edge_rows(dtype, budget, radial):
    """Channelwise forward keeping its per-edge coefficient rows and the backward reading them
    instead of deriving them again: bitwise the plain forward and backward (also with a small
    scratch budget, where the backward cuts the receivers into chunks the forward does not, and
    with the radial basis computed in the kernels), and within tolerance of the oracle."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    case = make_case(1, irreps_override=SMALL_L3, dtype=dtype)
    g = _gpu(case)
    phi = g.phi
    if radial:
        g.plan.set_radial(radial, case.raw.spec["rc"])
        phi = None
    if budget:
        g.plan.set_scratch_budget(budget)
    out = g.conv.forward(g.x, g.pos, g.shift, phi, g.A, schedule=_lib.CONVENTIONAL)
    grads = g.conv.backward(g.x, g.pos, g.shift, phi, g.A, g.grad_out)
    state = g.conv.state_buffer()
    assert state.numel() == _lib.state_size(g.plan, g.graph)
    out_k = g.conv.forward(g.x, g.pos, g.shift, phi, g.A, schedule=_lib.CONVENTIONAL, state=state)
    grads_k = g.conv.backward(g.x, g.pos, g.shift, phi, g.A, g.grad_out, state=state)
    torch.cuda.synchronize()
    print(f"kept rows {dtype} budget {budget} radial {radial}: {state.numel()} bytes", flush=True)
    assert torch.equal(out, out_k)
    for k in KEYS:
        assert torch.equal(grads[k], grads_k[k]), k
    if not radial:
        _compare(grads_k, _oracle_full(case), dtype, label=f"kept rows {dtype}")
    with pytest.raises(ValueError):   # the rows are kept by the conventional forward only
        g.conv.forward(g.x, g.pos, g.shift, phi, g.A, schedule=_lib.STREAMED, state=state)
