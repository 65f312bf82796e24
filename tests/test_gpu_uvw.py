"""Fully connected (uvw) streamed convolution: parity of the HIP path with the oracle (MI355X)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import conv
from tests.oracle_helpers import make_case

pytestmark = pytest.mark.gpu

KEYS = ("x", "pos", "edge_vec", "phi", "A")
RAGGED = dict(irreps_in="4x0e+3x1o+2x2e", irreps_out="3x0e+2x1o+5x2e", mode="uvw")
CFG4_SMALL = 512


def _gpu(case):
    from tests.gpu_helpers import GpuCase
    return GpuCase(case)


def _compare(got, ref, dtype, keys=KEYS, label=""):
    from tests.gpu_helpers import TOL, rel_err
    for k in keys:
        err = rel_err(got[k].cpu().numpy(), ref[k].numpy())
        print(f"{label} grad {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype], (k, err)


@pytest.mark.parametrize("dtype", ["float64", "float32"])
def test_uvw_ragged_forward_backward(dtype):
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(1, irreps_override=RAGGED, dtype=dtype)
    g = _gpu(case)
    out = g.forward(_lib.STREAMED).cpu().numpy()
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    err = rel_err(out, ref)
    print(f"uvw ragged {dtype} forward rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]
    ref_b = conv.backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A,
                          case.grad_out)
    _compare(g.backward(), ref_b, dtype, label=f"uvw ragged {dtype}")


def test_uvw_conventional_is_refused():
    from clebsch_gordan_tensor_receiver_amd import _lib
    case = make_case(1, irreps_override=RAGGED, dtype="float32")
    g = _gpu(case)
    with pytest.raises(_lib.CgtpError) as ei:
        g.forward(_lib.CONVENTIONAL)
    assert ei.value.status == 2


def test_uvw_chunked_scratch():
    # A small scratch budget forces many receiver and sender chunks.
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(1, irreps_override=RAGGED, dtype="float64")
    g = _gpu(case)
    g.plan.set_scratch_budget(64 << 10)
    out = g.forward(_lib.STREAMED).cpu().numpy()
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    assert rel_err(out, ref) <= TOL["float64"]
    ref_b = conv.backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A,
                          case.grad_out)
    _compare(g.backward(), ref_b, "float64", label="uvw chunked")


def test_uvw_config4_irreps_reduced_graph():
    """64x(0e,1o,2e) fully connected, SH lmax 2, on a 512-atom box at the same density (fp32)."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(4, n_nodes=CFG4_SMALL)
    g = _gpu(case)
    out = g.forward(_lib.STREAMED).cpu().numpy()
    ref = conv.forward_streamed(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                case.A).numpy()
    err = rel_err(out, ref)
    print(f"config 4 reduced forward rel err {err:.3e}", flush=True)
    assert err <= TOL["float32"]
    ref_b = conv.backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A,
                          case.grad_out)
    _compare(g.backward(), ref_b, "float32", label="config 4 reduced")


def test_uvw_config4_full_size_sampled():
    """16,384 atoms, ~857k edges: sampled receivers/senders/edges and A-bar in full (Eq. 36)."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(4)
    g = _gpu(case)
    out = g.forward(_lib.STREAMED).cpu().numpy()
    got = {k: v.cpu().numpy() for k, v in g.backward().items()}
    rng = np.random.default_rng(44)
    nodes = np.unique(np.concatenate([rng.choice(case.n_nodes, 12, replace=False), [0, case.n_nodes - 1]]))
    keep_r = np.isin(case.recv, nodes)
    ev = case.edge_vec[torch.as_tensor(np.nonzero(keep_r)[0])]
    m = conv.forward_conventional(case.problem, case.x, ev, case.recv[keep_r], case.send[keep_r],
                                  case.phi[keep_r], case.A).numpy()
    err = rel_err(out[nodes], m[nodes])
    print(f"config 4 sampled forward rel err {err:.3e}", flush=True)
    assert err <= TOL["float32"]
    keep = np.isin(case.send, nodes) | keep_r
    idx = np.nonzero(keep)[0]
    sub = conv.backward(case.problem, case.x, case.edge_vec[torch.as_tensor(idx)], case.recv[keep],
                        case.send[keep], case.phi[keep], case.A, case.grad_out, n_nodes=case.n_nodes)
    checks = {"x": (got["x"][nodes], sub["x"].numpy()[nodes]),
              "pos": (got["pos"][nodes], sub["pos"].numpy()[nodes]),
              "edge_vec": (got["edge_vec"][idx], sub["edge_vec"].numpy()),
              "phi": (got["phi"][idx], sub["phi"].numpy())}
    for k, (a, b) in checks.items():
        err = rel_err(a, b)
        print(f"config 4 sampled grad {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL["float32"], (k, err)


@pytest.fixture(scope="module")
def config4_grad_A():
    """Config 4 at full size (16,384 atoms, ~857k edges): the library's grad_A from the streamed
    forward + backward, computed once for the per-output-block oracle comparisons below."""
    case = make_case(4)
    g = _gpu(case)
    gA = g.backward(want=("A",))["A"].cpu().numpy()
    return case, gA


@pytest.mark.parametrize("block", [0, 1, 2])
def test_uvw_config4_full_size_grad_A_by_output_block(config4_grad_A, block):
    """A-bar sums over every edge of the graph (Sobek section 4.3, Eq. 36: A-bar = S^T m-bar per
    path): every path's columns, grouped by output block (0e, 1o, 2e) so that each oracle run
    stays within a test's time; the oracle forms the receiver state of one path at a time."""
    from tests.gpu_helpers import TOL, rel_err
    case, gA_gpu = config4_grad_A
    pick = [p.index for p in case.problem.paths if p.i_out == block]
    assert pick
    cols = np.concatenate([np.arange(case.problem.paths[k].weight_offset,
                                     case.problem.paths[k].weight_offset + case.problem.paths[k].n_weights)
                           for k in pick])
    ev = case.edge_vec
    parts = [conv.grad_A_streamed(case.problem, case.x, ev, case.recv, case.send, case.phi, case.grad_out,
                                  paths=[k]) for k in pick]
    ref = np.concatenate([t.numpy() for t in parts], axis=1)
    err = rel_err(gA_gpu[:, cols], ref)
    print(f"config 4 grad A, output block {block} (paths {pick}, all edges): rel err {err:.3e}", flush=True)
    assert err <= TOL["float32"]


@pytest.mark.parametrize("dtype", ["float32", "float64"])
def test_uvw_gemm_tile_loads_alignment_independent(dtype):
    """Multiplicities that are multiples of 4 let the GEMMs read their tiles in 16-byte groups
    when the tensors are 16-byte aligned; A and grad_out passed as views one element off that
    alignment take the element-by-element loads, which must give bit-identical results."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    spec = dict(irreps_in="8x0e+4x1o+4x2e", irreps_out="4x0e+8x1o+4x2e", mode="uvw")
    case = make_case(1, irreps_override=spec, dtype=dtype)
    g = _gpu(case)
    out = g.forward(_lib.STREAMED)
    grads = g.backward()

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    A_off, gout_off = shifted(g.A), shifted(g.grad_out)
    assert A_off.data_ptr() % 16 != 0 and gout_off.data_ptr() % 16 != 0
    out_off = g.conv.forward(g.x, g.pos, g.shift, g.phi, A_off, schedule=_lib.STREAMED)
    grads_off = g.conv.backward(g.x, g.pos, g.shift, g.phi, A_off, gout_off)
    torch.cuda.synchronize()
    assert torch.equal(out, out_off)
    for k in KEYS:
        assert torch.equal(grads[k], grads_off[k]), k
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    err = rel_err(out.cpu().numpy(), ref)
    print(f"uvw mul%4 {dtype} forward rel err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,budget", [("float64", 0), ("float32", 0), ("float64", 64 << 10)])
def test_uvw_kept_state_gives_identical_results(dtype, budget):
    """Forward keeping the receiver state and the backward reading it: bitwise the results of the
    plain forward and of the backward that recomputes the state (also with a small scratch budget,
    where the forward and the backward cut the receivers into different chunks)."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    case = make_case(1, irreps_override=RAGGED, dtype=dtype)
    g = _gpu(case)
    if budget:
        g.plan.set_scratch_budget(budget)
    out = g.forward(_lib.STREAMED)
    grads = g.backward()
    state = g.conv.state_buffer()
    assert state.numel() == _lib.state_size(g.plan, g.graph)
    out_k = g.conv.forward(g.x, g.pos, g.shift, g.phi, g.A, schedule=_lib.STREAMED, state=state)
    grads_k = g.conv.backward(g.x, g.pos, g.shift, g.phi, g.A, g.grad_out, state=state)
    torch.cuda.synchronize()
    assert torch.equal(out, out_k)
    for k in KEYS:
        assert torch.equal(grads[k], grads_k[k]), k
    # Without grad_A the state is not read: the other gradients are unchanged.
    part = g.conv.backward(g.x, g.pos, g.shift, g.phi, g.A, g.grad_out, want=("x", "phi"), state=state)
    assert torch.equal(part["x"], grads["x"]) and torch.equal(part["phi"], grads["phi"])


def test_kept_state_schedule_rule():
    """A fully connected plan keeps its receiver state in the streamed forward only."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    case = make_case(1, irreps_override=RAGGED, dtype="float64")
    g = _gpu(case)
    state = g.conv.state_buffer()
    with pytest.raises(ValueError):
        g.conv.forward(g.x, g.pos, g.shift, g.phi, g.A, schedule=_lib.CONVENTIONAL, state=state)
