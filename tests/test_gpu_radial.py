"""Radial basis computed inside the kernels from |r| (cgtp_plan_set_radial): parity with the
oracle's radial functions, including the position gradient through phi(r) (needs an MI355X)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import conv, radial
from tests.oracle_helpers import make_case

pytestmark = pytest.mark.gpu

SMALL_L3 = dict(irreps_in="96x0e+96x1o+96x2e", irreps_sh="1x0e+1x1o+1x2e+1x3o",
                irreps_out="96x0e+96x1o+96x2e+96x3o")
RAGGED_UVW = dict(irreps_in="4x0e+3x1o+2x2e", irreps_out="3x0e+2x1o+5x2e", mode="uvw")
KEYS = ("x", "pos", "edge_vec", "phi", "A")


def _oracle(case, kind, rc):
    ev = case.edge_vec
    phi = radial.basis(kind, radial.edge_lengths(ev), rc, case.phi.shape[1])
    m = conv.forward_conventional(case.problem, case.x, ev, case.recv, case.send, phi, case.A).numpy()
    b = conv.backward(case.problem, case.x, ev, case.recv, case.send, phi, case.A, case.grad_out,
                      n_nodes=case.n_nodes)
    ge = b["edge_vec"] + radial.edge_vec_grad(kind, ev, rc, b["phi"])
    gpos = torch.zeros(case.n_nodes, 3, dtype=torch.float64)
    gpos.index_add_(0, torch.as_tensor(case.send, dtype=torch.long), ge)
    gpos.index_add_(0, torch.as_tensor(case.recv, dtype=torch.long), -ge)
    return m, dict(b, edge_vec=ge, pos=gpos)


def _run(case, kind, rc, schedules):
    from tests.gpu_helpers import GpuCase
    g = GpuCase(case)
    g.plan.set_radial(kind, rc)
    outs = [g.conv.forward(g.x, g.pos, g.shift, None, g.A, schedule=s).cpu().numpy() for s in schedules]
    grads = g.conv.backward(g.x, g.pos, g.shift, None, g.A, g.grad_out)
    return outs, {k: v.cpu().numpy() for k, v in grads.items()}


@pytest.mark.parametrize("kind,cfg,ov,dtype", [
    (1, 1, None, "float64"),
    (2, 1, SMALL_L3, "float32"),
    (1, 1, SMALL_L3, "float32"),
    (2, 1, RAGGED_UVW, "float64"),
])
def test_fused_radial_matches_oracle(kind, cfg, ov, dtype):
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    case = make_case(cfg, irreps_override=ov, dtype=dtype)
    rc = case.raw.spec["rc"]
    uvw = ov is not None and ov.get("mode") == "uvw"
    scheds = (_lib.STREAMED,) if uvw else (_lib.CONVENTIONAL, _lib.STREAMED)
    outs, got = _run(case, kind, rc, scheds)
    m, b = _oracle(case, kind, rc)
    for o in outs:
        err = rel_err(o, m)
        print(f"radial kind {kind} {dtype} forward: rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype]
    for k in KEYS:
        err = rel_err(got[k][:len(b[k])], b[k].numpy())
        print(f"radial kind {kind} {dtype} grad {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype], k


def test_fused_bessel_equals_the_workload_phi():
    # The workloads draw phi with the same Bessel + envelope formula: the fused forward must match
    # the forward fed with the workload's phi (float64, config 1).
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import GpuCase, rel_err
    case = make_case(1)
    g = GpuCase(case)
    given = g.forward().cpu().numpy()
    f = GpuCase(case)
    f.plan.set_radial(1, case.raw.spec["rc"])
    fused = f.conv.forward(f.x, f.pos, f.shift, None, f.A, schedule=_lib.CONVENTIONAL).cpu().numpy()
    err = rel_err(fused, given)
    print(f"fused vs given phi: rel err {err:.3e}", flush=True)
    assert err <= 1e-12


def test_radial_argument_rules():
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import GpuCase
    case = make_case(1)
    g = GpuCase(case)
    g.plan.set_radial(1, 3.0)
    with pytest.raises(_lib.CgtpError) as e:   # phi must be NULL with a radial kind
        g.conv.forward(g.x, g.pos, g.shift, g.phi, g.A)
    assert e.value.status == 1
    h = GpuCase(case)
    with pytest.raises(_lib.CgtpError) as e:   # and present without one
        h.conv.forward(h.x, h.pos, h.shift, None, h.A)
    assert e.value.status == 1
    _ = np


def test_fused_radial_with_kept_state():
    """Fully connected plan with the in-kernel Gaussian basis: the receiver state kept by the
    forward gives the same forward output and gradients, bit for bit, as the recomputing path."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import GpuCase
    case = make_case(1, irreps_override=RAGGED_UVW, dtype="float64")
    g = GpuCase(case)
    g.plan.set_radial(2, case.raw.spec["rc"])
    out = g.conv.forward(g.x, g.pos, g.shift, None, g.A, schedule=_lib.STREAMED)
    grads = g.conv.backward(g.x, g.pos, g.shift, None, g.A, g.grad_out)
    state = g.conv.state_buffer()
    out_k = g.conv.forward(g.x, g.pos, g.shift, None, g.A, schedule=_lib.STREAMED, state=state)
    grads_k = g.conv.backward(g.x, g.pos, g.shift, None, g.A, g.grad_out, state=state)
    torch.cuda.synchronize()
    assert torch.equal(out, out_k)
    for k in KEYS:
        assert torch.equal(grads[k], grads_k[k]), k


NARROW16 = dict(irreps_in="16x0e+16x1o+16x2e", irreps_sh="1x0e+1x1o+1x2e+1x3o",
                irreps_out="16x0e+16x1o+16x2e+16x3o")


@pytest.mark.parametrize("kind,ov,dtype", [
    (1, None, "float64"),
    (2, SMALL_L3, "float32"),
    (1, NARROW16, "float32"),
    (2, None, "float64"),
    (2, RAGGED_UVW, "float64"),
    (1, RAGGED_UVW, "float64"),
    (1, RAGGED_UVW, "float32"),
])
def test_fused_radial_double_backward(kind, ov, dtype):
    """Double backward with phi computed from |r| in the kernels: every output against the oracle
    (phi-input double backward with phidot = phi'(|r|) r-hat.v, plus the chain through phi and
    the curvature of the basis on the edge vector); channelwise and fully connected plans."""
    from tests.gpu_helpers import GpuCase, TOL, rel_err
    from tests.oracle_helpers import effective_edge_direction, make_directions
    case = make_case(1, irreps_override=ov, dtype=dtype)
    rc = case.raw.spec["rc"]
    dirs = make_directions(case)
    dirs.pop("v_phi")
    g = GpuCase(case)
    g.plan.set_radial(kind, rc)
    dt = torch.float64 if dtype == "float64" else torch.float32
    dev = {k: torch.tensor(v, dtype=dt, device="cuda").contiguous() for k, v in dirs.items()}
    got = g.conv.double_backward(g.x, g.pos, g.shift, None, g.A, g.grad_out, **dev)
    v_e = effective_edge_direction(case, dirs["v_edge_vec"], dirs["v_pos"])
    ref = radial.double_backward(kind, rc, case.problem, case.x, case.edge_vec, case.recv, case.send, case.A,
                                 case.grad_out, v_x=dirs["v_x"], v_e=v_e, v_A=dirs["v_A"], n_nodes=case.n_nodes)
    for k in ("x", "pos", "edge_vec", "phi", "A", "grad_out"):
        err = rel_err(got[k].cpu().numpy()[:len(ref[k])], ref[k].numpy())
        print(f"radial kind {kind} {dtype} double backward {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype], k


def test_fused_radial_double_backward_argument_rules():
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import GpuCase
    case = make_case(1)
    g = GpuCase(case)
    g.plan.set_radial(1, case.raw.spec["rc"])
    with pytest.raises(_lib.CgtpError) as e:   # phi must be NULL
        g.conv.double_backward(g.x, g.pos, g.shift, g.phi, g.A, g.grad_out)
    assert e.value.status == 1
    with pytest.raises(_lib.CgtpError) as e:   # and so must v_phi
        g.conv.double_backward(g.x, g.pos, g.shift, None, g.A, g.grad_out, v_phi=g.phi)
    assert e.value.status == 1


def test_fused_radial_double_backward_uvw_config4_irreps():
    """Fully connected 64 x (0e, 1o, 2e), SH l <= 2, 8 Bessel functions, fp32, 300 atoms: every
    output against the oracle."""
    from tests.gpu_helpers import GpuCase, TOL, rel_err
    from tests.oracle_helpers import effective_edge_direction, make_directions
    case = make_case(4, n_nodes=300)
    rc = case.raw.spec["rc"]
    dirs = make_directions(case)
    dirs.pop("v_phi")
    g = GpuCase(case)
    g.plan.set_radial(1, rc)
    dev = {k: torch.tensor(v, dtype=torch.float32, device="cuda").contiguous() for k, v in dirs.items()}
    got = g.conv.double_backward(g.x, g.pos, g.shift, None, g.A, g.grad_out, **dev)
    v_e = effective_edge_direction(case, dirs["v_edge_vec"], dirs["v_pos"])
    ref = radial.double_backward(1, rc, case.problem, case.x, case.edge_vec, case.recv, case.send, case.A,
                                 case.grad_out, v_x=dirs["v_x"], v_e=v_e, v_A=dirs["v_A"], n_nodes=case.n_nodes)
    for k in ("x", "pos", "edge_vec", "phi", "A", "grad_out"):
        err = rel_err(got[k].cpu().numpy()[:len(ref[k])], ref[k].numpy())
        print(f"uvw config-4 irreps radial double backward {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL["float32"], k
