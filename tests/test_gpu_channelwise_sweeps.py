"""Channelwise irrep profiles of the channel-count and L_max sweeps (LunaTP, Figure 7: forward
scaling in the multiplicity and the maximum degree with the rest fixed): parity of the HIP
path with the oracle for every sweep point, on the 64-atom periodic graph with 8 radial functions
in float32, the plan the sweep times (needs an MI355X).

The points reach code paths the standard workloads touch less: 16 and 32 channels leave lanes of
every wave idle, 256 channels give four channel blocks per feature block, and L_max = 4 has 9 x 9
coupling paths that the receiver backward streams as vector coefficient rows."""

from __future__ import annotations

import pytest

from oracle import conv
from tests.oracle_helpers import make_case
from workloads.sweeps import CHANNEL_POINTS, LMAX_POINTS, channelwise_profile

pytestmark = pytest.mark.gpu

KEYS = ("x", "pos", "edge_vec", "phi", "A")
POINTS = [("channels", c) for c in CHANNEL_POINTS] + [("lmax", L) for L in LMAX_POINTS]


@pytest.mark.parametrize("axis,point", POINTS)
def test_sweep_point_matches_oracle(axis, point):
    from tests.gpu_helpers import TOL, GpuCase, rel_err
    irr_in, irr_sh, irr_out = channelwise_profile(axis, point)
    ov = dict(irreps_in=irr_in, irreps_sh=irr_sh, irreps_out=irr_out, mode="uvu")
    case = make_case(1, irreps_override=ov, dtype="float32")
    print(f"{axis} {point}: {case.problem.n_weights} weights per radial function, "
          f"{len(case.recv)} edges", flush=True)
    g = GpuCase(case)
    out = g.forward().cpu().numpy()
    grads = {k: v.cpu().numpy() for k, v in g.backward().items()}
    ref = conv.forward_conventional(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi,
                                    case.A).numpy()
    err = rel_err(out, ref)
    print(f"{axis} {point} forward: rel err {err:.3e}", flush=True)
    assert err <= TOL["float32"]
    b = conv.backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A,
                      case.grad_out, n_nodes=case.n_nodes)
    for k in KEYS:
        e = rel_err(grads[k][:len(b[k])], b[k].numpy())
        print(f"{axis} {point} grad {k}: rel err {e:.3e}", flush=True)
        assert e <= TOL["float32"], k
