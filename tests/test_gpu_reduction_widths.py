"""Backward and double-backward parity (needs an MI355X) for plans whose per-edge partial columns
are few and not a multiple of four: a handful of radial values K and one or two spherical-harmonic
degrees, at 16, 32 and 64 channels (four, two and one edge per wave step).  The fp32 kernels reduce
each edge's columns over the channels by transposing them inside the 16-lane rows four columns
at a time; a column count that leaves a group incomplete skips the missing folds, which these
cases exercise (1 to 7 columns beyond the last full group)."""

from __future__ import annotations

import numpy as np
import pytest

from oracle import conv
from tests.oracle_helpers import effective_edge_direction, make_case, make_directions

pytestmark = pytest.mark.gpu

CASES = [(c, K, sh) for c in (16, 32, 64) for K in (1, 3) for sh in ("1x0e", "1x0e+1x1o")]


def _narrow_case(c, K, sh):
    case = make_case(1, irreps_override=dict(irreps_in=f"{c}x0e+{c}x1o", irreps_sh=sh,
                                             irreps_out=f"{c}x0e+{c}x1o"), dtype="float32")
    # the first K radial values of the workload (the plan's K is the width of phi)
    case.phi = np.ascontiguousarray(case.phi[:, :K])
    case.A = np.ascontiguousarray(case.A[:K])
    case.raw.phi = np.ascontiguousarray(case.raw.phi[:, :K])
    return case


def _compare(got, ref, keys, label):
    from tests.gpu_helpers import TOL, rel_err
    for k in keys:
        err = rel_err(got[k].cpu().numpy()[:len(ref[k])], ref[k].numpy())
        print(f"{label} {k}: rel err {err:.3e}", flush=True)
        assert err <= TOL["float32"], (k, err)


@pytest.mark.parametrize("c,K,sh", CASES)
def test_backward_few_columns(c, K, sh):
    from tests.gpu_helpers import GpuCase
    case = _narrow_case(c, K, sh)
    ref = conv.backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A,
                        case.grad_out)
    _compare(GpuCase(case).backward(), ref, ("x", "pos", "edge_vec", "phi", "A"), f"{c} ch K={K} {sh}")


@pytest.mark.parametrize("c,K,sh", CASES)
def test_double_backward_few_columns(c, K, sh):
    from tests.gpu_helpers import GpuCase
    case = _narrow_case(c, K, sh)
    dirs = make_directions(case)
    v_e = effective_edge_direction(case, dirs.get("v_edge_vec"), dirs.get("v_pos"))
    ref = conv.double_backward(case.problem, case.x, case.edge_vec, case.recv, case.send, case.phi, case.A,
                               case.grad_out, v_x=dirs["v_x"], v_e=v_e, v_phi=dirs["v_phi"], v_A=dirs["v_A"])
    _compare(GpuCase(case).double_backward(dirs), ref, ("x", "pos", "edge_vec", "phi", "A", "grad_out"),
             f"{c} ch K={K} {sh} (double backward)")
