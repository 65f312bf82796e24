"""Scaling-sweep inputs and the bounded workspace of the library along both axes (host only).

The Sobek page's section 5.2 claims that streaming bounds the tensor-product workspace: peak
memory is the graph and the features plus a fixed scratch budget, never the E x N_w weight
tensor.  cgtp_workspace_size is host-side, so the bound is checked here for every sweep point of
the largest profile without a GPU.
"""

from __future__ import annotations

import numpy as np
import pytest

from workloads import sweeps


@pytest.fixture(scope="module")
def lib():
    from clebsch_gordan_tensor_receiver_amd import _lib
    import os
    if not os.path.exists(_lib.LIB_PATH):
        from clebsch_gordan_tensor_receiver_amd import build
        build.build()
    return _lib


def test_axes_span_the_page_range():
    # Both axes run from about 8.2e3 to 2.1e6 directed edges (section 5.1, "Scaling axes").
    lo_d, hi_d = sweeps.degree_graph(sweeps.DEGREES[0]), sweeps.degree_graph(sweeps.DEGREES[-1])
    lo_c = sweeps.copies_graph(sweeps.COPIES[0])
    assert lo_d.n_nodes == 2048 and 6e3 < lo_d.n_edges < 1.1e4 and 1.8e6 < hi_d.n_edges < 2.3e6
    assert lo_c.n_nodes == 256 and 6e3 < lo_c.n_edges < 1.1e4
    assert abs(hi_d.mean_degree - 1023) < 30 and abs(lo_d.mean_degree - 4) < 1


def test_copies_are_disjoint_repeats():
    g2, g4 = sweeps.copies_graph(2), sweeps.copies_graph(4)
    assert g4.n_edges == 2 * g2.n_edges and g4.n_nodes == 512
    assert np.all(g4.recv // 128 == g4.send // 128)  # no edge between copies
    one = sweeps.copies_graph(2)
    k = one.recv < 128
    r, s = one.recv[k], one.send[k]
    r2, s2 = one.recv[~k] - 128, one.send[~k] - 128
    assert sorted(zip(r.tolist(), s.tolist())) == sorted(zip(r2.tolist(), s2.tolist()))


@pytest.mark.parametrize("axis,point", [("degree", 1023), ("copies", 511), ("degree", 64)])
def test_workspace_is_bounded_along_the_axes(lib, axis, point):
    g = sweeps.sweep_graph(axis, point)
    graph = lib.Graph(g.n_nodes, g.recv, g.send, g.image)
    s = sweeps.PROFILES[3]
    plan = lib.Plan(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"], s["dtype"], s["K"])
    E, N, nw, K = g.n_edges, g.n_nodes, plan.info["n_weights"], s["K"]
    budget = 256 << 20
    for op in (0, 1):
        ws = lib.workspace_size(plan, graph, op)
        # scratch budget + edge-vector and G rows of at most one receiver chunk beyond it, + A-bar
        # slots (K x N_w per XCD group), never a multiple of E x N_w.
        assert ws <= budget + 64 * E + 8 * 4 * K * nw + (64 << 20), (op, ws)
        assert ws < 4 * E * nw / 8, (op, ws)


@pytest.mark.parametrize("axis,points", [("channels", sweeps.CHANNEL_POINTS), ("lmax", sweeps.LMAX_POINTS)])
def test_channelwise_sweep_profiles_match_the_oracle_paths(lib, axis, points):
    """Channelwise sweep plans: the library's path and weight counts equal the oracle's path
    enumeration for every point (17 paths for every multiplicity of the l <= 3 profile)."""
    from oracle.irreps import make_problem
    for pt in points:
        irr_in, irr_sh, irr_out = sweeps.channelwise_profile(axis, pt)
        prob = make_problem(irr_in, irr_sh, irr_out, "uvu")
        plan = lib.Plan(irr_in, irr_sh, irr_out, "uvu", "float32", 8)
        assert plan.info["n_paths"] == len(prob.paths)
        assert plan.info["n_weights"] == prob.n_weights
        if axis == "channels":
            assert len(prob.paths) == 17
