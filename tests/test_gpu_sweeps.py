"""Fully connected irrep profiles of the scaling sweeps (Sobek, section 5.1): parity of the HIP path
with the oracle on a small subgraph of the repeated-graph axis, and sampled parity at a larger
point (needs an MI355X)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import conv
from oracle.irreps import make_problem
from workloads import sweeps

pytestmark = pytest.mark.gpu

KEYS = ("x", "pos", "edge_vec", "phi", "A")


def _setup(g, L, keep=None):
    """Library run of profile L on graph g restricted to the edges `keep` (all if None)."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    s = sweeps.PROFILES[L]
    prob = make_problem(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"])
    keep = np.ones(g.n_edges, bool) if keep is None else keep
    recv, send, image = g.recv[keep], g.send[keep], g.image[keep]
    shift, phi = g.shift[keep], g.phi[keep]
    plan = _lib.Plan(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"], s["dtype"], s["K"])
    graph = _lib.Graph(g.n_nodes, recv, send, image)
    perm = graph.perm
    r32 = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731
    h = dict(x=sweeps.normal(1, (g.n_nodes, prob.c_in)),
             A=sweeps.normal(2, (s["K"], prob.n_weights), std=1.0 / np.sqrt(s["K"])),
             gout=sweeps.normal(3, (g.n_nodes, prob.c_out)), pos=r32(g.pos),
             shift=r32(shift[perm]), phi=r32(phi[perm]), recv=recv[perm], send=send[perm])
    dev = dict(dtype=torch.float32, device="cuda")
    conv_ = _lib.Convolution(plan, graph)
    t = {k: torch.tensor(h[k], **dev).contiguous() for k in ("x", "A", "gout", "pos", "shift", "phi")}
    out = conv_.forward(t["x"], t["pos"], t["shift"], t["phi"], t["A"], schedule=_lib.STREAMED)
    grads = conv_.backward(t["x"], t["pos"], t["shift"], t["phi"], t["A"], t["gout"])
    ev = conv.edge_vectors(h["pos"], h["shift"], h["recv"], h["send"])
    return prob, h, ev, out.cpu().numpy(), {k: v.cpu().numpy() for k, v in grads.items()}


@pytest.mark.parametrize("L", [1, 2, 3])
def test_profile_parity_small_graph(L):
    from tests.gpu_helpers import TOL, rel_err
    g = sweeps.copies_graph(2)
    keep = (g.recv % 128) < 6   # six receivers of each copy with all their in-edges (~370 edges)
    prob, h, ev, out, got = _setup(g, L, keep)
    print(f"profile L{L}: {int(keep.sum())} edges, N_w {prob.n_weights}", flush=True)
    ref = conv.forward_streamed(prob, h["x"], ev, h["recv"], h["send"], h["phi"], h["A"]).numpy()
    err = rel_err(out, ref)
    print(f"profile L{L} forward rel err {err:.3e}", flush=True)
    assert err <= TOL["float32"]
    b = conv.backward(prob, h["x"], ev, h["recv"], h["send"], h["phi"], h["A"], h["gout"], n_nodes=g.n_nodes)
    for k in KEYS:
        e = rel_err(got[k], b[k].numpy())
        print(f"profile L{L} grad {k} rel err {e:.3e}", flush=True)
        assert e <= TOL["float32"], k


def test_profile3_sampled_at_sixteen_copies():
    """128/64/64/64 on 16 copies (~63k edges, one receiver chunk): sampled rows and edges."""
    from tests.gpu_helpers import TOL, rel_err
    g = sweeps.copies_graph(16)
    prob, h, ev, out, got = _setup(g, 3)
    rng = np.random.default_rng(61)
    nodes = np.unique(np.concatenate([rng.choice(g.n_nodes, 6, replace=False), [0, g.n_nodes - 1]]))
    keep_r = np.isin(h["recv"], nodes)
    sel = torch.as_tensor(np.nonzero(keep_r)[0])
    m = conv.forward_streamed(prob, h["x"], ev[sel], h["recv"][keep_r], h["send"][keep_r], h["phi"][keep_r],
                              h["A"]).numpy()
    err = rel_err(out[nodes], m[nodes])
    print(f"16 copies sampled forward rel err {err:.3e}", flush=True)
    assert err <= TOL["float32"]
    keep = np.isin(h["send"], nodes) | keep_r
    idx = np.nonzero(keep)[0]
    sub = conv.backward(prob, h["x"], ev[torch.as_tensor(idx)], h["recv"][keep], h["send"][keep], h["phi"][keep],
                        h["A"], h["gout"], n_nodes=g.n_nodes)
    for k, (a, r) in {"x": (got["x"][nodes], sub["x"].numpy()[nodes]),
                      "pos": (got["pos"][nodes], sub["pos"].numpy()[nodes]),
                      "edge_vec": (got["edge_vec"][idx], sub["edge_vec"].numpy()),
                      "phi": (got["phi"][idx], sub["phi"].numpy())}.items():
        e = rel_err(a, r)
        print(f"16 copies sampled grad {k} rel err {e:.3e}", flush=True)
        assert e <= TOL["float32"], k
