"""Host-side checks of the C-ABI library (no GPU): exported symbols, plan tables against the
oracle's Clebsch-Gordan tensors and path enumeration, the CSR against the oracle's sort, and the
status codes of invalid calls."""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import cg, csr
from oracle.irreps import make_problem
from workloads import make_workload
from workloads.graphs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cgtp.h")


@pytest.fixture(scope="module")
def lib():
    from clebsch_gordan_tensor_receiver_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from clebsch_gordan_tensor_receiver_amd import build
        build.build()
    return _lib


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cgtp_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("cgtp_plan_create", "cgtp_graph_build", "cgtp_workspace_size", "cgtp_conv_forward",
              "cgtp_conv_backward", "cgtp_conv_double_backward", "cgtp_error_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    so = lib.load()
    for n in _declared():
        assert hasattr(so, n), n
    assert sorted(lib.EXPORTED) == sorted(_declared())


@pytest.mark.parametrize("config", sorted(CONFIGS))
def test_plan_matches_oracle_paths_and_cg(lib, config):
    s = CONFIGS[config]
    plan = lib.Plan(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"], s["dtype"], s["K"])
    prob = make_problem(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"])
    info = plan.info
    assert info["n_paths"] == len(prob.paths)
    assert info["n_weights"] == prob.n_weights
    assert (info["c_in"], info["c_out"], info["sh_dim"]) == (prob.c_in, prob.c_out, prob.sh_dim)
    assert info["num_radial"] == s["K"]
    nnz = 0
    for k, P in enumerate(prob.paths):
        d = plan.path(k)
        assert (d["i_in"], d["i_sh"], d["i_out"], d["l1"], d["l2"], d["l3"]) == (P.i_in, P.i_sh, P.i_out, P.l1, P.l2,
                                                                                  P.l3)
        assert (d["weight_offset"], d["n_weights"]) == (P.weight_offset, P.n_weights)
        idx, val = plan.cg_table(k)
        ref = cg.sparse_terms(P.l1, P.l2, P.l3)
        assert [tuple(r) for r in idx.tolist()] == [t[:3] for t in ref], k
        assert np.abs(val - np.array([t[3] for t in ref])).max() <= 1e-15
        nnz += len(ref)
    assert info["cg_nnz"] == nnz


def test_survey_table_counts(lib):
    # Path counts, weight counts and widths of the five workloads, as tabulated from the path rule.
    want = {1: (7, 56, 32, 72, 9), 2: (17, 2176, 1152, 2048, 16), 3: (17, 1088, 576, 1024, 16),
            4: (11, 45056, 576, 576, 9), 5: (106, 3392, 1568, 1568, 49)}
    for c, (P, nw, cin, cout, yd) in want.items():
        s = CONFIGS[c]
        info = lib.Plan(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"], s["dtype"], s["K"]).info
        assert (info["n_paths"], info["n_weights"], info["c_in"], info["c_out"], info["sh_dim"]) == (P, nw, cin, cout,
                                                                                                      yd), c


def _graph_vs_oracle(lib, n, recv, send, image):
    g = lib.Graph(n, recv, send, image)
    perm, row_ptr, col = csr.receiver_csr(n, recv, send, image)
    rp, c, sp, se = g.export()
    assert np.array_equal(g.perm, perm)
    assert np.array_equal(rp, row_ptr)
    assert np.array_equal(c, col)
    src_ptr, src_edge = csr.source_csr(n, col)
    assert np.array_equal(sp, src_ptr)
    assert np.array_equal(se, src_edge)


@pytest.mark.parametrize("config", [1, 2])
def test_graph_csr_bit_exact(lib, config):
    w = make_workload(config)
    _graph_vs_oracle(lib, w.n_nodes, w.recv, w.send, w.image)


def test_graph_edge_cases(lib):
    rng = np.random.default_rng(5)
    # Isolated nodes, repeated (recv, send) pairs told apart by the image index, self-loops of
    # periodic images, and ties broken by the input index.
    n = 9
    recv = rng.integers(0, 5, size=60).astype(np.int32)
    send = rng.integers(0, 5, size=60).astype(np.int32)
    image = rng.integers(-1, 2, size=(60, 3)).astype(np.int32)
    _graph_vs_oracle(lib, n, recv, send, image)
    _graph_vs_oracle(lib, n, recv, send, None)
    # Duplicate edges with identical keys keep their input order.
    _graph_vs_oracle(lib, 3, np.array([1, 1, 1, 0], np.int32), np.array([2, 2, 2, 2], np.int32), None)
    # No edges at all.
    g = lib.Graph(4, np.zeros(0, np.int32), np.zeros(0, np.int32))
    rp, c, sp, se = g.export()
    assert rp.tolist() == [0] * 5 and sp.tolist() == [0] * 5 and len(c) == 0 and len(se) == 0


def _status(fn):
    from clebsch_gordan_tensor_receiver_amd._lib import CgtpError
    with pytest.raises(CgtpError) as e:
        fn()
    return e.value.status


INVALID_ARG, UNSUPPORTED, WORKSPACE = 1, 2, 3


def test_invalid_plans_are_rejected(lib):
    mk = lib.Plan
    assert _status(lambda: mk("8x0e+bad", "1x0e+1x1o", "8x0e", "uvu")) == INVALID_ARG
    assert _status(lambda: mk("8x0e", "1x0e+1x2e", "8x0e", "uvu")) == INVALID_ARG      # SH degrees not 0..L
    assert _status(lambda: mk("8x0e", "1x0e+2x1o", "8x0e", "uvu")) == INVALID_ARG      # SH multiplicity
    assert _status(lambda: mk("8x0e", "1x1o+1x0e", "8x0e", "uvu")) == INVALID_ARG      # SH degree order
    assert mk("8x0e+8x1e", "1x0e+1x1e", "8x0e+8x1e", "uvu").info["n_paths"] == 5      # parity label as given
    assert _status(lambda: mk("8x0e", "1x0e", "8x0e", "uvu", num_radial=0)) == INVALID_ARG
    assert _status(lambda: mk("8x0e", "1x0e", "8x1o", "uvu")) == UNSUPPORTED           # no admissible path
    assert _status(lambda: mk("8x0e", "1x0e", "4x0e", "uvu")) == UNSUPPORTED           # uvu needs mul_in = mul_out
    sh7 = "+".join(f"1x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(8))
    assert _status(lambda: mk("8x0e", sh7, "8x0e", "uvu")) == UNSUPPORTED              # degrees above 6


def test_invalid_graphs_are_rejected(lib):
    i32 = lambda *v: np.array(v, np.int32)  # noqa: E731
    assert _status(lambda: lib.Graph(0, i32(), i32())) == INVALID_ARG
    assert _status(lambda: lib.Graph(3, i32(0, 3), i32(1, 1))) == INVALID_ARG
    assert _status(lambda: lib.Graph(3, i32(0, 1), i32(-1, 1))) == INVALID_ARG


def test_host_validation_before_any_device_work(lib):
    so = lib.load()
    plan = lib.Plan("8x0e+8x1o", "1x0e+1x1o", "8x0e+8x1o", "uvu", "float64", 4)
    uvw = lib.Plan("8x0e+8x1o", "1x0e+1x1o", "8x0e+8x1o", "uvw", "float64", 4)
    g = lib.Graph(3, np.array([0, 1], np.int32), np.array([1, 2], np.int32))
    n = ctypes.c_size_t()
    assert so.cgtp_workspace_size(plan.handle, g.handle, 2, ctypes.byref(n)) == 0 and n.value >= 256
    # Fully connected: double backward yes (phi an input), triple backward no.
    assert so.cgtp_workspace_size(uvw.handle, g.handle, 2, ctypes.byref(n)) == 0 and n.value >= 256
    assert so.cgtp_workspace_size(uvw.handle, g.handle, 3, ctypes.byref(n)) == UNSUPPORTED
    assert so.cgtp_plan_compile(uvw.handle, 1 << 3) == UNSUPPORTED
    nul = [None] * 10
    assert so.cgtp_conv_forward(plan.handle, g.handle, 0, *[None] * 6, None, 0, None) == INVALID_ARG
    assert so.cgtp_conv_forward(plan.handle, g.handle, 7, *[1] * 6, None, 0, None) == INVALID_ARG  # bad schedule
    assert so.cgtp_conv_backward(plan.handle, g.handle, *nul, None, None, 0, None) == INVALID_ARG
    assert so.cgtp_conv_double_backward(plan.handle, g.handle, *[None] * 18, 0, None) == INVALID_ARG
    assert so.cgtp_conv_double_backward(uvw.handle, g.handle, *[1] * 6, *[None] * 5, 1, *[None] * 5, 1, 16,
                                        None) == WORKSPACE
    # Workspace smaller than cgtp_workspace_size: refused before touching the device.
    assert so.cgtp_conv_backward(plan.handle, g.handle, *[1] * 6, 1, None, None, None, None, 1, 16, None) == WORKSPACE
    assert so.cgtp_conv_double_backward(plan.handle, g.handle, *[1] * 6, *[None] * 5, 1, *[None] * 5, 1, 16,
                                        None) == WORKSPACE
    first = ctypes.c_int(7)
    assert so.cgtp_check_edges(plan.handle, g.handle, None, None, None, 0, None, ctypes.byref(first)) == INVALID_ARG
    assert so.cgtp_check_edges(plan.handle, g.handle, 1, None, 1, 2, None, ctypes.byref(first)) == WORKSPACE
    assert so.cgtp_check_edges(plan.handle, g.handle, 1, None, 1, 2, None, None) == INVALID_ARG
    assert so.cgtp_plan_set_scratch_budget(plan.handle, 16) == INVALID_ARG
    # Radial basis: kinds 0..2, positive cutoff; phi NULL exactly when the plan computes it.
    assert so.cgtp_plan_set_radial(plan.handle, 3, 3.0) == INVALID_ARG
    assert so.cgtp_plan_set_radial(plan.handle, 1, 0.0) == INVALID_ARG
    assert so.cgtp_conv_forward(plan.handle, g.handle, 0, 1, 1, None, None, 1, 1, None, 0, None) == INVALID_ARG
    rad = lib.Plan("8x0e+8x1o", "1x0e+1x1o", "8x0e+8x1o", "uvu", "float64", 4)
    assert so.cgtp_plan_set_radial(rad.handle, 2, 3.0) == 0
    assert so.cgtp_conv_forward(rad.handle, g.handle, 0, 1, 1, None, 1, 1, 1, None, 0, None) == INVALID_ARG
    # The double backward of a radial plan takes neither phi nor a phi direction.
    assert so.cgtp_conv_double_backward(rad.handle, g.handle, 1, 1, None, 1, 1, 1, *[None] * 12, 0,
                                        None) == INVALID_ARG
    assert so.cgtp_conv_double_backward(rad.handle, g.handle, 1, 1, None, None, 1, 1, None, None, None, 1,
                                        *[None] * 8, 0, None) == INVALID_ARG
    assert so.cgtp_plan_path(plan.handle, 99, (ctypes.c_int32 * 9)()) == INVALID_ARG
    assert so.cgtp_error_string(WORKSPACE) == b"workspace too small"
    # Kept state: channelwise plans keep E rows of whole 16-byte units; fully connected ones N x state
    # width; buffer sizes checked before the device.
    assert so.cgtp_state_size(plan.handle, g.handle, ctypes.byref(n)) == 0
    rows = n.value
    assert rows >= 256 and rows % 16 == 0
    assert so.cgtp_conv_backward_with_state(plan.handle, g.handle, *[1] * 6, 1, rows - 1, *[None] * 5, 1, 16,
                                            None) == WORKSPACE
    assert so.cgtp_state_size(uvw.handle, g.handle, ctypes.byref(n)) == 0
    assert n.value >= 256 and n.value % (3 * 8) == 0
    assert so.cgtp_conv_forward_keep_state(uvw.handle, g.handle, *[1] * 6, None, 0, 1, 16, None) == WORKSPACE
    assert so.cgtp_conv_forward_keep_state(uvw.handle, g.handle, *[1] * 6, 1, n.value - 1, 1, 16, None) == WORKSPACE
    assert so.cgtp_conv_backward_with_state(uvw.handle, g.handle, *[1] * 6, None, 0, *[None] * 5, 1, 16,
                                            None) == WORKSPACE


def test_workspace_is_bounded_by_the_scratch_budget(lib):
    s = CONFIGS[2]
    w = make_workload(2)
    plan = lib.Plan(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"], s["dtype"], s["K"])
    g = lib.Graph(w.n_nodes, w.recv, w.send, w.image)
    big = [lib.workspace_size(plan, g, op) for op in (0, 1, 2)]
    plan.set_scratch_budget(1 << 20)
    small = [lib.workspace_size(plan, g, op) for op in (0, 1, 2)]
    for b, sm in zip(big, small):
        assert sm < b
    # The budget covers the per-edge rows, the edge partials and the A-bar partial slots; beyond it
    # only an E x 3 edge-vector buffer, 2 N int32 source bounds and alignment.  Never E x N_w.
    E, N = g.n_edges, g.n_nodes
    nw = plan.info["n_weights"]
    slots_min = 8 * plan.info["num_radial"] * nw * 4      # the eight slots of a chunk, at least
    for sm in small:
        assert sm <= (1 << 20) + slots_min + 4 * 3 * E + 8 * N + 4096
        assert sm < E * nw * 4


def test_workspace_bound_low_degree_large_graph(lib):
    """l <= 3, 128 channels on a 2M-edge graph of in-degree 4 (500k receivers): many receivers per
    edge, so the A-bar partial slots (one K x N_w block per group of 4 receivers) would outgrow
    the budget if the receivers per chunk were not capped.  Host only: workspace sizes."""
    s = CONFIGS[2]
    plan = lib.Plan(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"], s["dtype"], s["K"])
    rng = np.random.default_rng(7)
    N, deg = 500_000, 4
    recv = np.repeat(np.arange(N, dtype=np.int32), deg)
    send = rng.integers(0, N, size=N * deg).astype(np.int32)
    g = lib.Graph(N, recv, send)
    E = g.n_edges
    budget = 256 << 20
    for op in (0, 1, 2):
        ws = lib.workspace_size(plan, g, op)
        print(f"op {op}: workspace {ws / 2**20:.1f} MiB for {E} edges", flush=True)
        assert ws <= budget + 64 * E + (32 << 20), (op, ws)


def test_sweep_profile_weight_counts(lib):
    # Sobek, section 5.1 ("Representative irrep profiles"): the fully connected profiles 128/64,
    # 128/64/64 and 128/64/64/64 have N_w = 36,864, 73,728 and 131,072 radial weights.
    from workloads import sweeps
    want = {1: 36864, 2: 73728, 3: 131072}
    for L, s in sweeps.PROFILES.items():
        info = lib.Plan(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"], s["dtype"], s["K"]).info
        assert info["n_weights"] == want[L], L
        assert info["n_weights"] == make_problem(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"]).n_weights
