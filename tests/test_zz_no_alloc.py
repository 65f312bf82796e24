"""Allocation-free forward (cgtp_conv_forward_static) against cgtp_conv_forward (needs an MI355X).

The static entry point keeps the per-chunk rows of folded coefficients in the library's static
device array (CGTP_STATIC_SCRATCH_BYTES) instead of a caller workspace.  It is called here through
the C ABI on two inputs in a row, the second smaller, with one plan: its outputs must equal those of
the workspace entry point bit for bit (the same kernels; chunks that differ only in where receivers
are cut give the same per-receiver sums) and match the oracle.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from oracle import conv
from tests.oracle_helpers import make_case

pytestmark = pytest.mark.gpu

L3_128 = dict(irreps_in="128x0e+128x1o+128x2e", irreps_sh="1x0e+1x1o+1x2e+1x3o",
              irreps_out="128x0e+128x1o+128x2e+128x3o")
INVALID_ARG, UNSUPPORTED = 1, 2


class _Inputs:
    """Graph and device tensors of an oracle case, for a given plan."""

    def __init__(self, lib, case):
        w = case.raw
        self.case = case
        self.graph = lib.Graph(w.n_nodes, w.recv, w.send, w.image)
        perm = self.graph.perm
        assert np.array_equal(perm, case.perm)
        dev = dict(dtype=torch.float32, device="cuda")
        r32 = lambda a: a.astype(np.float32).astype(np.float64)  # noqa: E731
        self.x = torch.tensor(case.x, **dev)
        self.pos = torch.tensor(case.pos, **dev)
        self.shift = torch.tensor(r32(w.shift[perm]), **dev).contiguous()
        self.phi = torch.tensor(r32(w.phi[perm]), **dev).contiguous()
        self.A = torch.tensor(case.A, **dev)


def _static(lib, plan, inp, schedule, out):
    so = lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    return so.cgtp_conv_forward_static(plan.handle, inp.graph.handle, schedule, inp.x.data_ptr(), inp.pos.data_ptr(),
                                       inp.shift.data_ptr(), inp.phi.data_ptr(), inp.A.data_ptr(), out.data_ptr(),
                                       stream)


def _oracle_rows(case, rows):
    keep = np.isin(case.recv, rows)
    ev = case.edge_vec[torch.as_tensor(np.nonzero(keep)[0])]
    m = conv.forward_conventional(case.problem, case.x, ev, case.recv[keep], case.send[keep], case.phi[keep],
                                  case.A)
    return m.numpy()[rows]


@pytest.mark.parametrize("schedule", ["conventional", "streamed"])
def test_static_forward_matches_workspace_forward(schedule):
    from clebsch_gordan_tensor_receiver_amd import _lib
    from tests.gpu_helpers import TOL, rel_err
    sch = _lib.CONVENTIONAL if schedule == "conventional" else _lib.STREAMED
    big = make_case(2)                                               # 1,024 atoms, 91k edges
    small = make_case(1, irreps_override=L3_128, dtype="float32")     # 64 atoms, 2.2k edges
    assert big.A.shape == small.A.shape
    plan = _lib.Plan(L3_128["irreps_in"], L3_128["irreps_sh"], L3_128["irreps_out"], "uvu", "float32", 8)
    row_bytes = (plan.info["g_nnz"] + 3) // 4 * 4 * 4
    # The large graph's rows do not fit the static array in one chunk: the static call cuts chunks.
    assert len(big.recv) * row_bytes > ctypes.c_size_t(64 << 20).value
    ins = [_Inputs(_lib, big), _Inputs(_lib, small)]
    refs = []
    for inp in ins:                     # uploads the graphs, loads the kernels (allocating calls)
        inp.graph.upload()
        out = torch.empty((inp.case.n_nodes, plan.info["c_out"]), dtype=torch.float32, device="cuda")
        _lib.conv_forward(plan, inp.graph, sch, inp.x, inp.pos, inp.shift, inp.phi, inp.A, out,
                          torch.empty(_lib.workspace_size(plan, inp.graph, _lib.OP_FORWARD), dtype=torch.uint8,
                                      device="cuda"))
        refs.append(out)
    outs = [torch.full_like(r, float("nan")) for r in refs]
    torch.cuda.synchronize()
    # Two calls in a row, the second on the smaller graph; then both again with free memory watched.
    assert _static(_lib, plan, ins[0], sch, outs[0]) == 0, _lib.load().cgtp_last_error()
    assert _static(_lib, plan, ins[1], sch, outs[1]) == 0, _lib.load().cgtp_last_error()
    torch.cuda.synchronize()
    for o, r in zip(outs, refs):
        assert torch.equal(o, r)
    again = [torch.full_like(r, float("nan")) for r in refs]
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    assert _static(_lib, plan, ins[0], sch, again[0]) == 0
    assert _static(_lib, plan, ins[1], sch, again[1]) == 0
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    print(f"{schedule}: free device memory {free0} -> {free1} across two static calls", flush=True)
    assert free1 == free0
    for o, r in zip(again, refs):
        assert torch.equal(o, r)
    for inp, o, seed in ((ins[0], outs[0], 31), (ins[1], outs[1], 32)):
        c = inp.case
        rng = np.random.default_rng(seed)
        rows = np.unique(np.concatenate([rng.choice(c.n_nodes, min(24, c.n_nodes), replace=False),
                                         [0, c.n_nodes - 1]]))
        err = rel_err(o.cpu().numpy()[rows], _oracle_rows(c, rows))
        print(f"{schedule} static forward, {c.n_nodes} atoms: sampled rel err {err:.3e}", flush=True)
        assert err <= TOL["float32"]


def test_static_forward_preconditions():
    """Refused on the host, before any launch: a graph not on the device, kernels never loaded on
    it, a fully connected plan."""
    from clebsch_gordan_tensor_receiver_amd import _lib
    case = make_case(1, irreps_override=L3_128, dtype="float32")
    plan = _lib.Plan(L3_128["irreps_in"], L3_128["irreps_sh"], L3_128["irreps_out"], "uvu", "float32", 8)
    inp = _Inputs(_lib, case)
    out = torch.empty((case.n_nodes, plan.info["c_out"]), dtype=torch.float32, device="cuda")
    assert _static(_lib, plan, inp, _lib.CONVENTIONAL, out) == INVALID_ARG      # graph not uploaded
    inp.graph.upload()
    assert _static(_lib, plan, inp, _lib.CONVENTIONAL, out) == UNSUPPORTED      # kernels not loaded
    uvw = _lib.Plan("4x0e+4x1o", "1x0e+1x1o", "4x0e+4x1o", "uvw", "float32", 8)
    dev = dict(dtype=torch.float32, device="cuda")
    x = torch.zeros((case.n_nodes, uvw.info["c_in"]), **dev)
    A = torch.zeros((8, uvw.info["n_weights"]), **dev)
    o = torch.zeros((case.n_nodes, uvw.info["c_out"]), **dev)
    so = _lib.load()
    st = so.cgtp_conv_forward_static(uvw.handle, inp.graph.handle, _lib.STREAMED, x.data_ptr(), inp.pos.data_ptr(),
                                     inp.shift.data_ptr(), inp.phi.data_ptr(), A.data_ptr(), o.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    assert st == UNSUPPORTED
