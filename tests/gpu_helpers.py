"""GPU-side set-up for parity tests: the library's own CSR and device copies of the inputs."""

from __future__ import annotations

import numpy as np
import torch

from clebsch_gordan_tensor_receiver_amd import _lib

TOL = {"float32": 1e-5, "float64": 1e-11}


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


class GpuCase:
    """Library plan + graph for an oracle ``Case``; inputs sorted with the library's permutation."""

    def __init__(self, case):
        w = case.raw
        s = w.spec
        p = case.problem
        self.case = case
        self.plan = _lib.Plan(_irreps(p.irreps_in), _irreps(p.irreps_sh), _irreps(p.irreps_out), p.mode,
                              case.dtype, case.phi.shape[1])
        self.graph = _lib.Graph(w.n_nodes, w.recv, w.send, w.image)
        perm = self.graph.perm
        self.conv = _lib.Convolution(self.plan, self.graph)
        dt = torch.float64 if case.dtype == "float64" else torch.float32
        dev = dict(dtype=dt, device="cuda")
        rnd = (lambda a: a.astype(np.float32).astype(np.float64)) if case.dtype == "float32" else (lambda a: a)
        self.x = torch.tensor(case.x, **dev)
        self.pos = torch.tensor(case.pos, **dev)
        self.shift = torch.tensor(rnd(w.shift[perm]), **dev).contiguous()
        self.phi = torch.tensor(rnd(w.phi[perm]), **dev).contiguous()
        self.A = torch.tensor(case.A, **dev)
        self.grad_out = torch.tensor(case.grad_out, **dev)
        self.perm = perm
        _ = s

    def forward(self, schedule=_lib.CONVENTIONAL):
        return self.conv.forward(self.x, self.pos, self.shift, self.phi, self.A, schedule=schedule)

    def backward(self, **kw):
        return self.conv.backward(self.x, self.pos, self.shift, self.phi, self.A, self.grad_out, **kw)

    def double_backward(self, dirs: dict, **kw):
        """dirs: host arrays v_x, v_pos, v_edge_vec, v_phi, v_A (receiver-sorted edges); missing = zero."""
        dt = torch.float64 if self.case.dtype == "float64" else torch.float32
        dev = {k: (torch.tensor(v, dtype=dt, device="cuda").contiguous() if v is not None else None)
               for k, v in dirs.items()}
        return self.conv.double_backward(self.x, self.pos, self.shift, self.phi, self.A, self.grad_out, **dev, **kw)


def _irreps(blocks) -> str:
    return "+".join(f"{b.mul}x{b.l}{'e' if b.parity > 0 else 'o'}" for b in blocks)
