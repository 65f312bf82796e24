"""Shared helpers for tests: seeded problem set-up on top of ``workloads`` and ``oracle``."""

from __future__ import annotations

import dataclasses
import os

import numpy as np
import torch

from oracle import conv, csr
from oracle.irreps import make_problem
from workloads import make_workload, normal_tensor

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


@dataclasses.dataclass
class Case:
    config: int
    problem: object
    n_nodes: int
    recv: np.ndarray       # receiver-sorted
    send: np.ndarray
    shift: np.ndarray      # (E, 3) receiver-sorted
    image: np.ndarray
    perm: np.ndarray       # sorted position -> original edge index
    row_ptr: np.ndarray
    col: np.ndarray
    pos: np.ndarray
    x: np.ndarray
    phi: np.ndarray        # receiver-sorted
    A: np.ndarray
    grad_out: np.ndarray
    dtype: str
    raw: object

    @property
    def edge_vec(self):
        return conv.edge_vectors(self.pos, self.shift, self.recv, self.send)


def _round(a, dtype):
    return a.astype(np.float32).astype(np.float64) if dtype == "float32" else a


def make_case(config: int, n_nodes=None, dtype=None, irreps_override=None) -> Case:
    w = make_workload(config, n_nodes=n_nodes)
    s = dict(w.spec)
    if irreps_override:
        s.update(irreps_override)
    dtype = dtype or s["dtype"]
    P = make_problem(s["irreps_in"], s["irreps_sh"], s["irreps_out"], s["mode"])
    perm, row_ptr, col = csr.receiver_csr(w.n_nodes, w.recv, w.send, w.image)
    K = s["K"]
    pos = _round(w.pos, dtype)
    shift = _round(w.shift[perm], dtype)
    x = normal_tensor(config, 1, (w.n_nodes, P.c_in), dtype=dtype)
    A = normal_tensor(config, 2, (K, P.n_weights), std=1.0 / np.sqrt(K), dtype=dtype)
    g = normal_tensor(config, 3, (w.n_nodes, P.c_out), dtype=dtype)
    phi = _round(w.phi[perm], dtype)
    return Case(config, P, w.n_nodes, w.recv[perm].astype(np.int32), w.send[perm].astype(np.int32),
                shift, w.image[perm], perm, row_ptr, col, pos, x, phi, A, g, dtype, w)


def wigner_from_sh(l: int, R: np.ndarray, n_samples: int = 64, seed: int = 0) -> np.ndarray:
    """D^l(R) with Y_l(R n) = D^l(R) Y_l(n), fitted by least squares over random directions."""
    from oracle.sh import sh_l, unit
    g = np.random.default_rng(seed)
    n = unit(torch.as_tensor(g.normal(size=(n_samples, 3))))
    Y = sh_l(l, n).numpy()
    YR = sh_l(l, n @ torch.as_tensor(R).T).numpy()
    D, *_ = np.linalg.lstsq(Y, YR, rcond=None)
    return D.T


def random_rotation(seed: int) -> np.ndarray:
    g = np.random.default_rng(seed)
    q, r = np.linalg.qr(g.normal(size=(3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def rotate_features(blocks, feat: np.ndarray, R: np.ndarray, improper: bool = False) -> np.ndarray:
    out = feat.copy()
    for b in blocks:
        D = wigner_from_sh(b.l, R)
        if improper:
            D = D * b.parity
        v = feat[:, b.offset:b.offset + b.size].reshape(-1, b.dim, b.mul)
        out[:, b.offset:b.offset + b.size] = np.einsum("ab,nbu->nau", D, v).reshape(len(feat), -1)
    return out


def make_directions(case: Case) -> dict:
    """Seeded cotangent directions of the double backward, N(0, 1), rounded to the case's dtype.

    Per-edge directions are drawn in the generator's edge order and permuted into receiver-sorted
    order like phi.  v_e is the effective edge-vector direction v_edge_vec + v_pos[send] - v_pos[recv]
    that the oracle takes.
    """
    c = case
    E = len(c.recv)
    v = dict(
        v_x=normal_tensor(c.config, 4, c.x.shape, dtype=c.dtype),
        v_pos=normal_tensor(c.config, 5, c.pos.shape, dtype=c.dtype),
        v_edge_vec=normal_tensor(c.config, 6, (E, 3), dtype=c.dtype)[c.perm],
        v_phi=normal_tensor(c.config, 7, c.phi.shape, dtype=c.dtype)[c.perm],
        v_A=normal_tensor(c.config, 9, c.A.shape, dtype=c.dtype),
    )
    return v


def effective_edge_direction(case: Case, v_edge_vec=None, v_pos=None) -> np.ndarray:
    e = np.zeros((len(case.recv), 3))
    if v_edge_vec is not None:
        e = e + v_edge_vec
    if v_pos is not None:
        e = e + v_pos[case.send] - v_pos[case.recv]
    return e
