"""Scaling sweeps shaped like the Sobek page's section 5.1 ("Scaling axes", "Representative irrep
profiles"): inputs only, no convolution arithmetic.

* Degree axis: one set of 2,048 uniform positions (periodic box at 0.1 atoms/A^3, Morton order);
  the cutoff is chosen per point so that the expected receiver degree is 4 ... 1,023.
* Graph-count axis: one 128-node graph of expected degree 32 (same density), repeated B = 2 ... 511
  times as disjoint copies (node indices offset by 128 per copy).

Both axes span about 8.2e3 to 2.1e6 directed edges.  The irrep profiles hold 128 scalar channels
and 64 channels per non-scalar order, inputs equal to outputs with alternating parity, one SH copy
per order up to L_max, fully connected paths and K = 16 radial functions (Gaussian basis), fp32.

Seeds: PCG64(1000 * SWEEP_SEED + stream) with stream 0 positions, 1 node features, 2 radial
matrix A, 3 output cotangent, 8 edge-order shuffle; the repeated graph draws its positions from
stream 10.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

from .graphs import _morton_order, gaussian_basis, neighbour_list

SWEEP_SEED = 61
DENSITY = 0.1                     # atoms per cubic Angstrom
K = 16
DEGREES = (4, 8, 16, 32, 64, 128, 256, 512, 1023)
COPIES = (2, 4, 8, 16, 32, 64, 128, 256, 511)


def _alt(lmax: int, scalar_mul: int = 128, mul: int = 64) -> str:
    parts = [f"{scalar_mul}x0e"] + [f"{mul}x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(1, lmax + 1)]
    return "+".join(parts)


def _sh(lmax: int) -> str:
    return "+".join(f"1x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(lmax + 1))


# Profiles with blocks of different multiplicities: the node and edge irreps of LunaTP's kernel
# microbenchmark cases (Appendix A.1, table of cases C1-C10) that mix multiplicities, with outputs
# equal to the inputs (channelwise paths join blocks of equal multiplicity).  C1 labels its
# degree-1 edge block "1e" as the page does.
LUNATP_HETERO = {
    "C1": dict(irreps_in="128x0e+64x1e+32x2e", irreps_sh="1x0e+1x1e+1x2e"),
    "C3": dict(irreps_in="128x0e+64x1o+32x2e+32x3o", irreps_sh=None),
    "C5": dict(irreps_in="320x0e+96x1o+64x2e+32x3o+32x4e", irreps_sh=None),
    "C7": dict(irreps_in="128x0e+64x1o+32x2e+32x3o+32x4e+32x5o", irreps_sh=None),
    "C9": dict(irreps_in="128x0e+64x1o+32x2e+32x3o+32x4e+32x5o+32x6e", irreps_sh=None),
}


def lunatp_profile(case: str) -> dict:
    """irreps_in / irreps_sh / irreps_out of a LunaTP heterogeneous case (SH up to its largest degree)."""
    d = LUNATP_HETERO[case]
    lmax = max(int(tok.split("x")[1][:-1]) for tok in d["irreps_in"].split("+"))
    return dict(irreps_in=d["irreps_in"], irreps_sh=d["irreps_sh"] or _sh(lmax), irreps_out=d["irreps_in"])


# L_max -> irreps of the "128/64", "128/64/64" and "128/64/64/64" profiles.
PROFILES = {L: dict(irreps_in=_alt(L), irreps_sh=_sh(L), irreps_out=_alt(L), mode="uvw", dtype="float32", K=K)
            for L in (1, 2, 3)}


@dataclasses.dataclass
class SweepGraph:
    axis: str                # "degree" or "copies"
    point: int               # target degree or copy count
    n_nodes: int
    recv: np.ndarray         # (E,) int32, seeded random order
    send: np.ndarray
    image: np.ndarray        # (E, 3) int32
    shift: np.ndarray        # (E, 3) float64
    pos: np.ndarray          # (N, 3) float64
    box: np.ndarray
    rc: float
    phi: np.ndarray          # (E, K) float64

    @property
    def n_edges(self) -> int:
        return int(self.recv.shape[0])

    @property
    def mean_degree(self) -> float:
        return self.n_edges / self.n_nodes


def _rng(stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * SWEEP_SEED + stream))


def _cutoff(degree: float) -> float:
    """Radius whose sphere holds `degree` atoms on average at DENSITY."""
    return (3.0 * degree / (4.0 * math.pi * DENSITY)) ** (1.0 / 3.0)


def _uniform(n: int, stream: int):
    box = np.full(3, (n / DENSITY) ** (1.0 / 3.0))
    pos = _rng(stream).uniform(0.0, 1.0, size=(n, 3)) * box
    return pos[_morton_order(pos, box, _cutoff(32.0))], box


def _finish(axis, point, pos, box, rc, recv, send, image) -> SweepGraph:
    perm = _rng(8).permutation(len(recv))
    recv, send, image = recv[perm], send[perm], image[perm]
    shift = image.astype(np.float64) * box[None, :]
    r = np.linalg.norm(pos[send] - pos[recv] + shift, axis=1)
    return SweepGraph(axis, point, len(pos), recv, send, image, shift, pos, box, rc, gaussian_basis(r, rc, K))


def degree_graph(degree: int) -> SweepGraph:
    """Radius graph on 2,048 fixed positions with the cutoff of expected degree `degree`."""
    pos, box = _uniform(2048, 0)
    rc = _cutoff(degree)
    recv, send, image = neighbour_list(pos, box, rc)
    return _finish("degree", degree, pos, box, rc, recv, send, image)


def copies_graph(copies: int) -> SweepGraph:
    """`copies` disjoint copies of one 128-node graph of expected degree 32."""
    pos1, box = _uniform(128, 10)
    rc = _cutoff(32.0)
    r1, s1, i1 = neighbour_list(pos1, box, rc)
    off = (np.arange(copies, dtype=np.int64) * 128)[:, None]
    recv = (r1[None, :] + off).reshape(-1).astype(np.int32)
    send = (s1[None, :] + off).reshape(-1).astype(np.int32)
    image = np.tile(i1, (copies, 1))
    pos = np.tile(pos1, (copies, 1))  # copies share coordinates; they never exchange edges
    return _finish("copies", copies, pos, box, rc, recv, send, image)


# Skewed in-degrees (the "task ordering" setting of LunaTP section 4.2): 4,096 uniform positions at
# DENSITY; receiver i keeps the senders within its own cutoff, chosen for an expected degree
# d_i = 32 exp(sigma z_i), z_i ~ N(0, 1) (stream 12), clipped to [4, 1024].  Point = 10 sigma.
SKEW_POINTS = (0, 5, 10, 15)
# The channelwise profile measured on it: the l <= 3, 128-channel irreps of the diamond workload
# with this module's K = 16 Gaussian radial functions.
SKEW_PROFILE = dict(irreps_in=_alt(2, 128, 128), irreps_sh=_sh(3), irreps_out=_alt(3, 128, 128), mode="uvu",
                    dtype="float32", K=K)


def skew_graph(point: int, n: int = 4096) -> SweepGraph:
    sigma = point / 10.0
    pos, box = _uniform(n, 11)
    z = _rng(12).normal(size=n)
    deg = np.clip(np.round(32.0 * np.exp(sigma * z)), 4, 1024)
    rcut = np.array([_cutoff(d) for d in deg])
    recv, send, image = neighbour_list(pos, box, float(rcut.max()))
    r = np.linalg.norm(pos[send] - pos[recv] + image * box[None, :], axis=1)
    keep = r < rcut[recv]
    return _finish("skew", point, pos, box, float(rcut.max()), recv[keep], send[keep], image[keep])


def sweep_graph(axis: str, point: int) -> SweepGraph:
    if axis == "skew":
        return skew_graph(point)
    return degree_graph(point) if axis == "degree" else copies_graph(point)


# Channelwise sweeps on the 1,024-atom diamond graph (the l <= 3 workload's graph):
# multiplicity C of C x (0e,1o,2e) -> C x (0e,1o,2e,3o) with SH l <= 3, and L of
# 64 x (0..L) -> 64 x (0..L) with SH l <= L (parities (-1)^l).
CHANNEL_POINTS = (16, 32, 64, 128, 256)
LMAX_POINTS = (1, 2, 3, 4)


def channelwise_profile(axis: str, point: int):
    """(irreps_in, irreps_sh, irreps_out) of a channelwise sweep point (axis "channels" or "lmax")."""
    if axis == "channels":
        return _alt(2, point, point), _sh(3), _alt(3, point, point)
    return _alt(point, 64, 64), _sh(point), _alt(point, 64, 64)


def normal(stream: int, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws rounded to float32 (kept as float64)."""
    return _rng(stream).normal(0.0, std, size=shape).astype(np.float32).astype(np.float64)
