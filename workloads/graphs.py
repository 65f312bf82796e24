"""Synthetic atomistic graphs shaped like the workloads on the source pages.

Every random draw comes from a NumPy PCG64 generator seeded with
``1000 * config + stream`` (stream 0 positions, 1 node features, 2 radial
matrix A, 3 output cotangent, 4..7 and 9 double-backward directions, 8 edge-order
shuffle).  The five configurations are:

1. 64 uniform atoms in a 6 A periodic cube, cutoff 3 A, 8x0e+8x1o -> 8x0e+8x1o+8x2e,
   SH lmax 2, channelwise, 8 Bessel functions, float64.
2. 1,024-atom perturbed diamond (4x4x8 conventional cells, a = 3.57 A, jitter
   sigma 0.05 A), cutoff 5 A, 128x(0e,1o,2e) -> 128x(0e,1o,2e,3o), SH lmax 3,
   channelwise, 8 Bessel functions, float32.
3. The graph of 2 with 64 channels, float64.
4. 16,384 uniform atoms at 0.1 atoms/A^3, cutoff 5 A, 64x(0e,1o,2e) in and out,
   SH lmax 2, fully connected, 8 Bessel functions, float32.
5. 4,096 uniform atoms at 60 expected neighbours within 6 A, 32x(0e..6e) in and
   out, SH lmax 6, channelwise, 16 Gaussian functions, float32.

Uniform configurations are sorted into Morton (Z-curve) order of their cell
coordinates, as molecular-dynamics codes do, so that neighbouring receivers
share senders.  The neighbour list enumerates periodic images explicitly and
keeps every (receiver, sender, image) triple with 0 < |r| < r_c; the edge
vector is ``pos[send] - pos[recv] + shift``.  Edges are returned in a seeded
random order (not receiver-sorted): sorting them is part of the method.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
from scipy.spatial import cKDTree


def _alt(mul: int, lmax: int) -> str:
    return "+".join(f"{mul}x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(lmax + 1))


def _sh(lmax: int) -> str:
    return _alt(1, lmax)


CONFIGS: Dict[int, dict] = {
    1: dict(name="tiny-uvu-l2-f64", kind="uniform", n=64, box=(6.0, 6.0, 6.0), rc=3.0,
            irreps_in="8x0e+8x1o", irreps_sh=_sh(2), irreps_out="8x0e+8x1o+8x2e",
            mode="uvu", dtype="float64", radial="bessel", K=8, graph_seed=1),
    2: dict(name="mace-uvu-l3-f32", kind="diamond", cells=(4, 4, 8), a=3.57, jitter=0.05, rc=5.0,
            irreps_in=_alt(128, 2), irreps_sh=_sh(3), irreps_out=_alt(128, 3),
            mode="uvu", dtype="float32", radial="bessel", K=8, graph_seed=2),
    3: dict(name="mace-uvu-l3-f64", kind="diamond", cells=(4, 4, 8), a=3.57, jitter=0.05, rc=5.0,
            irreps_in=_alt(64, 2), irreps_sh=_sh(3), irreps_out=_alt(64, 3),
            mode="uvu", dtype="float64", radial="bessel", K=8, graph_seed=2),
    4: dict(name="uvw-l2-f32", kind="uniform", n=16384, density=0.1, rc=5.0,
            irreps_in=_alt(64, 2), irreps_sh=_sh(2), irreps_out=_alt(64, 2),
            mode="uvw", dtype="float32", radial="bessel", K=8, graph_seed=4),
    5: dict(name="uvu-l6-f32", kind="uniform", n=4096, neighbours=60.0, rc=6.0,
            irreps_in=_alt(32, 6), irreps_sh=_sh(6), irreps_out=_alt(32, 6),
            mode="uvu", dtype="float32", radial="gaussian", K=16, graph_seed=5),
}


@dataclasses.dataclass
class Workload:
    config: int
    spec: dict
    pos: np.ndarray          # (N, 3) float64
    box: np.ndarray          # (3,) orthorhombic periodic box lengths
    recv: np.ndarray         # (E,) int32, receiver i of edge i <- j
    send: np.ndarray         # (E,) int32, sender j
    shift: np.ndarray        # (E, 3) float64 Cartesian image shift (integer multiples of box)
    image: np.ndarray        # (E, 3) int32 image indices
    phi: np.ndarray          # (E, K) radial basis values (float64; round per dtype at use)
    x_seed: int
    dtype: str

    @property
    def n_nodes(self) -> int:
        return int(self.pos.shape[0])

    @property
    def n_edges(self) -> int:
        return int(self.recv.shape[0])

    def rng(self, stream: int) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64(1000 * self.config + stream))


def _rng(config: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * config + stream))


def _diamond(cells, a, jitter, rng):
    basis = np.array([[0, 0, 0], [0, .5, .5], [.5, 0, .5], [.5, .5, 0],
                      [.25, .25, .25], [.25, .75, .75], [.75, .25, .75], [.75, .75, .25]])
    nx, ny, nz = cells
    pts = []
    for ix in range(nx):
        for iy in range(ny):
            for iz in range(nz):
                pts.append((basis + np.array([ix, iy, iz])) * a)
    pos = np.concatenate(pts, axis=0)
    pos = pos + rng.normal(0.0, jitter, size=pos.shape)
    box = np.array([nx * a, ny * a, nz * a], dtype=np.float64)
    pos = np.mod(pos, box)
    return pos, box


def _morton_order(pos, box, rc):
    ncell = np.maximum(1, np.floor(box / rc).astype(np.int64))
    c = np.minimum((pos / box * ncell).astype(np.int64), ncell - 1)
    key = np.zeros(len(pos), dtype=np.int64)
    for bit in range(11):
        for d in range(3):
            key |= ((c[:, d] >> bit) & 1) << (3 * bit + d)
    return np.argsort(key, kind="stable")


def _uniform(n, box, rng, rc):
    pos = rng.uniform(0.0, 1.0, size=(n, 3)) * box
    order = _morton_order(pos, box, rc)
    return pos[order], box


def neighbour_list(pos: np.ndarray, box: np.ndarray, rc: float):
    """All (recv i, send j, image n) with 0 < |pos_j + n*box - pos_i| < rc."""
    tree = cKDTree(pos)
    reach = np.ceil(rc / box).astype(int)
    recvs, sends, imgs = [], [], []
    for nx in range(-reach[0], reach[0] + 1):
        for ny in range(-reach[1], reach[1] + 1):
            for nz in range(-reach[2], reach[2] + 1):
                n = np.array([nx, ny, nz])
                other = cKDTree(pos + n * box)
                sdm = tree.sparse_distance_matrix(other, rc, output_type="ndarray")
                if len(sdm) == 0:
                    continue
                i = sdm["i"].astype(np.int64)
                j = sdm["j"].astype(np.int64)
                d = sdm["v"]
                keep = (d > 0.0) & (d < rc)
                recvs.append(i[keep])
                sends.append(j[keep])
                imgs.append(np.broadcast_to(n, (int(keep.sum()), 3)))
    recv = np.concatenate(recvs)
    send = np.concatenate(sends)
    image = np.concatenate(imgs).astype(np.int32)
    return recv.astype(np.int32), send.astype(np.int32), image


def bessel_basis(r: np.ndarray, rc: float, K: int) -> np.ndarray:
    """sqrt(2/rc) sin(n pi r / rc) / r times the p=6 polynomial envelope, n = 1..K."""
    d = r / rc
    env = 1.0 - 28.0 * d ** 6 + 48.0 * d ** 7 - 21.0 * d ** 8
    n = np.arange(1, K + 1, dtype=np.float64)
    return (math.sqrt(2.0 / rc) * np.sin(np.outer(r, n) * math.pi / rc) / r[:, None]) * env[:, None]


def gaussian_basis(r: np.ndarray, rc: float, K: int) -> np.ndarray:
    """exp(-(r - mu_k)^2 / (2 D^2)), mu_k = k rc / (K-1), D = rc / (K-1)."""
    mu = np.arange(K, dtype=np.float64) * rc / (K - 1)
    delta = rc / (K - 1)
    return np.exp(-((r[:, None] - mu[None, :]) ** 2) / (2.0 * delta * delta))


def make_workload(config: int, n_nodes: Optional[int] = None) -> Workload:
    """Build the graph and radial inputs of ``config``.

    ``n_nodes`` overrides the atom count of uniform configurations (the box is
    rescaled to keep the density), which tests use for reduced sizes.
    """
    spec = dict(CONFIGS[config])
    gseed = spec["graph_seed"]
    rng = _rng(gseed, 0)
    rc = spec["rc"]
    if spec["kind"] == "diamond":
        pos, box = _diamond(spec["cells"], spec["a"], spec["jitter"], rng)
    else:
        n = int(n_nodes or spec["n"])
        if "box" in spec and n_nodes is None:
            box = np.array(spec["box"], dtype=np.float64)
        elif "box" in spec:
            vol = float(np.prod(spec["box"])) * n / spec["n"]
            box = np.full(3, vol ** (1.0 / 3.0))
        elif "density" in spec:
            box = np.full(3, (n / spec["density"]) ** (1.0 / 3.0))
        else:
            dens = spec["neighbours"] / (4.0 / 3.0 * math.pi * rc ** 3)
            box = np.full(3, (n / dens) ** (1.0 / 3.0))
        pos, box = _uniform(n, box, rng, rc)
        spec["n"] = n
    recv, send, image = neighbour_list(pos, box, rc)
    perm = _rng(gseed, 8).permutation(len(recv))
    recv, send, image = recv[perm], send[perm], image[perm]
    shift = image.astype(np.float64) * box[None, :]
    r = np.linalg.norm(pos[send] - pos[recv] + shift, axis=1)
    if spec["radial"] == "bessel":
        phi = bessel_basis(r, rc, spec["K"])
    else:
        phi = gaussian_basis(r, rc, spec["K"])
    return Workload(config=config, spec=spec, pos=pos, box=box, recv=recv, send=send,
                    shift=shift, image=image, phi=phi, x_seed=config, dtype=spec["dtype"])


def normal_tensor(config: int, stream: int, shape, std: float = 1.0, dtype: str = "float64") -> np.ndarray:
    """N(0, std^2) draws from stream ``stream`` of ``config``, rounded to ``dtype``."""
    v = _rng(config, stream).normal(0.0, std, size=shape)
    return v.astype(dtype).astype(np.float64) if dtype == "float32" else v
