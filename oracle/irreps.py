"""Irreps strings, the ir_mul feature layout and path enumeration (oracle).

Sobek section 2.2 (Eqs. 3-5): features are a direct sum of blocks
x_{l,sigma} in R^{C x (2l+1)}, C_x = sum C (2l+1); a path couples an input
block (l1, s1) with a spherical-harmonic block (l2, s2) into an output block
(l3, s3) when |l1 - l2| <= l3 <= l1 + l2 and s3 = s1 s2.  Section 2.3 (Eq. 6)
distinguishes channelwise ``uvu`` (input channel u feeds output channel u,
one weight per channel, so mul_in must equal mul_out) from fully connected
``uvw`` (a weight for every (u, w) pair).  Section 2.4 (Eqs. 8-9): n_pi =
C_in C_out for uvw (C for uvu) and N_w = sum_pi n_pi.

Readings (the pages are silent): paths are taken in lexicographic order of
(input block, SH block, output block) indices; several paths into one output
block are summed; the columns of A are ordered path-major, then u (uvu) or
(u, w) with u major (uvw); blocks use the ir_mul layout (Sobek section 4.5):
element (m, u) of a block at offset o with multiplicity C sits at o + m C + u.
"""

from __future__ import annotations

import dataclasses
import re
from typing import List, Tuple


@dataclasses.dataclass(frozen=True)
class Block:
    mul: int
    l: int
    parity: int  # +1 even, -1 odd
    offset: int  # start within the flattened feature vector

    @property
    def dim(self) -> int:
        return 2 * self.l + 1

    @property
    def size(self) -> int:
        return self.mul * self.dim


def parse(s: str) -> List[Block]:
    blocks = []
    off = 0
    for tok in s.replace(" ", "").split("+"):
        m = re.fullmatch(r"(\d+)x(\d+)([eo])", tok)
        if not m:
            raise ValueError(f"bad irreps token {tok!r}")
        mul, l, p = int(m.group(1)), int(m.group(2)), (1 if m.group(3) == "e" else -1)
        b = Block(mul, l, p, off)
        blocks.append(b)
        off += b.size
    return blocks


def total_dim(blocks: List[Block]) -> int:
    return sum(b.size for b in blocks)


@dataclasses.dataclass(frozen=True)
class Path:
    index: int
    i_in: int
    i_sh: int
    i_out: int
    l1: int
    l2: int
    l3: int
    weight_offset: int  # first column of this path in A
    n_weights: int


@dataclasses.dataclass
class Problem:
    irreps_in: List[Block]
    irreps_sh: List[Block]
    irreps_out: List[Block]
    mode: str
    paths: List[Path]

    @property
    def n_weights(self) -> int:
        return sum(p.n_weights for p in self.paths)

    @property
    def c_in(self) -> int:
        return total_dim(self.irreps_in)

    @property
    def c_out(self) -> int:
        return total_dim(self.irreps_out)

    @property
    def sh_dim(self) -> int:
        return total_dim(self.irreps_sh)

    @property
    def lmax_sh(self) -> int:
        return max(b.l for b in self.irreps_sh)


def make_problem(irreps_in: str, irreps_sh: str, irreps_out: str, mode: str) -> Problem:
    bi, bs, bo = parse(irreps_in), parse(irreps_sh), parse(irreps_out)
    for b in bs:
        if b.mul != 1:
            raise ValueError("spherical-harmonic irreps must have multiplicity 1")
    if [b.l for b in bs] != list(range(len(bs))):
        raise ValueError("spherical-harmonic irreps must be 0..lmax in order")
    # The edge blocks always hold the real spherical harmonics of the edge direction; their parity
    # label, normally (-1)^l, only enters path selection.  LunaTP's profile C1 (Appendix A.1, table
    # of node, edge and output irreps) labels its degree-1 edge block "1e"; that label is accepted
    # as given (the resulting operator is then rotation- but not inversion-equivariant).
    if mode not in ("uvu", "uvw"):
        raise ValueError(mode)
    paths: List[Path] = []
    off = 0
    for i, a in enumerate(bi):
        for j, s in enumerate(bs):
            for k, o in enumerate(bo):
                if not (abs(a.l - s.l) <= o.l <= a.l + s.l):
                    continue
                if a.parity * s.parity != o.parity:
                    continue
                if mode == "uvu":
                    if a.mul != o.mul:
                        continue
                    n = a.mul
                else:
                    n = a.mul * o.mul
                paths.append(Path(len(paths), i, j, k, a.l, s.l, o.l, off, n))
                off += n
    return Problem(bi, bs, bo, mode, paths)


def path_counts(problem: Problem) -> Tuple[int, int]:
    return len(problem.paths), problem.n_weights
