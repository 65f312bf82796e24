"""Receiver and source CSR of the edge list (oracle; test infrastructure only).

LunaTP section 4.1 stores the adjacency "in CSR format by destination node,
with the edges of node i in the range [rowptr[i], rowptr[i+1])"; section 4.4
and Sobek section 4.3 add a CSR by source node for the node-feature gradient.
Reading for ties (the pages give none): edges are ordered by the key
(receiver, sender, image_x, image_y, image_z, original index); the source CSR
lists, for each sender, the receiver-sorted edge positions in increasing
order.  Written as plain Python loops over a dictionary of buckets, so that it
shares nothing with the library's counting sort.
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def receiver_csr(n_nodes: int, recv, send, image: Optional[np.ndarray] = None):
    """Return (perm, row_ptr, col): perm[k] = original index of the k-th sorted edge."""
    E = len(recv)
    keys = []
    for e in range(E):
        img = tuple(int(v) for v in image[e]) if image is not None else (0, 0, 0)
        keys.append((int(recv[e]), int(send[e])) + img + (e,))
    keys.sort()
    perm = np.array([k[-1] for k in keys], dtype=np.int32)
    row_ptr = np.zeros(n_nodes + 1, dtype=np.int32)
    for k in keys:
        row_ptr[k[0] + 1] += 1
    row_ptr = np.cumsum(row_ptr).astype(np.int32)
    col = np.array([k[1] for k in keys], dtype=np.int32)
    return perm, row_ptr, col


def source_csr(n_nodes: int, sorted_send):
    """Return (src_ptr, src_edge) grouping sorted edge positions by sender."""
    buckets = {j: [] for j in range(n_nodes)}
    for pos, j in enumerate(sorted_send):
        buckets[int(j)].append(pos)
    src_ptr = [0]
    src_edge = []
    for j in range(n_nodes):
        src_edge.extend(buckets[j])
        src_ptr.append(len(src_edge))
    return np.array(src_ptr, dtype=np.int32), np.array(src_edge, dtype=np.int32)
