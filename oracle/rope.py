"""Rotary position embedding at tree positions, and the KV append of the new
nodes (test infrastructure).

What is computed (SwiftSpec summary, Section 3.3: the masked-attention kernel
fuses the position embedding, RoPE; Section 3.2: the tree cache keeps each
node's KV where it was computed, so a node's position must not depend on
where the node sits in the cache):

* a node's position is that of its token in the sequence it continues: the
  root (the last prefix token) is at P - 1, a node at depth k below it at
  P - 1 + k (depth = nodes on the path from the root, the node included);
* RoPE rotates each pair of channels (j, j + d/2), j < d/2, by the angle
  position * base**(-2 j / d) (the "rotate half" pairing);
* the append writes the new nodes' rotated keys and their values to cache
  rows P + i.

Readings (the pages name RoPE but fix neither the pairing nor the base):
rotate-half pairing, base a parameter (10000 in the tests).
"""
import numpy as np

from .tree import depth


def rope(x, pos, base: float = 10000.0) -> np.ndarray:
    """x [..., d] rotated as at position ``pos`` (float64)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = float(pos) * np.power(float(base), -2.0 * np.arange(h) / d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def tree_positions(parent, n: int, P: int) -> np.ndarray:
    """Position of each tree node: P - 1 + depth."""
    return np.array([P - 1 + depth(parent, i) for i in range(n)], dtype=np.int64)


def rope_append(q, k_new, v_new, prefix_len, parent, n_nodes, n_q: int, expand: bool,
                base: float = 10000.0):
    """Rotated queries [B][n_q][Hq][d] and, per sequence, {cache row: (k, v)}
    for the rows the append writes (float64).  Row slot s holds node s
    (verify) or node n - n_q + s (expand); slots without a node are NaN."""
    B = q.shape[0]
    q_out = np.full(q.shape, np.nan)
    rows = []
    for b in range(B):
        P, n = int(prefix_len[b]), int(n_nodes[b])
        pos = tree_positions(parent[b], n, P)
        rb = {}
        for s in range(n_q):
            node = n - n_q + s if expand else s
            if not 0 <= node < n:
                continue
            q_out[b, s] = rope(q[b, s], pos[node], base)
            rb[P + node] = (rope(k_new[b, s], pos[node], base), np.asarray(v_new[b, s], np.float64))
        rows.append(rb)
    return q_out, rows
