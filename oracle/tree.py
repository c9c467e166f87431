"""Draft-tree helpers by brute force (test infrastructure).

The draft tree holds one token per node; an edge parent -> child means "the
child's token follows the parent's" (SwiftSpec summary, Section 3.1, the
definition of a draft tree).  Nodes are stored in topological order with
``-1 <= parent[i] < i``; ``-1`` marks a child of the root, the root being the
last token of the prefix cache (the cache layout of Section 3.2).
"""
from typing import List

import numpy as np


def is_valid_parent(parent, n: int) -> bool:
    """True iff ``-1 <= parent[i] < i`` for every node ``i < n``."""
    return all(-1 <= int(parent[i]) < i for i in range(n))


def ancestors(parent, i: int) -> List[int]:
    """Tree ancestors of node ``i`` (nearest first), by following parent links."""
    out = []
    u = int(parent[i])
    while u >= 0:
        out.append(u)
        u = int(parent[u])
    return out


def root_path(parent, i: int) -> List[int]:
    """Nodes from the top of the tree down to ``i`` inclusive."""
    return ancestors(parent, i)[::-1] + [int(i)]


def depth(parent, i: int) -> int:
    """Number of tree nodes on the path from the root to ``i`` (a child of the root has depth 1)."""
    return 1 + len(ancestors(parent, i))


def descendants(parent, v: int, n: int) -> List[int]:
    """All nodes ``u`` (ascending) whose ancestor walk reaches ``v`` (``v`` excluded)."""
    return [u for u in range(n) if v in ancestors(parent, u)]


def visible_tree_columns(parent, i: int) -> np.ndarray:
    """Tree nodes a query at node ``i`` may attend to: its ancestors and itself."""
    return np.array(sorted(ancestors(parent, i) + [int(i)]), dtype=np.int64)
