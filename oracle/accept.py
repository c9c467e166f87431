"""Greedy longest-accepted-path selection by brute force (test infrastructure).

What is computed (draft-length co-design article, "how speculative decoding
works" and the Acceptance Length glossary entry; SwiftSpec summary,
Section 3.1.2 Figure 2, where the target's output is the root, the accepted
draft tokens and one token of its own):

* The target's greedy token after node ``i`` is ``a[i] = argmax logits[i]``.
* Node ``i`` is *accepted* when every node ``u`` on its root path carries the
  token the target itself would emit at that point: the token expected of a
  child of the root is ``root_tok`` (the target's choice after the last
  verified token), and of any other node the parent's ``a``.
* The output is the deepest accepted node (``best``), its root path, its
  depth (``path_len``) and the target's own next token ``bonus = a[best]``
  (``root_tok`` when nothing is accepted).

Readings: ties in the argmax go to the lowest vocabulary index; when several
accepted nodes share the maximum depth (only possible with duplicate sibling
tokens) the lowest node index wins.  With the root token stored as node 0
(target side) ``path_len`` is the acceptance length AL, in ``[1, 1 + D]``.

This enumerates every node's root path independently -- deliberately unlike
the GPU's bitmask method.
"""
import numpy as np

from .tree import root_path


def argmax_first(row) -> int:
    """Index of the first maximum of ``row`` (exact comparison in float64)."""
    r = np.asarray(row, dtype=np.float64)
    best = 0
    for j in range(1, r.shape[0]):
        if r[j] > r[best]:
            best = j
    return best


def _argmax_rows(logits_b, n):
    # np.argmax returns the first occurrence of the maximum, like argmax_first.
    return [int(np.argmax(np.asarray(logits_b[i], dtype=np.float64))) for i in range(n)]


def accept_greedy_path(logits, parent, tok, n_nodes, root_tok, n_max=None):
    """Returns ``path [B][n_max]`` (-1 padded), ``path_len [B]``, ``bonus [B]`` (int32)."""
    B = len(n_nodes)
    if n_max is None:
        n_max = parent.shape[1]
    path_out = np.full((B, n_max), -1, dtype=np.int32)
    path_len = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        a = _argmax_rows(logits[b], n)
        best, best_depth = -1, 0
        for i in range(n):
            rp = root_path(parent[b], i)
            ok = int(tok[b, rp[0]]) == int(root_tok[b])
            for x, y in zip(rp[:-1], rp[1:]):
                ok = ok and int(tok[b, y]) == a[x]
            if ok and len(rp) > best_depth:
                best, best_depth = i, len(rp)
        if best < 0:
            bonus[b] = int(root_tok[b])
            continue
        rp = root_path(parent[b], best)
        path_out[b, : len(rp)] = rp
        path_len[b] = len(rp)
        bonus[b] = a[best]
    return path_out, path_len, bonus
