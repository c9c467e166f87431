"""Evolving-tree-cache re-root and KV compaction (test infrastructure).

What is computed (SwiftSpec summary, Section 3.2 and Figure 4; Section 3.1.2
and Figure 2):

* Invariant: the KV cache of a sequence is the prefix cache (verified
  tokens, contiguous) followed immediately by the tree cache (the remaining
  draft nodes, contiguous).
* Update: walk the verified path ``v_0 .. v_{k-1}`` down the tree; those
  nodes join the prefix, in path order, right after the old prefix.  If the
  last verified token is in the tree (``keep``), the subtree under it stays
  valid: its nodes' KV is pulled forward to directly after the new prefix and
  its children become children of the new root.  Otherwise (the target's
  token is not in the tree) a new, empty tree starts.  KV is moved, never
  recomputed.

Readings: kept nodes keep their original relative order; the promoted path
is root-first; with ``k = 0`` and ``keep`` nothing changes; with ``k = 0`` and
not ``keep`` the tree is dropped.  Cache rows at or past the new end
``P + k + |kept|`` are left as they were ("don't care").  Parent entries at
or past the new node count are set to -1.
"""
import numpy as np

from .tree import descendants


def _pos_index(b, p, block_table, block_size):
    if block_table is None:
        return (b, p)
    return (int(block_table[b, p // block_size]), p % block_size)


def tree_cache_reroot(kv_layers, prefix_len, parent, n_nodes, path, path_len, keep,
                      block_table=None, block_size: int = 0):
    """Re-root every sequence; returns new copies.

    ``kv_layers``: list of ``(K, V)`` numpy arrays (any dtype, moved bit for
    bit), contiguous ``[B][T_cap][Hkv][d]`` or paged pools with
    ``block_table``.  Returns ``(new_kv_layers, prefix_len, parent, n_nodes)``.
    """
    B = len(prefix_len)
    n_max = parent.shape[1]
    new_layers = [(k.copy(), v.copy()) for (k, v) in kv_layers]
    P_out = np.array(prefix_len, dtype=np.int32).copy()
    par_out = np.array(parent, dtype=np.int32).copy()
    n_out = np.array(n_nodes, dtype=np.int32).copy()
    for b in range(B):
        P = int(prefix_len[b])
        n = int(n_nodes[b])
        k = int(path_len[b])
        v = [int(x) for x in path[b, :k]]
        if k == 0 and keep[b]:
            continue
        kept = descendants(parent[b], v[-1], n) if (keep[b] and k > 0) else []
        moves = [(P + j, P + v[j]) for j in range(k)] + \
                [(P + k + r, P + kept[r]) for r in range(len(kept))]
        for (K_old, V_old), (K_new, V_new) in zip(kv_layers, new_layers):
            for dst, src in moves:
                K_new[_pos_index(b, dst, block_table, block_size)] = \
                    K_old[_pos_index(b, src, block_table, block_size)]
                V_new[_pos_index(b, dst, block_table, block_size)] = \
                    V_old[_pos_index(b, src, block_table, block_size)]
        newpar = np.full(n_max, -1, dtype=np.int32)
        for r, u in enumerate(kept):
            pu = int(parent[b, u])
            newpar[r] = -1 if pu == v[-1] else kept.index(pu)
        par_out[b] = newpar
        P_out[b] = P + k
        n_out[b] = len(kept)
    return new_layers, P_out, par_out, n_out


def reroot_node_arrays(parent, n: int, path, k: int, keep: bool, tok, cum=None):
    """The per-node arrays the draft keeps beside its tree, after the re-root
    of one sequence (SwiftSpec summary, Section 3.1.1 Algorithm 1: Re-root,
    then Select on the re-rooted tree; Section 3.2: the kept subtree is pulled
    forward).

    ``tok`` (node tokens) and ``cum`` (cumulative log-probabilities, the
    weights of the maximum-likelihood expansion, Section 3.1.3) follow the
    node mapping of ``tree_cache_reroot``: kept node ``kept[r]`` becomes node
    ``r``.  The last verified node ``v = path[k-1]`` becomes the root, and a
    node's weight is the sum of values from the root down to it, so the kept
    weights are re-based: ``cum'[r] = cum[kept[r]] - cum[v]``, the weight of
    the path from the new root.  Entries at or past the new node count read
    -1 (tok) and -inf (cum).  ``k = 0`` with ``keep`` changes nothing.
    Returns ``(tok', cum')`` (``cum'`` None when ``cum`` is None); cum is
    stored as float32, the difference taken in float64 and rounded once.
    """
    tok = np.asarray(tok, dtype=np.int32)
    n_max = tok.shape[0]
    if k == 0 and keep:
        return tok.copy(), None if cum is None else np.asarray(cum, np.float32).copy()
    v = [int(x) for x in path[:k]]
    kept = descendants(parent, v[-1], n) if (keep and k > 0) else []
    tok2 = np.full(n_max, -1, dtype=np.int32)
    for r, u in enumerate(kept):
        tok2[r] = tok[u]
    if cum is None:
        return tok2, None
    cum = np.asarray(cum, dtype=np.float32)
    cum2 = np.full(n_max, -np.inf, dtype=np.float32)
    for r, u in enumerate(kept):
        cum2[r] = np.float32(np.float64(cum[u]) - np.float64(cum[v[-1]]))
    return tok2, cum2
