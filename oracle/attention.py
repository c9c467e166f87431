"""Explicit-mask tree attention in float64 (test infrastructure).

What is computed (SwiftSpec summary, Section 3.1.3 and Figure 3; Section 3.2;
draft-length co-design article, key mechanism):

* The KV cache of sequence ``b`` is the prefix cache (``P`` verified tokens,
  positions ``0..P-1``) followed by the tree cache (node ``i`` at ``P + i``).
* A query at tree node ``i`` may attend to every prefix position and to the
  tree positions of its ancestors and of itself -- the non-square
  ``rows x (prefix + tree)`` mask of Figure 3, where each new leaf sees only
  its ancestors (and itself).
* Grouped-query attention: query head ``h`` reads KV head ``h // G`` with
  ``G = Hq / Hkv`` query heads per KV head.
* Softmax attention with a caller-given ``scale``; the log-sum-exp of the
  scaled, masked scores (natural log) is returned beside the output.

Readings where the pages are silent: the scale is an argument (1/sqrt(d) in
the workloads); LSE uses the natural logarithm; queries and keys arrive with
any positional rotation already applied.
"""
import numpy as np

from .bf16 import to_f64
from .tree import visible_tree_columns


def gather_sequence_kv(k, v, b: int, T: int, dtype: str, block_table=None, block_size: int = 0,
                       kv_head=None):
    """Positions ``0..T-1`` of sequence ``b`` as float64 ``[T][Hkv][d]`` arrays.

    Contiguous caches are ``[B][T_cap][Hkv][d]``; paged pools are
    ``[num_blocks][block_size][Hkv][d]`` where position ``t`` of sequence
    ``b`` lives in block ``block_table[b][t // block_size]`` at slot
    ``t % block_size``.  ``kv_head`` optionally selects one KV head.
    """
    sel = slice(None) if kv_head is None else slice(kv_head, kv_head + 1)
    if block_table is None:
        ks = k[b, :T, sel]
        vs = v[b, :T, sel]
    else:
        nb = (T + block_size - 1) // block_size
        blocks = np.asarray(block_table[b, :nb], dtype=np.int64)
        ks = k[blocks][:, :, sel].reshape(nb * block_size, -1, k.shape[-1])[:T]
        vs = v[blocks][:, :, sel].reshape(nb * block_size, -1, v.shape[-1])[:T]
    return to_f64(ks, dtype), to_f64(vs, dtype)


def tree_attention(q_rows, k_seq, v_seq, P: int, parent, q_nodes, G: int, scale: float,
                   heads=None):
    """Attention for one sequence.

    ``q_rows``: float64 ``[n_q][Hq][d]`` queries of tree nodes ``q_nodes``;
    ``k_seq``/``v_seq``: float64 ``[P + n][Hkv][d]``; ``parent``: the tree.
    Returns ``O`` ``[n_q][Hq][d]`` and ``LSE`` ``[Hq][n_q]`` (float64); heads
    not listed in ``heads`` are left as NaN.
    """
    n_q, Hq, d = q_rows.shape
    T = k_seq.shape[0]
    mask = np.zeros((n_q, T), dtype=bool)
    mask[:, :P] = True
    for r, i in enumerate(q_nodes):
        mask[r, P + visible_tree_columns(parent, int(i))] = True
    O = np.full((n_q, Hq, d), np.nan)
    LSE = np.full((Hq, n_q), np.nan)
    for h in (range(Hq) if heads is None else heads):
        hk = h // G
        S = scale * (q_rows[:, h, :] @ k_seq[:, hk, :].T)
        S[~mask] = -np.inf
        m = S.max(axis=1)
        E = np.exp(S - m[:, None])
        l = E.sum(axis=1)
        LSE[h] = m + np.log(l)
        O[:, h, :] = (E / l[:, None]) @ v_seq[:, hk, :]
    return O, LSE


def _run(case, q, q_nodes_of, batches, heads):
    B, Hq, d = case.B, case.Hq, case.d
    n_q = q.shape[1]
    O = np.full((B, n_q, Hq, d), np.nan)
    LSE = np.full((B, Hq, n_q), np.nan)
    for b in (range(B) if batches is None else batches):
        P = int(case.prefix_len[b])
        n = int(case.n_nodes[b])
        nodes = q_nodes_of(n)
        rows = [r for r, i in enumerate(nodes) if 0 <= i < n]
        if not rows:
            continue
        ks, vs = gather_sequence_kv(case.k, case.v, b, P + n, case.dtype, case.block_table,
                                    case.block_size)
        qr = to_f64(q[b, rows], case.dtype)
        o, lse = tree_attention(qr, ks, vs, P, case.parent[b], [nodes[r] for r in rows],
                                case.G, case.scale, heads)
        O[b, rows] = o
        LSE[b][:, rows] = lse
    return O, LSE


def verify(case, batches=None, heads=None):
    """Verification: the queries are every tree node ``0..n_nodes[b]-1``.

    Rows ``>= n_nodes[b]`` are NaN (they are not outputs).
    """
    return _run(case, case.q, lambda n: list(range(case.q.shape[1])), batches, heads)


def expand(case, q_expand, w: int, batches=None, heads=None):
    """Expansion: the queries are the ``w`` newest nodes ``n-w .. n-1``.

    ``q_expand`` is ``[B][w][Hq][d]``; row ``r`` is node ``n - w + r``.
    Rows whose node index would be negative are NaN.
    """
    return _run(case, q_expand, lambda n: [n - w + r for r in range(w)], batches, heads)
