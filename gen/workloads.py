"""Seeded synthetic workloads at the shapes the speculative-decoding pages use.

Every array is drawn from numpy's ``default_rng`` keyed by a fixed seed (and a
per-array tag), so the oracle and the GPU path see identical bytes.  bf16
tensors are returned as ``uint16`` bit patterns (round-to-nearest-even from
float32 normals); fp32 tensors as ``float32``.

Layout conventions shared by both sides (they are the library's layouts):

* queries ``q``: ``[B][n_q][Hq][d]``;
* contiguous KV cache ``k``/``v``: ``[B][T_cap][Hkv][d]``; the prefix occupies
  positions ``0..P-1`` and tree node ``i`` sits at position ``P + i``;
* paged KV pool: ``[num_blocks][block_size][Hkv][d]`` with ``block_table``
  ``[B][max_blocks]`` (int32, -1 where unused);
* tree: ``parent[b][i]`` with ``-1 <= parent[i] < i``; ``-1`` means "child of
  the root", the root being the last prefix token.  Target-side trees put the
  root token itself at node 0 (``parent[0] = -1`` and ``parent[i] >= 0`` for
  ``i >= 1``).

Cache rows past ``P + n`` (and unused paged slots) are filled with NaN so
that any stray read shows up in the results.

Nothing here computes the method (no masks, softmax, argmax, acceptance or
compaction).  Planting a path only writes chosen logits to +16 / -16, far
outside what an N(0,1) draw reaches.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)
PLANT_HI = np.float32(16.0)   # planted argmax value (N(0,1) never gets there)
PLANT_LO = np.float32(-16.0)  # planted "certainly not the argmax" value


# ----------------------------------------------------------------------------
# elementary draws
# ----------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even) and return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(shape, key, dtype: str, parallel: bool = True) -> np.ndarray:
    """N(0,1) array of ``shape`` drawn in rows along axis 0.

    Row ``r`` comes from ``default_rng(key + [r])`` so that generation can run
    on several threads and stays identical for any thread count
    (``parallel=False`` for callers that are already on a worker thread).
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    if out.size == 0:
        return out
    rows = shape[0]
    per = int(np.prod(shape[1:])) if len(shape) > 1 else 1

    def work(r):
        x = np.random.default_rng(list(key) + [r]).standard_normal(per, dtype=np.float32)
        if dtype == "bf16":
            out[r] = bf16_bits_from_f32(x).reshape(shape[1:])
        else:
            out[r] = x.reshape(shape[1:])

    if parallel and rows * per > 4_000_000:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(rows)))
    else:
        for r in range(rows):
            work(r)
    return out


def _nan_fill(dtype: str):
    return BF16_NAN_BITS if dtype == "bf16" else np.float32(np.nan)


def _sibling_distinct_tokens(rng, parent: np.ndarray, vocab: int) -> np.ndarray:
    """Token ids, distinct among nodes that share a parent (-1 group included)."""
    n = parent.shape[0]
    tok = np.empty(n, dtype=np.int32)
    for p in np.unique(parent):
        idx = np.nonzero(parent == p)[0]
        tok[idx] = rng.choice(vocab, size=idx.size, replace=False)
    return tok


def _walk_up(parent: np.ndarray, e: int) -> list:
    """Node ids from the top of the tree down to ``e`` (input construction)."""
    out = []
    u = int(e)
    while u >= 0:
        out.append(u)
        u = int(parent[u])
    return out[::-1]


def _plant_path(logits: np.ndarray, parent: np.ndarray, tok: np.ndarray, n: int, e: int) -> list:
    """Make the target's greedy choices follow the draft down to node ``e``.

    Along the root path of ``e`` each node's row gets +16 at the next node's
    token; every child of ``e`` gets -16 at its own token in ``e``'s row, so
    the walk stops at ``e``.  Returns the path (top-down).
    """
    path = _walk_up(parent[:n], e)
    for a, b in zip(path[:-1], path[1:]):
        logits[a, tok[b]] = PLANT_HI
    for c in range(n):
        if parent[c] == e:
            logits[e, tok[c]] = PLANT_LO
    return path


# ----------------------------------------------------------------------------
# the case container
# ----------------------------------------------------------------------------

@dataclass
class Case:
    name: str
    dtype: str                    # "f32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    d: int
    n_max: int
    T_cap: int                    # logical capacity (tokens) per sequence
    scale: float
    q: np.ndarray                 # [B][n_max][Hq][d] verify queries (all nodes)
    k: np.ndarray                 # contiguous [B][T_cap][Hkv][d] or pool [NB][bs][Hkv][d]
    v: np.ndarray
    prefix_len: np.ndarray        # [B] int32
    parent: np.ndarray            # [B][n_max] int32
    n_nodes: np.ndarray           # [B] int32
    block_table: Optional[np.ndarray] = None  # [B][max_blocks] int32 (paged only)
    block_size: int = 0
    vocab: int = 0
    tok: Optional[np.ndarray] = None          # [B][n_max] int32
    root_tok: Optional[np.ndarray] = None     # [B] int32
    logits: Optional[np.ndarray] = None       # [B][n_max][vocab] float32
    planted: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def paged(self) -> bool:
        return self.block_table is not None


def _contiguous_kv(key, B, P_max, n_max, Hkv, d, dtype, prefix_len, n_nodes, tail=16):
    T_cap = int(P_max + n_max + tail)
    k = _normal((B, T_cap, Hkv, d), list(key) + [11], dtype)
    v = _normal((B, T_cap, Hkv, d), list(key) + [12], dtype)
    for b in range(B):
        end = int(prefix_len[b] + n_nodes[b])
        k[b, end:] = _nan_fill(dtype)
        v[b, end:] = _nan_fill(dtype)
    return T_cap, k, v


def _paged_kv(key, rng, B, prefix_len, n_nodes, n_max, Hkv, d, dtype, block_size, max_blocks,
              spare_blocks=4):
    """Paged pool with physical blocks in a seeded random order.

    Sequence ``b`` uses ``ceil((P_b + n_max) / block_size)`` blocks (room for
    its tree); the keys (values) of sequence ``b`` are one stream from
    ``default_rng(key + [21 (22), b, 0])`` in logical token order, scattered
    into their blocks.
    """
    need = [(int(prefix_len[b]) + n_max + block_size - 1) // block_size for b in range(B)]
    total = int(sum(need)) + spare_blocks
    perm = rng.permutation(total).astype(np.int32)
    pool_k = np.empty((total, block_size, Hkv, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    pool_v = np.empty_like(pool_k)
    pool_k[...] = _nan_fill(dtype)
    pool_v[...] = _nan_fill(dtype)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    at = 0
    jobs = []
    for b in range(B):
        table[b, : need[b]] = perm[at: at + need[b]]
        at += need[b]
        jobs.append(b)

    def fill(b):
        T = need[b] * block_size
        valid = int(prefix_len[b] + n_nodes[b])
        kk = _normal((1, T, Hkv, d), list(key) + [21, b], dtype, parallel=False)[0]
        vv = _normal((1, T, Hkv, d), list(key) + [22, b], dtype, parallel=False)[0]
        kk[valid:] = _nan_fill(dtype)
        vv[valid:] = _nan_fill(dtype)
        blocks = table[b, : need[b]]
        pool_k[blocks] = kk.reshape(need[b], block_size, Hkv, d)
        pool_v[blocks] = vv.reshape(need[b], block_size, Hkv, d)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, jobs))
    return pool_k, pool_v, table


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

def config1_tiny(seed: int = 1) -> Case:
    """Tiny fp32 case: B=1, Hq=8, Hkv=1, d=64, prefix 128, a 16-node forest.

    Parents are uniform in ``[-1, i-1]`` (several children of the root), tokens
    live in a 256-word vocabulary and differ among siblings.  One planted path
    ends at a random node; ``root_tok`` is the token of its first node.  The
    expand call uses the last 4 nodes (a 4 x 144 mask), verify uses all 16.
    """
    rng = np.random.default_rng([seed, 0])
    B, Hq, Hkv, d, P, n, V = 1, 8, 1, 64, 128, 16, 256
    parent = np.empty((B, n), dtype=np.int32)
    parent[0, 0] = -1
    for i in range(1, n):
        parent[0, i] = rng.integers(-1, i)
    prefix_len = np.full(B, P, dtype=np.int32)
    n_nodes = np.full(B, n, dtype=np.int32)
    tok = _sibling_distinct_tokens(rng, parent[0], V)[None, :]
    logits = rng.standard_normal((B, n, V), dtype=np.float32)
    e = int(rng.integers(0, n))
    path = _plant_path(logits[0], parent[0], tok[0], n, e)
    root_tok = np.array([tok[0, path[0]]], dtype=np.int32)
    q = _normal((B, n, Hq, d), [seed, 1], "f32")
    T_cap, k, v = _contiguous_kv([seed], B, P, n, Hkv, d, "f32", prefix_len, n_nodes)
    return Case("tiny", "f32", B, Hq, Hkv, d, n, T_cap, 1.0 / np.sqrt(d), q, k, v,
                prefix_len, parent, n_nodes, vocab=V, tok=tok, root_tok=root_tok,
                logits=logits, planted={"end": [e], "path_len": [len(path)], "expand_w": 4})


def _geometric_matches(rng, p_accept: float, D: int, B: int) -> np.ndarray:
    """Matched-draft counts K with P(K >= k) = p_accept**k, capped at D."""
    return np.minimum(rng.geometric(1.0 - p_accept, size=B) - 1, D).astype(np.int32)


def _chain_case(name, seed, B, Hq, Hkv, d, P, D, vocab, prefix_len=None, paged=False,
                block_size=16, max_blocks=0, p_accept=0.7) -> Case:
    rng = np.random.default_rng([seed, 0])
    n = D + 1
    if prefix_len is None:
        prefix_len = np.full(B, P, dtype=np.int32)
    n_nodes = np.full(B, n, dtype=np.int32)
    parent = np.tile(np.arange(-1, n - 1, dtype=np.int32), (B, 1))
    tok = rng.integers(0, vocab, size=(B, n), dtype=np.int32)
    root_tok = tok[:, 0].copy()
    K = _geometric_matches(rng, p_accept, D, B)
    logits = np.empty((B, n, vocab), dtype=np.float32)
    for b in range(B):
        logits[b] = np.random.default_rng([seed, 3, b]).standard_normal((n, vocab), dtype=np.float32)
        for j in range(int(K[b])):
            logits[b, j, tok[b, j + 1]] = PLANT_HI
        if K[b] < D:
            logits[b, K[b], tok[b, K[b] + 1]] = PLANT_LO
    q = _normal((B, n, Hq, d), [seed, 1], "bf16")
    if paged:
        k, v, table = _paged_kv([seed], rng, B, prefix_len, n_nodes, n, Hkv, d, "bf16",
                                block_size, max_blocks)
        T_cap = max_blocks * block_size
    else:
        T_cap, k, v = _contiguous_kv([seed], B, int(prefix_len.max()), n, Hkv, d, "bf16",
                                     prefix_len, n_nodes, tail=0)
        table = None
    return Case(name, "bf16", B, Hq, Hkv, d, n, T_cap, 1.0 / np.sqrt(d), q, k, v,
                prefix_len.astype(np.int32), parent, n_nodes, block_table=table,
                block_size=block_size if paged else 0, vocab=vocab, tok=tok,
                root_tok=root_tok, logits=logits,
                planted={"matches": K.tolist(), "path_len": (K + 1).tolist()})


def config2_chain(seed: int = 2, B: int = 16, P: int = 32768) -> Case:
    """Chain verify: D=15, Hq=64, Hkv=8 (G=8 -> 128 rows per KV head), d=128,
    bf16, batch 16, prefix 32768; the target agrees with the draft for a
    geometric(0.7) number of tokens (vocabulary 32000)."""
    return _chain_case("chain_verify", seed, B, 64, 8, 128, P, 15, 32000)


def config3_tree(seed: int = 3, B: int = 8, P: int = 4096) -> Case:
    """Llama-70B-shaped per-GPU share at TP=4: Hq=16, Hkv=2, d=128, bf16,
    batch 8, prefix 4096, an 8-node target tree (node 0 = root token,
    parent[i] uniform in [0, i-1]) with a planted accepted path."""
    rng = np.random.default_rng([seed, 0])
    Hq, Hkv, d, n, V = 16, 2, 128, 8, 32000
    parent = np.empty((B, n), dtype=np.int32)
    tok = np.empty((B, n), dtype=np.int32)
    root_tok = np.empty(B, dtype=np.int32)
    logits = np.empty((B, n, V), dtype=np.float32)
    ends, lens = [], []
    for b in range(B):
        parent[b, 0] = -1
        for i in range(1, n):
            parent[b, i] = rng.integers(0, i)
        tok[b] = _sibling_distinct_tokens(rng, parent[b], V)
        root_tok[b] = tok[b, 0]
        logits[b] = np.random.default_rng([seed, 3, b]).standard_normal((n, V), dtype=np.float32)
        e = int(rng.integers(0, n))
        path = _plant_path(logits[b], parent[b], tok[b], n, e)
        ends.append(e)
        lens.append(len(path))
    prefix_len = np.full(B, P, dtype=np.int32)
    n_nodes = np.full(B, n, dtype=np.int32)
    q = _normal((B, n, Hq, d), [seed, 1], "bf16")
    T_cap, k, v = _contiguous_kv([seed], B, P, n, Hkv, d, "bf16", prefix_len, n_nodes, tail=0)
    return Case("tree_verify_l70b", "bf16", B, Hq, Hkv, d, n, T_cap, 1.0 / np.sqrt(d), q, k, v,
                prefix_len, parent, n_nodes, vocab=V, tok=tok, root_tok=root_tok, logits=logits,
                planted={"end": ends, "path_len": lens})


def config5_paged(seed: int = 5, m: int = 32, block_size: int = 16) -> Case:
    """Two alternating batches of m=32 requests (64 resident), prefix lengths
    uniform in [512, 8192], paged KV in 16-token blocks in a seeded random
    physical order, chain k=5 (6 query nodes), Hq=64, Hkv=8, d=128, bf16.
    Batch s is requests ``[s*m, (s+1)*m)``."""
    rng = np.random.default_rng([seed, 100])
    B = 2 * m
    prefix_len = rng.integers(512, 8193, size=B).astype(np.int32)
    D = 5
    max_blocks = (8192 + D + 1 + block_size - 1) // block_size
    c = _chain_case("paged_alternating", seed, B, 64, 8, 128, 0, D, 32000, prefix_len=prefix_len,
                    paged=True, block_size=block_size, max_blocks=max_blocks)
    c.planted["batch_size"] = m
    return c


@dataclass
class ExpandCase:
    """Draft-side expansion rounds (Llama-8B-shaped draft)."""
    name: str
    dtype: str
    Hq: int
    Hkv: int
    d: int
    P: int
    n0: int
    w: int
    rounds: int
    vocab: int
    scale: float
    T_cap: int
    k: np.ndarray           # [1][T_cap][Hkv][d] bf16 bits (prefix + all future tree slots)
    v: np.ndarray
    parent0: np.ndarray     # [n0] initial forest (parents uniform in [-1, i-1])
    tok0: np.ndarray        # [n0] tokens of the initial nodes (distinct among siblings)
    logits_root: np.ndarray  # [vocab] float32 (distribution after the root)
    logits0: np.ndarray      # [n0][vocab] float32
    logits_new: np.ndarray   # [rounds][w][vocab] float32
    q_new: np.ndarray        # [rounds][1][w][Hq][d] bf16 bits

    @property
    def n_max(self) -> int:
        return self.n0 + self.w * self.rounds


def config4_expand(seed: int = 4) -> ExpandCase:
    """Draft expansion: Hq=32, Hkv=8, d=128, bf16, batch 1, prefix 2048, an
    initial 64-node tree, then d=4 rounds of w=8 new leaves over vocabulary
    32000.  The new leaves' K/V are pre-drawn at tree slots 64..95 (their
    values do not depend on which candidates win)."""
    rng = np.random.default_rng([seed, 0])
    Hq, Hkv, d, P, n0, w, R, V = 32, 8, 128, 2048, 64, 8, 4, 32000
    parent0 = np.empty(n0, dtype=np.int32)
    parent0[0] = -1
    for i in range(1, n0):
        parent0[i] = rng.integers(-1, i)
    tok0 = _sibling_distinct_tokens(rng, parent0, V)
    logits_root = np.random.default_rng([seed, 3, 0]).standard_normal(V, dtype=np.float32)
    logits0 = np.random.default_rng([seed, 3, 1]).standard_normal((n0, V), dtype=np.float32)
    logits_new = np.random.default_rng([seed, 3, 2]).standard_normal((R, w, V), dtype=np.float32)
    n_max = n0 + w * R
    T_cap = P + n_max
    k = _normal((1, T_cap, Hkv, d), [seed, 11], "bf16")
    v = _normal((1, T_cap, Hkv, d), [seed, 12], "bf16")
    q_new = _normal((R, 1, w, Hq, d), [seed, 1], "bf16")
    return ExpandCase("draft_expand_l8b", "bf16", Hq, Hkv, d, P, n0, w, R, V, 1.0 / np.sqrt(d),
                      T_cap, k, v, parent0, tok0, logits_root, logits0, logits_new, q_new)


# ----------------------------------------------------------------------------
# generic small cases for parity sweeps
# ----------------------------------------------------------------------------

def random_case(seed: int, B: int, Hq: int, Hkv: int, d: int, P_range=(0, 300), n_max: int = 16,
                n_range=None, dtype: str = "bf16", target_side: bool = False, paged: bool = False,
                block_size: int = 16, vocab: int = 512, chain: bool = False) -> Case:
    """A small seeded case with ragged per-sequence prefix lengths and tree sizes.

    ``target_side`` puts the root token at node 0 (parents of later nodes are
    >= 0); otherwise parents are uniform in ``[-1, i-1]``.  ``chain`` makes
    every sequence a chain.  Logits carry a planted path per sequence.
    """
    rng = np.random.default_rng([seed, 0])
    lo, hi = P_range
    prefix_len = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    if n_range is None:
        n_range = (1, n_max)
    n_nodes = rng.integers(n_range[0], n_range[1] + 1, size=B).astype(np.int32)
    parent = np.full((B, n_max), -1, dtype=np.int32)
    tok = np.zeros((B, n_max), dtype=np.int32)
    root_tok = np.zeros(B, dtype=np.int32)
    logits = np.random.default_rng([seed, 3]).standard_normal((B, n_max, vocab), dtype=np.float32)
    lens = []
    for b in range(B):
        n = int(n_nodes[b])
        for i in range(1, n):
            if chain:
                parent[b, i] = i - 1
            elif target_side:
                parent[b, i] = rng.integers(0, i)
            else:
                parent[b, i] = rng.integers(-1, i)
        tok[b, :n] = _sibling_distinct_tokens(rng, parent[b, :n], vocab)
        e = int(rng.integers(0, n)) if n > 0 else -1
        if e >= 0:
            path = _plant_path(logits[b], parent[b], tok[b], n, e)
            root_tok[b] = tok[b, path[0]]
            lens.append(len(path))
        else:
            lens.append(0)
    q = _normal((B, n_max, Hq, d), [seed, 1], dtype)
    if paged:
        max_blocks = (int(prefix_len.max()) + n_max + block_size - 1) // block_size
        k, v, table = _paged_kv([seed], rng, B, prefix_len, n_nodes, n_max, Hkv, d, dtype,
                                block_size, max_blocks)
        T_cap = max_blocks * block_size
    else:
        T_cap, k, v = _contiguous_kv([seed], B, int(prefix_len.max()), n_max, Hkv, d, dtype,
                                     prefix_len, n_nodes)
        table = None
    return Case(f"random{seed}", dtype, B, Hq, Hkv, d, n_max, T_cap, 1.0 / np.sqrt(d), q, k, v,
                prefix_len, parent, n_nodes, block_table=table,
                block_size=block_size if paged else 0, vocab=vocab, tok=tok,
                root_tok=root_tok, logits=logits, planted={"path_len": lens})
