"""Structured inputs that make full-size attention parity able to fail.

With N(0, 1) data at a prefix of tens of thousands of positions, one 32-position
KV tile carries about a thousandth of the softmax mass, so dropping, repeating
or misplacing a tile moves the outputs by less than the bf16 float bars.  The
two input families here give every tile a visible signature while keeping the
shapes, tree, prefix lengths and (paged) block table of a workload:

* ``counting_inputs``: all queries are zero.  Every visible score is then 0,
  so each visible position has weight exactly 1 and a query row's result is
  the plain mean of the value rows it may see.  Values are small-integer
  indicator codes:
    - prefix position t: 1.0 in channel (t // 32) mod n_pc (its tile's code),
      n_pc = d - 16 prefix channels;
    - tree node j (position P + j): 1.0 in channel n_pc + (j mod 15);
    - last channel (d - 1): the integer 1 + (b * Hkv + h) mod 127, the same
      at every valid position of sequence b, KV head h.
  Keys are a finite pattern (1.0 in channel t mod d) that cannot change a zero
  score.

* ``needle_inputs``: every prefix tile j of every (sequence, KV head) holds
  one "needle" at a seeded offset whose key is beta_j * u (u a seeded +-1
  vector of that (sequence, KV head), beta_j in 38/64 .. 44/64), and every
  tree node's key is a needle too; all other keys are 0.  Query rows are
  alpha * u with alpha in 12/16 .. 20/16 per row, so every row scores each
  needle at alpha * beta * d * scale (5 to 10 at d = 128) and every other
  position at 0: each tile carries a comparable share of the mass.  Values
  are 1.0 in the needle tile's code channel (prefix tile j: j mod n_pc; tree
  node j: n_pc + j mod 15) and 0 elsewhere, plus the identity code in the
  last channel.  A tile read with another tile's keys puts its mass on a
  zero value row, so its code channel drops.

Every number stored is exact in bfloat16.  Rows past a sequence's end (and
unused pool slots) are NaN, as in the workloads, so a stray read shows up.
Nothing here computes the method: no masks, softmax or reductions.
"""
from __future__ import annotations

import copy

import numpy as np

from .workloads import BF16_NAN_BITS, Case, bf16_bits_from_f32

TILE = 32
TREE_CODES = 15


def n_prefix_channels(d: int) -> int:
    return d - TREE_CODES - 1


def id_code(b: int, h: int, Hkv: int) -> int:
    return 1 + (b * Hkv + h) % 127


def _bits(x) -> np.uint16:
    return bf16_bits_from_f32(np.asarray([x], dtype=np.float32))[0]


ONE = _bits(1.0)


def _logical_to_storage(case: Case, seq_arrays, what: str):
    """Writes per-sequence logical arrays ``[T_b][Hkv][d]`` (bf16 bits) into
    a contiguous ``[B][T_cap][Hkv][d]`` array or the paged pool of ``case``
    (same block table); everything else is NaN."""
    if case.block_table is None:
        out = np.empty((case.B, case.T_cap, case.Hkv, case.d), dtype=np.uint16)
        out[...] = BF16_NAN_BITS
        for b, a in enumerate(seq_arrays):
            out[b, : a.shape[0]] = a
        return out
    pool = np.empty(getattr(case, what).shape, dtype=np.uint16)
    pool[...] = BF16_NAN_BITS
    bs = case.block_size
    for b, a in enumerate(seq_arrays):
        T = a.shape[0]
        nb = (T + bs - 1) // bs
        blocks = case.block_table[b, :nb].astype(np.int64)
        padded = np.empty((nb * bs,) + a.shape[1:], dtype=np.uint16)
        padded[...] = BF16_NAN_BITS
        padded[:T] = a
        pool[blocks] = padded.reshape(nb, bs, *a.shape[1:])
    return pool


def _value_codes(case: Case, b: int, T: int, P: int, tile_code_rows) -> np.ndarray:
    """Value rows of sequence b: tile / node codes in the rows listed by
    ``tile_code_rows`` (positions and their code channels), identity code in
    the last channel of every row."""
    d, Hkv = case.d, case.Hkv
    v = np.zeros((T, Hkv, d), dtype=np.uint16)
    pos, ch = tile_code_rows
    v[pos, :, ch] = ONE
    for h in range(Hkv):
        v[:, h, d - 1] = _bits(float(id_code(b, h, Hkv)))
    return v


def counting_inputs(case: Case) -> Case:
    """Zero queries, indicator-coded values (see the module docstring)."""
    assert case.dtype == "bf16"
    d = case.d
    npc = n_prefix_channels(d)
    c = copy.copy(case)
    c.q = np.zeros_like(case.q)
    ks, vs = [], []
    for b in range(case.B):
        P, n = int(case.prefix_len[b]), int(case.n_nodes[b])
        T = P + n
        t = np.arange(T)
        k = np.zeros((T, case.Hkv, d), dtype=np.uint16)
        k[t, :, t % d] = ONE
        ks.append(k)
        ch = np.where(t < P, (t // TILE) % npc, npc + ((t - P) % TREE_CODES))
        vs.append(_value_codes(case, b, T, P, (t, ch)))
    c.k = _logical_to_storage(case, ks, "k")
    c.v = _logical_to_storage(case, vs, "v")
    c.name = case.name + "_counting"
    c.planted = dict(case.planted, id_codes=np.array(
        [[id_code(b, h, case.Hkv) for h in range(case.Hkv)] for b in range(case.B)]))
    return c


def needle_inputs(case: Case, seed: int) -> Case:
    """One needle per prefix tile and per tree node (see the module docstring)."""
    assert case.dtype == "bf16"
    d, Hkv, G = case.d, case.Hkv, case.G
    npc = n_prefix_channels(d)
    rng = np.random.default_rng([seed, 77])
    c = copy.copy(case)
    u = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=(case.B, Hkv, d))
    alpha = (12 + rng.integers(0, 9, size=case.q.shape[:3])).astype(np.float32) / 16.0
    q = alpha[..., None] * u[:, None, np.repeat(np.arange(Hkv), G), :]
    c.q = bf16_bits_from_f32(q.astype(np.float32)).reshape(case.q.shape)
    ks, vs = [], []
    needles = []
    for b in range(case.B):
        P, n = int(case.prefix_len[b]), int(case.n_nodes[b])
        T = P + n
        ntile = (P + TILE - 1) // TILE
        k = np.zeros((T, Hkv, d), dtype=np.uint16)
        pos_all, ch_all = [], []
        for h in range(Hkv):
            span = np.minimum(TILE, P - TILE * np.arange(ntile))
            off = (rng.random(ntile) * span).astype(np.int64)
            pos = TILE * np.arange(ntile) + off
            beta = (38 + rng.integers(0, 7, size=ntile + n)).astype(np.float32) / 64.0
            rows = np.r_[pos, P + np.arange(n)]
            k[rows, h, :] = bf16_bits_from_f32(beta[:, None] * u[b, h][None, :])
            pos_all.append(rows)
            ch_all.append(np.r_[np.arange(ntile) % npc, npc + np.arange(n) % TREE_CODES])
        needles.append(pos_all)
        ks.append(k)
        v = np.zeros((T, Hkv, d), dtype=np.uint16)
        for h in range(Hkv):
            v[pos_all[h], h, ch_all[h]] = ONE
            v[:, h, d - 1] = _bits(float(id_code(b, h, Hkv)))
        vs.append(v)
    c.k = _logical_to_storage(case, ks, "k")
    c.v = _logical_to_storage(case, vs, "v")
    c.name = case.name + "_needles"
    c.planted = dict(case.planted, needles=needles)
    return c
