"""Pins for the re-root / compaction oracle.

* Figure 4 of the SwiftSpec summary (Section 3.2): exact post-re-root layout
  for every parent array consistent with the caption.
* Figure 2 (Section 3.1.2): the keep and the out-of-tree cases.
* The collapse walkthrough (critique section): repeated out-of-tree tokens.
* Invariants: a chain moves nothing; topological order, moved multiset,
  token positions; re-rooting twice equals once along the joined path.
"""
import itertools

import numpy as np
import pytest

import oracle
from gen import random_case


def _pattern_kv(B, T, Hkv=2, d=4):
    """KV rows that name their own (sequence, position): row value = 1000*b + t."""
    k = np.zeros((B, T, Hkv, d), dtype=np.float32)
    for b in range(B):
        for t in range(T):
            k[b, t] = 1000 * b + t
    return k, -k


def _fig4_parents(fx):
    toks = fx["tree_tokens"]
    idx = {t: i for i, t in enumerate(toks)}
    choices = []
    for i, t in enumerate(toks):
        if t in fx["fixed_parent"]:
            p = fx["fixed_parent"][t]
            choices.append([-1] if p == "root" else [idx[p]])
        else:
            choices.append(list(range(-1, i)))
    out = []
    for p in itertools.product(*choices):
        p = np.array(p, dtype=np.int32)
        under = oracle.descendants(p, idx["t15"], len(toks))
        if any(idx[t] in under for t in fx["not_under_t15"]):
            continue
        out.append(p)
    return out


def test_fig4_reroot_layout(golden):
    fx = golden("fig4_reroot.json")
    toks = fx["tree_tokens"]
    idx = {t: i for i, t in enumerate(toks)}
    P = len(fx["prefix_tokens"])
    n = len(toks)
    parents = _fig4_parents(fx)
    assert len(parents) == 60
    for par in parents:
        k, v = _pattern_kv(1, P + n + 4)
        path = np.full((1, n), -1, dtype=np.int32)
        path[0, :2] = [idx[t] for t in fx["path"]]
        layers, P1, par1, n1 = oracle.tree_cache_reroot(
            [(k, v)], np.array([P]), par[None], np.array([n]), path, np.array([2]),
            np.array([fx["keep"]]))
        k1, v1 = layers[0]
        assert P1[0] == fx["expected_prefix_len"]
        assert n1[0] == fx["expected_n_nodes"]
        assert par1[0, :2].tolist() == fx["expected_parent"]
        assert (par1[0, 2:] == -1).all()
        for row, tname in fx["expected_rows"].items():
            old = P + idx[tname]
            assert old == fx["expected_rows_old_position"][row]
            np.testing.assert_array_equal(k1[0, int(row)], k[0, old])
            np.testing.assert_array_equal(v1[0, int(row)], v[0, old])
        np.testing.assert_array_equal(k1[0, :P], k[0, :P])    # the prefix never moves


def test_fig2_keep_then_out_of_tree(golden):
    fx = golden("fig2_iterations.json")
    toks = fx["tree_tokens"]
    idx = {t: i for i, t in enumerate(toks)}
    n = len(toks)
    rng = np.random.default_rng(2)
    under = sorted(idx[t] for t in fx["under_t6"])
    checked = 0
    while checked < 200:
        par = np.array([rng.integers(-1, i) if i else -1 for i in range(n)], dtype=np.int32)
        par[idx["t3"]] = -1
        par[idx["t6"]] = idx["t3"]
        for u in under:                   # hang t9..t12 under t6 or under each other
            par[u] = rng.choice([idx["t6"]] + [x for x in under if x < u])
        if oracle.descendants(par, idx["t6"], n) != under:
            continue
        checked += 1
        P = 5
        k, v = _pattern_kv(1, P + n)
        path = np.full((1, n), -1, dtype=np.int32)
        path[0, :2] = [idx[t] for t in fx["iter1"]["path"]]
        layers, P1, par1, n1 = oracle.tree_cache_reroot(
            [(k, v)], np.array([P]), par[None], np.array([n]), path, np.array([2]),
            np.array([True]))
        assert P1[0] == P + fx["iter1"]["prefix_growth"]
        assert n1[0] == len(fx["iter1"]["expected_tree"])
        k1 = layers[0][0]
        for r, t in enumerate(fx["iter1"]["expected_tree"]):
            np.testing.assert_array_equal(k1[0, P1[0] + r], k[0, P + idx[t]])
        # iteration 2: t9 verified, the target's next token t16 is outside the tree
        t9_new = fx["iter1"]["expected_tree"].index("t9")
        assert par1[0, t9_new] == -1
        path2 = np.full((1, n), -1, dtype=np.int32)
        path2[0, 0] = t9_new
        layers2, P2, par2, n2 = oracle.tree_cache_reroot(
            layers, P1, par1, n1, path2, np.array([1]), np.array([fx["iter2"]["keep"]]))
        assert n2[0] == fx["iter2"]["expected_n_nodes"]
        assert P2[0] == P1[0] + fx["iter2"]["prefix_growth"]
        np.testing.assert_array_equal(layers2[0][0][0, P1[0]], k[0, P + idx["t9"]])


def test_collapse_walkthrough(golden):
    fx = golden("collapse_walkthrough.json")
    n = fx["tree_nodes_per_step"]
    P = 10
    k, v = _pattern_kv(1, P + 3 * n + 2)
    layers = [(k, v)]
    Pc = np.array([P])
    rng = np.random.default_rng(5)
    for step in range(fx["steps"]):
        par = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, n)]], dtype=np.int32)
        path = np.full((1, n), -1, dtype=np.int32)
        path[0, 0] = 0                        # only the root token is verified
        layers, P2, par2, n2 = oracle.tree_cache_reroot(layers, Pc, par, np.array([n]), path,
                                                        np.array([1]), np.array([False]))
        assert n2[0] == fx["expected_n_nodes_after_each_step"]
        assert P2[0] - Pc[0] == fx["expected_prefix_growth_per_step"]
        Pc = P2


def test_chain_reroot_moves_nothing():
    c = random_case(21, B=4, Hq=2, Hkv=2, d=8, P_range=(0, 30), n_max=9, n_range=(1, 9),
                    dtype="bf16", chain=True, target_side=True)
    L = np.array([int(np.random.default_rng(b).integers(1, c.n_nodes[b] + 1)) for b in range(4)])
    path = np.full((4, 9), -1, dtype=np.int32)
    for b in range(4):
        path[b, : L[b]] = np.arange(L[b])
    layers, P1, par1, n1 = oracle.tree_cache_reroot([(c.k, c.v)], c.prefix_len, c.parent,
                                                    c.n_nodes, path, L, np.zeros(4, bool))
    np.testing.assert_array_equal(layers[0][0], c.k)
    np.testing.assert_array_equal(layers[0][1], c.v)
    np.testing.assert_array_equal(P1, c.prefix_len + L)
    assert (n1 == 0).all() and (par1 == -1).all()


def _depths(parent, n):
    dep = np.zeros(n, dtype=np.int64)
    for i in range(n):
        dep[i] = 1 + (dep[parent[i]] if parent[i] >= 0 else 0)
    return dep


@pytest.mark.parametrize("seed", range(25))
def test_invariants_random_trees(seed):
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(1, 20))
    P = int(rng.integers(0, 9))
    par = np.array([rng.integers(-1, i) if i else -1 for i in range(n)], dtype=np.int32)
    end = int(rng.integers(0, n))
    full = oracle.root_path(par, end)
    k, v = _pattern_kv(1, P + n)
    for keep in (False, True):
        for cut in range(0, len(full) + 1):
            path = np.full((1, n), -1, dtype=np.int32)
            path[0, :cut] = full[:cut]
            layers, P1, par1, n1 = oracle.tree_cache_reroot(
                [(k, v)], np.array([P]), par[None], np.array([n]), path, np.array([cut]),
                np.array([keep]))
            k1 = layers[0][0]
            m = int(n1[0])
            if cut == 0 and keep:
                assert P1[0] == P and m == n
                np.testing.assert_array_equal(par1[0, :n], par)
                continue
            assert P1[0] == P + cut
            assert oracle.is_valid_parent(par1[0], m)
            # moved rows: promoted path then the subtree under its last node
            src = [int(x) - P for x in k1[0, P: P + cut + m, 0, 0]]
            kept = [u for u in range(n) if keep and cut > 0 and
                    full[cut - 1] in oracle.ancestors(par, u)]
            assert src == full[:cut] + kept
            # every kept token keeps its position P - 1 + depth
            d_old, d_new = _depths(par, n), _depths(par1[0], m)
            for r, u in enumerate(kept):
                assert P1[0] - 1 + d_new[r] == P - 1 + d_old[u]
            if keep and 0 < cut < len(full):
                # re-rooting again along the rest of the path == re-rooting once
                rest = [kept.index(x) for x in full[cut:]]
                p2 = np.full((1, n), -1, dtype=np.int32)
                p2[0, : len(rest)] = rest
                l2, P2, par2, n2 = oracle.tree_cache_reroot(layers, P1, par1, n1, p2,
                                                            np.array([len(rest)]),
                                                            np.array([True]))
                p3 = np.full((1, n), -1, dtype=np.int32)
                p3[0, : len(full)] = full
                l3, P3, par3, n3 = oracle.tree_cache_reroot([(k, v)], np.array([P]), par[None],
                                                            np.array([n]), p3,
                                                            np.array([len(full)]),
                                                            np.array([True]))
                assert P2[0] == P3[0] and n2[0] == n3[0]
                np.testing.assert_array_equal(par2, par3)
                e = P3[0] + n3[0]
                np.testing.assert_array_equal(l2[0][0][0, :e], l3[0][0][0, :e])


def test_paged_reroot_moves_through_block_table():
    c = random_case(31, B=2, Hq=2, Hkv=1, d=4, P_range=(14, 40), n_max=12, n_range=(8, 12),
                    dtype="f32", paged=True, block_size=8)
    cc = random_case(31, B=2, Hq=2, Hkv=1, d=4, P_range=(14, 40), n_max=12, n_range=(8, 12),
                     dtype="f32")
    np.testing.assert_array_equal(c.parent, cc.parent)
    path = np.full((2, 12), -1, dtype=np.int32)
    L = np.zeros(2, dtype=np.int32)
    for b in range(2):
        rp = oracle.root_path(c.parent[b], int(c.n_nodes[b]) - 1)
        path[b, : len(rp)] = rp
        L[b] = len(rp)
    keep = np.array([True, True])
    lp, P1, par1, n1 = oracle.tree_cache_reroot([(c.k, c.v)], c.prefix_len, c.parent, c.n_nodes,
                                                path, L, keep, c.block_table, c.block_size)
    # compare with the contiguous view of the same paged cache
    for b in range(2):
        T = int(c.prefix_len[b] + c.n_nodes[b])
        ks, _ = oracle.gather_sequence_kv(c.k, c.v, b, T, "f32", c.block_table, c.block_size)
        kc = ks[None].astype(np.float32)
        lc, P2, par2, n2 = oracle.tree_cache_reroot([(kc, kc)], c.prefix_len[b:b + 1],
                                                    c.parent[b:b + 1], c.n_nodes[b:b + 1],
                                                    path[b:b + 1], L[b:b + 1], keep[b:b + 1])
        e = int(P2[0] + n2[0])
        k1, _ = oracle.gather_sequence_kv(lp[0][0], lp[0][1], b, e, "f32", c.block_table,
                                          c.block_size)
        np.testing.assert_array_equal(k1, lc[0][0][0, :e].astype(np.float64))
