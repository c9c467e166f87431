"""Pins for the draft-side oracle (oracle/draft.py).

* Figure 2 of the SwiftSpec summary (Section 3.1.2): the walk along (t3, t6)
  re-roots at t6 and keeps its subtree; after that re-root the walk along
  (t9, t16) stops at t9 because t16 is not in the tree.
* The walk along the tokens of any node's root path returns that path, one
  more token that is a child's extends it, one that is not ends it.
* The chosen subtree maximises the expected accepted tokens, the sum of
  exp(cum) over its nodes, among all subtrees of bs nodes (exhaustive search
  on small trees), and is always a valid tree.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle.topw import log_softmax


def _tok_id(name):
    return int(name[1:])


def test_fig2_token_walk_then_reroot(golden):
    fx = golden("fig2_iterations.json")
    toks = fx["tree_tokens"]
    idx = {t: i for i, t in enumerate(toks)}
    n = len(toks)
    tok = np.array([_tok_id(t) for t in toks], dtype=np.int32)
    rng = np.random.default_rng(5)
    under = sorted(idx[t] for t in fx["under_t6"])
    checked = 0
    while checked < 100:
        par = np.array([rng.integers(-1, i) if i else -1 for i in range(n)], dtype=np.int32)
        par[idx["t3"]] = -1
        par[idx["t6"]] = idx["t3"]
        for u in under:
            par[u] = rng.choice([idx["t6"]] + [x for x in under if x < u])
        if oracle.descendants(par, idx["t6"], n) != under:
            continue
        # sibling tokens must differ for a walk to be unambiguous
        sib = {}
        if any(sib.setdefault((int(par[c]), int(tok[c])), c) != c for c in range(n)):
            continue
        checked += 1
        path, keep = oracle.token_walk(par, tok, n, [_tok_id(t) for t in fx["iter1"]["path"]])
        assert path == [idx[t] for t in fx["iter1"]["path"]] and keep == fx["iter1"]["keep"]
        P = 5
        k = np.zeros((1, P + n, 1, 2), dtype=np.float32)
        pth = np.full((1, n), -1, dtype=np.int32)
        pth[0, :len(path)] = path
        _, P1, par1, n1 = oracle.tree_cache_reroot([(k, k)], np.array([P]), par[None],
                                                    np.array([n]), pth, np.array([len(path)]),
                                                    np.array([keep]))
        tok1 = np.array([_tok_id(t) for t in fx["iter1"]["expected_tree"]], dtype=np.int32)
        path2, keep2 = oracle.token_walk(par1[0], tok1, int(n1[0]), [9, 16])
        assert [fx["iter1"]["expected_tree"][i] for i in path2] == fx["iter2"]["path"]
        assert keep2 == fx["iter2"]["keep"]


def _random_tree(rng, n, V=6):
    par = np.array([rng.integers(-1, i) if i else -1 for i in range(n)], dtype=np.int32)
    tok = np.zeros(n, dtype=np.int32)
    for i in range(n):
        used = {int(tok[c]) for c in range(i) if par[c] == par[i]}
        tok[i] = rng.choice([t for t in range(V + n) if t not in used])
    return par, tok


@pytest.mark.parametrize("seed", range(6))
def test_walk_recovers_every_root_path(seed):
    rng = np.random.default_rng([seed, 40])
    n = int(rng.integers(1, 14))
    par, tok = _random_tree(rng, n)
    assert oracle.token_walk(par, tok, n, []) == ([], True)
    for x in range(n):
        rp = oracle.root_path(par, x)
        assert oracle.token_walk(par, tok, n, [int(tok[v]) for v in rp]) == (rp, True)
        kids = [c for c in range(n) if par[c] == x]
        absent = max(int(t) for t in tok) + 1
        assert oracle.token_walk(par, tok, n, [int(tok[v]) for v in rp] + [absent]) == (rp, False)
        for c in kids:
            assert oracle.token_walk(par, tok, n, [int(tok[v]) for v in rp] + [int(tok[c])]) == \
                (rp + [c], True)
    # a first token that no child of the root carries: nothing matches
    assert oracle.token_walk(par, tok, n, [10 ** 6, int(tok[0])]) == ([], False)


def test_walk_duplicate_siblings_follow_lowest_index():
    par = np.array([-1, -1, 1, 0], dtype=np.int32)
    tok = np.array([7, 7, 3, 3], dtype=np.int32)
    assert oracle.token_walk(par, tok, 4, [7, 3]) == ([0, 3], True)


def _closed_subsets(par, n, bs):
    for sub in itertools.combinations(range(n), bs):
        s = set(sub)
        if all(par[v] < 0 or int(par[v]) in s for v in sub):
            yield sub


@pytest.mark.parametrize("seed", range(8))
def test_select_is_the_best_subtree(seed):
    rng = np.random.default_rng([seed, 41])
    n = int(rng.integers(2, 10))
    par, tok = _random_tree(rng, n)
    V = int(tok.max()) + 1
    lg = rng.standard_normal((n + 1, V))
    cum = oracle.cumulative_scores(par, tok, lg[0], lg[1:], n)
    assert all(par[i] < 0 or cum[i] <= cum[par[i]] + 1e-15 for i in range(n))
    for bs in range(1, n + 1):
        best = max(_closed_subsets(par, n, bs), key=lambda s: sum(np.exp(cum[list(s)])))
        nodes, new_par, toks = oracle.select_subtree(par, tok, cum, n, bs)
        assert nodes.tolist() == list(best)
        for k, v in enumerate(nodes):
            p = int(par[v])
            assert new_par[k] == (-1 if p < 0 else nodes.tolist().index(p))
            assert new_par[k] < k and toks[k] == tok[v]


def test_select_ties_stay_a_subtree():
    """All-equal logits: cum depends on depth only; the choice fills the
    shallow levels first, lowest indices first, and stays closed."""
    rng = np.random.default_rng(42)
    for _ in range(20):
        n = int(rng.integers(2, 30))
        par, tok = _random_tree(rng, n)
        V = int(tok.max()) + 1
        cum = oracle.cumulative_scores(par, tok, np.zeros(V), np.zeros((n, V)), n)
        for bs in (1, n // 2, n):
            nodes, new_par, _ = oracle.select_subtree(par, tok, cum, n, bs)
            s = set(nodes.tolist())
            assert all(par[v] < 0 or int(par[v]) in s for v in s)
            depth = {v: oracle.depth(par, v) for v in range(n)}
            cut = max(depth[v] for v in s)
            # shallower levels complete, the last level filled from its lowest indices
            assert all(depth[v] >= cut for v in range(n) if v not in s)
            last = sorted(v for v in range(n) if depth[v] == cut)
            assert sorted(v for v in s if depth[v] == cut) == last[:len([v for v in s if depth[v] == cut])]


def test_fig2_reroot_moves_tokens_with_the_nodes(golden):
    """Figure 2, iteration 1: after re-rooting at t6 the draft's next tree is
    t9..t12 (their tokens in that order); iteration 2: t16 is outside the
    tree, nothing is kept."""
    fx = golden("fig2_iterations.json")
    toks = fx["tree_tokens"]
    idx = {t: i for i, t in enumerate(toks)}
    n = len(toks)
    par = np.full(n, -1, dtype=np.int32)
    par[idx["t6"]] = idx["t3"]
    for t in fx["under_t6"]:
        par[idx[t]] = idx["t6"]
    tok = np.array([_tok_id(t) for t in toks], dtype=np.int32)
    path = [idx[t] for t in fx["iter1"]["path"]]
    tok1, _ = oracle.reroot_node_arrays(par, n, path, len(path), True, tok)
    m = len(fx["iter1"]["expected_tree"])
    assert tok1[:m].tolist() == [_tok_id(t) for t in fx["iter1"]["expected_tree"]]
    assert (tok1[m:] == -1).all()
    _, _, par1, n1 = oracle.tree_cache_reroot([], np.array([5]), par[None], np.array([n]),
                                              np.array([path + [-1] * (n - 2)]),
                                              np.array([2]), np.array([True]))
    p2, keep2 = oracle.token_walk(par1[0], tok1, int(n1[0]), [9, 16])
    tok2, _ = oracle.reroot_node_arrays(par1[0], int(n1[0]), p2, len(p2), keep2, tok1)
    assert keep2 is False and (tok2 == -1).all()


@pytest.mark.parametrize("seed", range(10))
def test_reroot_rebases_weights_to_the_new_root(seed):
    """Re-rooting commutes with the definition of the weights: the weights of
    the re-rooted tree, computed from scratch with the new root's own
    distribution (the old row of the last verified node) and the kept nodes'
    rows in their new order, equal the re-based, moved weights."""
    rng = np.random.default_rng(300 + seed)
    n, V = int(rng.integers(2, 14)), 7
    par, tok = _random_tree(rng, n, V)
    root_row = rng.standard_normal(V + n)
    rows = rng.standard_normal((n, V + n))
    cum = oracle.cumulative_scores(par, tok, root_row, rows, n).astype(np.float32)
    end = int(rng.integers(0, n))
    path = oracle.root_path(par, end)
    k = int(rng.integers(1, len(path) + 1))
    tok2, cum2 = oracle.reroot_node_arrays(par, n, path, k, True, tok, cum)
    _, _, par2, n2 = oracle.tree_cache_reroot([], np.array([0]), par[None], np.array([n]),
                                              np.array([path + [-1] * (n - len(path))]),
                                              np.array([k]), np.array([True]))
    n2 = int(n2[0])
    kept = oracle.descendants(par, path[k - 1], n)
    assert n2 == len(kept) and tok2[:n2].tolist() == [int(tok[u]) for u in kept]
    fresh = oracle.cumulative_scores(par2[0], tok2, rows[path[k - 1]], rows[kept], n2)
    np.testing.assert_allclose(cum2[:n2], fresh, rtol=2e-6, atol=2e-6)
    assert np.all(np.isneginf(cum2[n2:])) and np.all(tok2[n2:] == -1)
    # dropping the tree (no keep) leaves nothing; k = 0 with keep changes nothing
    t3, c3 = oracle.reroot_node_arrays(par, n, path, k, False, tok, cum)
    assert (t3 == -1).all() and np.all(np.isneginf(c3))
    t4, c4 = oracle.reroot_node_arrays(par, n, path, 0, True, tok, cum)
    assert np.array_equal(t4, tok) and np.array_equal(c4, cum)
