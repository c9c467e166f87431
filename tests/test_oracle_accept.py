"""Pins for the greedy acceptance oracle.

The oracle enumerates every node's root path.  These tests check it against
the textbook verification loop (walk down from the root, following the child
whose token is the target's greedy choice, stop at the first mismatch -- the
draft-length co-design article's description), on every parent array of up
to 6 nodes, against the acceptance-length bound 1 <= AL <= 1 + D, and against
the planted paths of the seeded workloads.
"""
import itertools

import numpy as np
import pytest

import oracle
from gen import config1_tiny, random_case
from gen.workloads import _chain_case


def _greedy_walk(parent, tok, n, root_tok, a):
    """Sequential speculative-decoding check, one level at a time."""
    cur, expected, path = -1, int(root_tok), []
    while True:
        nxt = [c for c in range(n) if int(parent[c]) == cur and int(tok[c]) == expected]
        if not nxt:
            break
        assert len(nxt) == 1  # sibling tokens are distinct
        cur = nxt[0]
        path.append(cur)
        expected = a[cur]
    return path, expected


def _all_parent_arrays(n, target_side):
    rng = [[-1]] + [list(range(0 if target_side else -1, i)) for i in range(1, n)]
    for p in itertools.product(*rng):
        yield np.array(p, dtype=np.int32)


@pytest.mark.parametrize("n,target_side", [(1, False), (2, False), (3, False), (4, False),
                                           (5, False), (6, True), (5, True)])
def test_exhaustive_small_trees_match_greedy_walk(n, target_side):
    rng = np.random.default_rng(n * 10 + target_side)
    vocab = 8
    count = 0
    for parent in _all_parent_arrays(n, target_side):
        for rep in range(3):
            tok = np.empty(n, dtype=np.int32)
            for p in np.unique(parent):
                idx = np.nonzero(parent == p)[0]
                tok[idx] = rng.choice(vocab, size=idx.size, replace=False)
            logits = rng.standard_normal((n, vocab)).astype(np.float32)
            # bias each row toward one of its children's tokens most of the time
            for i in range(n):
                kids = np.nonzero(parent == i)[0]
                if kids.size and rng.random() < 0.8:
                    logits[i, tok[rng.choice(kids)]] = 5.0
            roots = np.nonzero(parent == -1)[0]
            root_tok = tok[0] if target_side else (tok[rng.choice(roots)] if rng.random() < 0.85
                                                   else vocab - 1 - rep)
            a = [int(np.argmax(logits[i])) for i in range(n)]
            path, bonus = _greedy_walk(parent, tok, n, root_tok, a)
            po, pl, bo = oracle.accept_greedy_path(logits[None], parent[None], tok[None],
                                                   np.array([n]), np.array([root_tok]))
            assert pl[0] == len(path)
            assert po[0, : pl[0]].tolist() == path
            assert (po[0, pl[0]:] == -1).all()
            assert bo[0] == bonus
            if target_side:
                assert 1 <= pl[0] <= n
            count += 1
    assert count > 0


@pytest.mark.parametrize("D,seed", [(1, 0), (5, 1), (15, 2), (15, 3), (9, 4)])
def test_chain_first_mismatch_and_al_bound(D, seed):
    rng = np.random.default_rng(seed)
    B, vocab = 64, 6
    n = D + 1
    parent = np.tile(np.arange(-1, n - 1, dtype=np.int32), (B, 1))
    tok = rng.integers(0, vocab, size=(B, n)).astype(np.int32)
    logits = rng.standard_normal((B, n, vocab)).astype(np.float32)
    for b in range(B):
        for j in range(n - 1):
            if rng.random() < 0.7:
                logits[b, j, tok[b, j + 1]] = 4.0
    po, pl, bo = oracle.accept_greedy_path(logits, parent, tok, np.full(B, n), tok[:, 0])
    for b in range(B):
        a = logits[b].argmax(axis=1)
        m = 0
        while m < D and tok[b, m + 1] == a[m]:
            m += 1
        assert pl[b] == 1 + m                     # AL = accepted drafts + 1
        assert 1 <= pl[b] <= 1 + D
        assert po[b, : pl[b]].tolist() == list(range(1 + m))
        assert bo[b] == a[m]


def test_planted_geometric_matches_are_recovered():
    c = _chain_case("small_chain", 9, 24, 2, 1, 8, 5, 15, 300)
    po, pl, bo = oracle.accept_greedy_path(c.logits, c.parent, c.tok, c.n_nodes, c.root_tok)
    assert pl.tolist() == c.planted["path_len"]
    assert (pl >= 1).all() and (pl <= 16).all()


def test_planted_forest_path_is_recovered():
    c = config1_tiny()
    po, pl, bo = oracle.accept_greedy_path(c.logits, c.parent, c.tok, c.n_nodes, c.root_tok)
    assert pl[0] == c.planted["path_len"][0]
    assert po[0, pl[0] - 1] == c.planted["end"][0]
    for seed in range(20):
        r = random_case(seed, B=4, Hq=1, Hkv=1, d=4, P_range=(0, 3), n_max=12, dtype="f32")
        _, pl, _ = oracle.accept_greedy_path(r.logits, r.parent, r.tok, r.n_nodes, r.root_tok)
        assert pl.tolist() == r.planted["path_len"]


def test_argmax_ties_take_lowest_index():
    row = np.array([0.5, 1.0, -2.0, 3.0, 0.0, 0.0, 0.0, 3.0], dtype=np.float32)
    assert oracle.argmax_first(row) == 3
    logits = np.zeros((1, 2, 8), dtype=np.float32)
    logits[0, 0] = row
    parent = np.array([[-1, 0]], dtype=np.int32)
    tok = np.array([[5, 3]], dtype=np.int32)
    po, pl, bo = oracle.accept_greedy_path(logits, parent, tok, np.array([2]), np.array([5]))
    assert pl[0] == 2 and bo[0] == 0          # row 1 is all zeros: first index
    tok[0, 1] = 7                              # the other maximum does not count
    po, pl, bo = oracle.accept_greedy_path(logits, parent, tok, np.array([2]), np.array([5]))
    assert pl[0] == 1 and bo[0] == 3


def test_duplicate_siblings_take_deepest_then_lowest_index():
    # root -> {0: tok 4, 1: tok 4}; 1 -> 2 (tok 6); a[1] = 6 so node 2 is accepted
    vocab = 8
    parent = np.array([[-1, -1, 1, 0]], dtype=np.int32)
    tok = np.array([[4, 4, 6, 6]], dtype=np.int32)
    logits = np.zeros((1, 4, vocab), dtype=np.float32)
    logits[0, 1, 6] = 1.0
    logits[0, 0, 1] = 1.0
    po, pl, bo = oracle.accept_greedy_path(logits, parent, tok, np.array([4]), np.array([4]))
    assert pl[0] == 2 and po[0, :2].tolist() == [1, 2]
    # both branches reach depth 2 (node 2 under node 1, node 3 under node 0):
    # the lower node index, node 2, wins
    logits[0, 0, 6] = 2.0
    po, pl, bo = oracle.accept_greedy_path(logits, parent, tok, np.array([4]), np.array([4]))
    assert pl[0] == 2 and po[0, :2].tolist() == [1, 2]
    # equal depth 1 only (no grandchildren accepted): lowest index among {0, 1}
    logits[0, 0, 6] = 0.0
    logits[0, 1, 6] = 0.0
    po, pl, bo = oracle.accept_greedy_path(logits, parent, tok, np.array([4]), np.array([4]))
    assert pl[0] == 1 and po[0, 0] == 0


def test_nothing_accepted_gives_root_token_bonus():
    parent = np.array([[-1, 0, -1]], dtype=np.int32)
    tok = np.array([[1, 2, 3]], dtype=np.int32)
    logits = np.zeros((1, 3, 4), dtype=np.float32)
    po, pl, bo = oracle.accept_greedy_path(logits, parent, tok, np.array([3]), np.array([0]))
    assert pl[0] == 0 and bo[0] == 0 and (po == -1).all()
    po, pl, bo = oracle.accept_greedy_path(logits, parent, tok, np.array([0]), np.array([2]))
    assert pl[0] == 0 and bo[0] == 2
