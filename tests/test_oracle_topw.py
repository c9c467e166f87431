"""Pins for the top-w maximum-likelihood candidate selection (host side of the
draft expansion rounds): closed forms and order properties."""
import numpy as np
import pytest

import oracle
from gen import config4_expand


def _tree(rng, n, vocab):
    par = np.array([rng.integers(-1, i) if i else -1 for i in range(n)], dtype=np.int32)
    tok = np.empty(n, dtype=np.int32)
    for p in np.unique(par):
        idx = np.nonzero(par == p)[0]
        tok[idx] = rng.choice(vocab, size=idx.size, replace=False)
    return par, tok


def test_uniform_logits_closed_form():
    rng = np.random.default_rng(1)
    vocab, n = 16, 6
    par, tok = _tree(rng, n, vocab)
    root = np.zeros(vocab)
    rows = np.zeros((n, vocab))
    cum = oracle.cumulative_scores(par, tok, root, rows, n)
    dep = np.zeros(n)
    for i in range(n):
        dep[i] = 1 + (dep[par[i]] if par[i] >= 0 else 0)
    np.testing.assert_allclose(cum, -dep * np.log(vocab), rtol=1e-13)
    # all scores of the root's candidates are -log V, the best possible: the
    # w picks are the root's free tokens in increasing order
    p, t, s = oracle.select_top_w(par, tok, cum, root, rows, n, 5)
    taken = set(tok[par == -1].tolist())
    assert p.tolist() == [-1] * 5
    assert t.tolist() == [x for x in range(vocab) if x not in taken][:5]
    np.testing.assert_allclose(s, -np.log(vocab))


@pytest.mark.parametrize("seed", range(8))
def test_selection_order_properties(seed):
    rng = np.random.default_rng(10 + seed)
    vocab, n, w = 12, int(rng.integers(1, 9)), 8
    par, tok = _tree(rng, n, vocab)
    root = rng.standard_normal(vocab)
    rows = rng.standard_normal((n, vocab))
    cum = oracle.cumulative_scores(par, tok, root, rows, n)
    p, t, s = oracle.select_top_w(par, tok, cum, root, rows, n, w)
    # no pick duplicates an existing child or another pick
    existing = {(int(par[i]), int(tok[i])) for i in range(n)}
    picks = list(zip(p.tolist(), t.tolist()))
    assert len(set(picks)) == w and not (set(picks) & existing)
    # scores are non-increasing and no unpicked candidate beats the last pick
    assert (np.diff(s) <= 0).all()
    def lsm(x):
        return x - np.log(np.exp(x - x.max()).sum()) - x.max()
    for pp in range(-1, n):
        base = 0.0 if pp < 0 else cum[pp]
        sc = base + lsm(root if pp < 0 else rows[pp])
        for tt in range(vocab):
            if (pp, tt) in existing or (pp, tt) in picks:
                continue
            assert sc[tt] <= s[-1] + 1e-12
    # adding a constant to any logits row changes nothing (softmax shift)
    p2, t2, s2 = oracle.select_top_w(par, tok, oracle.cumulative_scores(par, tok, root + 3.0,
                                                                        rows - 7.5, n),
                                     root + 3.0, rows - 7.5, n, w)
    assert p2.tolist() == p.tolist() and t2.tolist() == t.tolist()
    np.testing.assert_allclose(s2, s, rtol=1e-11, atol=1e-11)


def test_ties_prefer_lower_parent_then_token():
    vocab = 4
    par = np.array([-1], dtype=np.int32)
    tok = np.array([0], dtype=np.int32)
    root = np.zeros(vocab)
    rows = np.array([[np.log(4.0) + 0.0] * vocab])  # node 0's children score cum(0) - log 4
    cum = oracle.cumulative_scores(par, tok, root, rows, 1)
    p, t, s = oracle.select_top_w(par, tok, cum, root, rows, 1, 5)
    # root candidates (tokens 1,2,3) score -log4; node-0 candidates score -2 log4
    assert p.tolist() == [-1, -1, -1, 0, 0] and t.tolist() == [1, 2, 3, 0, 1]


def test_expand_workload_rounds_are_well_formed():
    c = config4_expand()
    par = c.parent0.copy()
    tok = c.tok0.copy()
    rows = c.logits0.copy()
    n = c.n0
    for r in range(c.rounds):
        cum = oracle.cumulative_scores(par, tok, c.logits_root, rows, n)
        p, t, s = oracle.select_top_w(par, tok, cum, c.logits_root, rows, n, c.w)
        par = np.r_[par, p]
        tok = np.r_[tok, t]
        rows = np.r_[rows, c.logits_new[r]]
        n += c.w
        assert oracle.is_valid_parent(par, n)
    assert n == c.n_max


def test_cumulative_scores_hand_example():
    """A node's weight adds the log-probability of its token under its
    PARENT's distribution (SwiftSpec summary, Section 3.1.3, maximum-likelihood
    expansion).  Every row is a different distribution, written as the logs of
    hand-picked probabilities, so reading a node's own row, a sibling's row or
    the wrong token gives a different number."""
    root = np.log([0.5, 0.25, 0.25])
    rows = np.log([[0.1, 0.6, 0.3],     # after node 0
                   [0.2, 0.2, 0.6],     # after node 1
                   [0.7, 0.2, 0.1],     # after node 2
                   [0.05, 0.9, 0.05]])  # after node 3
    par = np.array([-1, 0, 1, 0], dtype=np.int32)
    tok = np.array([1, 2, 0, 0], dtype=np.int32)
    cum = oracle.cumulative_scores(par, tok, root, rows, 4)
    # node 0: root's p(1) = 0.25; node 1: then node 0's p(2) = 0.3;
    # node 2: then node 1's p(0) = 0.2; node 3 (node 0's child): node 0's p(0) = 0.1
    expect = np.log([0.25, 0.25 * 0.3, 0.25 * 0.3 * 0.2, 0.25 * 0.1])
    np.testing.assert_allclose(cum, expect, rtol=1e-14, atol=1e-14)
    # unnormalised rows give the same weights (the log-softmax normalises)
    cum2 = oracle.cumulative_scores(par, tok, root + 2.0, rows - 1.5, 4)
    np.testing.assert_allclose(cum2, expect, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_grown_tree_weights_equal_selection_scores(seed):
    """The score select_top_w reports for a new leaf is the weight that leaf
    has in the grown tree: cumulative_scores of the tree with the picks
    appended reproduces it (the two functions compute the same definition
    from different ends: per candidate, and per node of the result)."""
    rng = np.random.default_rng(40 + seed)
    vocab, n, w = 9, int(rng.integers(1, 7)), 5
    par, tok = _tree(rng, n, vocab)
    root = rng.standard_normal(vocab) * 2.0
    rows = rng.standard_normal((n + w, vocab)) * 2.0
    cum = oracle.cumulative_scores(par, tok, root, rows, n)
    p, t, s = oracle.select_top_w(par, tok, cum, root, rows[:n], n, w)
    par2 = np.r_[par, p].astype(np.int32)
    tok2 = np.r_[tok, t].astype(np.int32)
    cum2 = oracle.cumulative_scores(par2, tok2, root, rows, n + w)
    np.testing.assert_allclose(cum2[:n], cum, rtol=0, atol=0)
    np.testing.assert_allclose(cum2[n:], s, rtol=1e-13, atol=1e-13)
