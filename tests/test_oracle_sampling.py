"""Pins for the sampling-verification oracle (temperature > 0).

The defining property of speculative sampling is that it is lossless: when
the draft tokens are drawn from the draft's distribution, every token the
verifier emits has exactly the target's distribution.  The oracle is used
as a black box here: acceptance probabilities and bonus-token probabilities
are measured by bisection over its uniform inputs (the decisions are
monotone in them), then averaged over every possible draft, exactly, on a
small vocabulary.  A dropped max(0, .), a residual taken against the wrong
distribution, a wrong row, p/q swapped or a missing renormalisation each
break one of these equalities.  Further pins: p == q accepts every first
child and samples the bonus as numpy's searchsorted does, and the
temperature -> 0 limit equals the (separately pinned) greedy verifier.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _threshold(pred, iters=60):
    """sup {u in [0, 1): pred(u)} for a predicate true on an initial interval."""
    if not pred(0.0):
        return 0.0
    top = np.nextafter(1.0, 0.0)
    if pred(top):
        return 1.0
    lo, hi = 0.0, 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if pred(mid):
            lo = mid
        else:
            hi = mid
    return lo


def _bonus_measure(bonus_of_u, V):
    """Probability of each bonus token for u uniform on [0, 1) (map nondecreasing in u)."""
    edges = [0.0]
    for t in range(1, V):
        edges.append(_threshold(lambda u, t=t: bonus_of_u(u) < t))
    edges.append(1.0)
    return np.diff(np.asarray(edges))


FORCE_REJECT = float(np.nextafter(1.0, 0.0))


class _Tree:
    """Target-side tree: node 0 is the root token (parent -1), rows per node."""

    def __init__(self, parent, tok, tgt, dft, root_tok, T):
        self.parent = np.asarray([parent], np.int32)
        self.tok = np.asarray([tok], np.int32)
        self.tgt = np.asarray([tgt], np.float64)
        self.dft = np.asarray([dft], np.float64)
        self.root = np.asarray([root_tok], np.int32)
        self.n = len(parent)
        self.T = T

    def run(self, u_acc, u_b):
        ua = np.asarray([u_acc], np.float64)
        path, plen, bonus = oracle.accept_sampling_path(
            self.tgt, self.dft, self.parent, self.tok, np.asarray([self.n]), self.root, ua,
            np.asarray([u_b]), self.T)
        return list(path[0, : plen[0]]), int(bonus[0])


def _rand_logits(rng, V, scale=1.5):
    return rng.normal(size=V) * scale


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_single_child_is_lossless(T):
    rng = np.random.default_rng(11)
    V = 5
    lp, lq = _rand_logits(rng, V), _rand_logits(rng, V)
    p, q = oracle.softmax_t(lp, T), oracle.softmax_t(lq, T)
    zeros = np.zeros(V)
    first = np.zeros(V)
    for x in range(V):  # the draft token of the root's child, drawn from q
        tr = _Tree([-1, 0], [3, x], [lp, zeros], [lq, zeros], 3, T)
        a = _threshold(lambda u: len(tr.run([0.0, u], 0.5)[0]) == 2)
        assert a == pytest.approx(min(1.0, p[x] / q[x]), abs=1e-12)
        b = _bonus_measure(lambda u: tr.run([0.0, FORCE_REJECT], u)[1], V)
        first += q[x] * (a * np.eye(V)[x] + (1.0 - a) * b)
    np.testing.assert_allclose(first, p, atol=1e-12)


def test_two_siblings_are_lossless():
    rng = np.random.default_rng(12)
    V, T = 4, 1.0
    lp, lq = _rand_logits(rng, V, 2.0), _rand_logits(rng, V, 2.0)
    p, q = oracle.softmax_t(lp, T), oracle.softmax_t(lq, T)
    zeros = np.zeros(V)
    first = np.zeros(V)
    for x1 in range(V):
        for x2 in range(V):  # two independent draws from q under the root
            tr = _Tree([-1, 0, 0], [0, x1, x2], [lp, zeros, zeros], [lq, zeros, zeros], 0, T)
            a1 = _threshold(lambda u: tr.run([0.0, u, 0.0], 0.5)[0][1:] == [1])
            a2 = _threshold(lambda u: tr.run([0.0, FORCE_REJECT, u], 0.5)[0][1:] == [2])
            b = _bonus_measure(lambda u: tr.run([0.0, FORCE_REJECT, FORCE_REJECT], u)[1], V)
            out = a1 * np.eye(V)[x1] + (1 - a1) * (a2 * np.eye(V)[x2] + (1 - a2) * b)
            first += q[x1] * q[x2] * out
    np.testing.assert_allclose(first, p, atol=1e-12)


def test_second_level_uses_the_accepted_node_row():
    # root -> a -> b: given that a (token y) is accepted, the next emitted token
    # must follow the target's row after a, whatever the row after the root is.
    rng = np.random.default_rng(13)
    V, T = 4, 1.0
    l0p, l0q = _rand_logits(rng, V), _rand_logits(rng, V)
    l1p = [_rand_logits(rng, V) for _ in range(V)]
    l1q = [_rand_logits(rng, V) for _ in range(V)]
    zeros = np.zeros(V)
    for y in range(V):
        p1, q1 = oracle.softmax_t(l1p[y], T), oracle.softmax_t(l1q[y], T)
        second = np.zeros(V)
        for x2 in range(V):
            tr = _Tree([-1, 0, 1], [2, y, x2], [l0p, l1p[y], zeros], [l0q, l1q[y], zeros], 2, T)
            # a accepted (u = 0 accepts any token with p > 0); measure b's test
            a = _threshold(lambda u: len(tr.run([0.0, 0.0, u], 0.5)[0]) == 3)
            b = _bonus_measure(lambda u: tr.run([0.0, 0.0, FORCE_REJECT], u)[1], V)
            second += q1[x2] * (a * np.eye(V)[x2] + (1 - a) * b)
        np.testing.assert_allclose(second, p1, atol=1e-12)


def test_equal_distributions_accept_first_children_and_sample_by_cdf():
    rng = np.random.default_rng(14)
    V, n = 50, 12
    for trial in range(20):
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        tok = [int(t) for t in rng.integers(0, V, size=n)]
        logits = rng.normal(size=(n, V)) * 2
        T = float(rng.uniform(0.5, 1.5))
        u = rng.uniform(size=n)
        ub = float(rng.uniform())
        tr = _Tree(parent, tok, logits, logits, tok[0], T)
        path, bonus = tr.run(u, ub)
        # expected: first child at every level, down to a leaf
        want = [0]
        while True:
            kids = [i for i in range(n) if parent[i] == want[-1]]
            if not kids:
                break
            want.append(kids[0])
        assert path == want
        p = oracle.softmax_t(logits[want[-1]], T)
        cdf = np.cumsum(p)
        assert bonus == int(np.searchsorted(cdf, ub * cdf[-1], side="right"))


def test_zero_temperature_limit_is_greedy():
    rng = np.random.default_rng(15)
    V, n, B = 40, 24, 30
    # logits on an integer grid with distinct values: at T = 1e-3 every
    # non-maximal probability underflows to exactly 0 in float64
    tgt = np.stack([[rng.permutation(V).astype(np.float64) for _ in range(n)] for _ in range(B)])
    dft = np.stack([[rng.permutation(V).astype(np.float64) for _ in range(n)] for _ in range(B)])
    parent = np.full((B, n), -1, np.int32)
    tok = np.zeros((B, n), np.int32)
    for b in range(B):
        for i in range(1, n):
            parent[b, i] = int(rng.integers(0, i))
        tok[b, 0] = 7
        for i in range(1, n):
            p = parent[b, i]
            used = {int(tok[b, j]) for j in range(1, i) if parent[b, j] == p}
            # half of the nodes carry the target's greedy token (if still free)
            want = int(np.argmax(tgt[b, p]))
            t = want if (rng.uniform() < 0.6 and want not in used) else int(rng.integers(0, V))
            while t in used:
                t = int(rng.integers(0, V))
            tok[b, i] = t
    n_nodes = np.full(B, n, np.int32)
    root = tok[:, 0].copy()
    u = rng.uniform(size=(B, n))
    ub = rng.uniform(size=B)
    got = oracle.accept_sampling_path(tgt, dft, parent, tok, n_nodes, root, u, ub, 1e-3)
    want = oracle.accept_greedy_path(tgt, parent, tok, n_nodes, root)
    for g, w in zip(got, want):
        np.testing.assert_array_equal(g, w)
    assert max(want[1]) >= 3  # the case exercises deep paths


def test_no_matching_top_node_and_leaf_root():
    V = 6
    lp = np.log(np.array([0.1, 0.2, 0.3, 0.1, 0.2, 0.1]))
    tr = _Tree([-1, 0], [4, 1], [lp, lp], [lp, lp], 2, 1.0)
    assert tr.run([0.5, 0.5], 0.5) == ([], 2)  # root_tok 2 is not node 0's token
    tr = _Tree([-1], [4], [lp], [lp], 4, 1.0)
    # a leaf root: the bonus comes from its own row; cumulative 0.1 0.3 0.6 ...
    assert tr.run([0.5], 0.25) == ([0], 1)
    assert tr.run([0.5], 0.35) == ([0], 2)
    assert tr.run([0.5], 0.0) == ([0], 0)


def test_residual_and_margins():
    r, z = oracle.residual([0.5, 0.3, 0.2], [0.2, 0.5, 0.3])
    np.testing.assert_allclose(r, [1.0, 0.0, 0.0])
    assert z == pytest.approx(0.3)
    r, z = oracle.residual([0.5, 0.5], [0.5, 0.5])
    np.testing.assert_allclose(r, [0.5, 0.5])
    assert z == 0.0
    t, gap = oracle.sample_inverse_cdf([0.25, 0.25, 0.5], 0.3)
    assert t == 1 and gap == pytest.approx(0.05)
    # margins are reported and vanish as a uniform approaches a decision boundary
    V = 4
    lp, lq = np.log([0.4, 0.3, 0.2, 0.1]), np.log([0.1, 0.6, 0.2, 0.1])
    tgt = np.asarray([[lp, lp]])
    dft = np.asarray([[lq, lq]])
    par = np.asarray([[-1, 0]], np.int32)
    tok = np.asarray([[0, 1]], np.int32)
    res = oracle.accept_sampling_path(tgt, dft, par, tok, np.asarray([2]), np.asarray([0]),
                                      np.asarray([[0.0, 0.5 - 1e-9]]), np.asarray([0.5]), 1.0,
                                      margins=True)
    assert list(res[0][0, :2]) == [0, 1]  # 0.3/0.6 = 0.5 > u
    assert res[3][0][0] < 1e-8
