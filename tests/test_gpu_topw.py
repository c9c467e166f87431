"""GPU parity of tree_expand_top_w against the float64 oracle (oracle/topw.py).

The kernel scores candidates in fp32, the oracle in fp64, so which candidates
win is compared exactly only where the fp64 scores are separated by more than
the fp32 error; within that margin any of the near-equal candidates is a
correct pick, and the test checks the picks are valid and in order instead.
The cumulative scores written for the new nodes are compared with the fp64
scores of the same candidates."""
import numpy as np
import pytest

from helpers import dev_tensor, ensure_built

import oracle
from oracle.topw import log_softmax
from gen import config4_expand, random_case

pytestmark = pytest.mark.gpu

SCORE_TOL = 2e-4  # fp32 log-softmax of a 32000-way row: a few 1e-6 relative


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _fp64_scores(parent, tok, cum, logits, n):
    """Every candidate's fp64 score: dict (p, t) -> score (p = -1 is the root)."""
    V = logits.shape[1]
    out = {}
    for p in range(-1, n):
        row = logits[p + 1].astype(np.float64)
        lsm = log_softmax(row)
        base = 0.0 if p < 0 else float(cum[p])
        taken = {int(tok[c]) for c in range(n) if int(parent[c]) == p}
        for t in range(V):
            if t not in taken:
                out[(p, t)] = base + lsm[t]
    return out


def _check_round(par0, tok0, cum0, n0, logits, w, n_max, par1, tok1, cum1, n1):
    """One sequence's expansion step: GPU result (…1) against the oracle."""
    avail = sum(int(logits.shape[1]) - sum(1 for c in range(n0) if int(par0[c]) == p)
                for p in range(-1, n0))   # candidates that exist at all
    take = min(w, n_max - n0, avail)
    assert n1 == n0 + take
    # existing nodes untouched
    np.testing.assert_array_equal(par1[:n0], par0[:n0])
    np.testing.assert_array_equal(tok1[:n0], tok0[:n0])
    if take == 0:
        return
    # one more than taken, to see the margin at the boundary
    P, T, S = oracle.select_top_w(par0, tok0, cum0.astype(np.float64), logits[0], logits[1:], n0,
                                  take + 1)
    got = [(int(par1[n0 + k]), int(tok1[n0 + k])) for k in range(take)]
    want = [(int(P[k]), int(T[k])) for k in range(take)]
    separated = all(S[k] - S[k + 1] > SCORE_TOL for k in range(len(S) - 1))
    if separated:
        assert got == want
        np.testing.assert_allclose(cum1[n0:n0 + take], S[:take], rtol=1e-5, atol=SCORE_TOL)
        return
    # near ties: the picks must be valid, distinct, ordered and as good as the oracle's
    scores = _fp64_scores(par0, tok0, cum0, logits, n0)
    assert len(set(got)) == take
    s_got = np.array([scores[g] for g in got])       # KeyError = a taken token was picked
    assert np.all(np.diff(s_got) <= SCORE_TOL)
    assert s_got[-1] >= S[take - 1] - SCORE_TOL
    np.testing.assert_allclose(cum1[n0:n0 + take], s_got, rtol=1e-5, atol=SCORE_TOL)


def _run(ta, logits, par, tok, cum, n, w, dtype="f32"):
    """One tree_expand_top_w call; returns the GPU's tree and the logits as
    the kernel read them (bf16 rounding done on the host, before upload)."""
    import torch
    lg_host = torch.from_numpy(np.ascontiguousarray(logits))
    if dtype == "bf16":
        lg_host = lg_host.to(torch.bfloat16)
    lg = lg_host.cuda()
    d_par, d_tok = dev_tensor(par.copy()), dev_tensor(tok.copy())
    d_cum, d_n = dev_tensor(cum.astype(np.float32).copy()), dev_tensor(n.astype(np.int32).copy())
    ta.tree_expand_top_w(lg, d_par, d_tok, d_cum, d_n, w)
    torch.cuda.synchronize()
    return (d_par.cpu().numpy(), d_tok.cpu().numpy(), d_cum.cpu().numpy(), d_n.cpu().numpy(),
            lg_host.float().numpy())


@pytest.mark.parametrize("seed,V,w,dtype", [
    (1, 50, 4, "f32"), (2, 1000, 8, "f32"), (3, 32000, 8, "f32"), (4, 32000, 16, "bf16"),
    (5, 777, 1, "f32"), (6, 4096, 12, "bf16"), (7, 33, 16, "f32")])
def test_topw_random_trees(ta, seed, V, w, dtype):
    c = random_case(seed, B=3, Hq=1, Hkv=1, d=64, P_range=(0, 2), n_max=40, n_range=(1, 30),
                    dtype="f32", vocab=V)
    rng = np.random.default_rng([seed, 7])
    logits = rng.standard_normal((c.B, c.n_max + 1, V), dtype=np.float32)
    cum = np.zeros((c.B, c.n_max), dtype=np.float32)
    for b in range(c.B):
        n = int(c.n_nodes[b])
        lg = logits[b].astype(np.float64)
        if dtype == "bf16":
            import torch
            lg = torch.from_numpy(logits[b]).to(torch.bfloat16).float().numpy().astype(np.float64)
        cum[b, :n] = oracle.cumulative_scores(c.parent[b], c.tok[b], lg[0], lg[1:], n)
    par1, tok1, cum1, n1, lg_used = _run(ta, logits, c.parent, c.tok, cum, c.n_nodes, w, dtype)
    for b in range(c.B):
        _check_round(c.parent[b], c.tok[b], cum[b], int(c.n_nodes[b]), lg_used[b], w, c.n_max,
                     par1[b], tok1[b], cum1[b], int(n1[b]))


def test_topw_excludes_existing_children_and_capacity(ta):
    """The best logits of a row belong to existing children: they must not be
    picked again; a nearly full tree appends only up to n_max."""
    V, n_max = 500, 12
    parent = np.array([[-1, -1, 0, 0, 1, 2, -1, -1, -1, -1, -1, -1],
                       [-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, -1, -1]], dtype=np.int32)
    tok = np.array([[5, 6, 7, 8, 9, 10, 0, 0, 0, 0, 0, 0],
                    [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 0, 0]], dtype=np.int32)
    n = np.array([6, 10], dtype=np.int32)
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((2, n_max + 1, V), dtype=np.float32)
    for b in range(2):
        for c in range(int(n[b])):
            logits[b, parent[b, c] + 1, tok[b, c]] = 9.0     # children hold their row's maximum
    cum = np.zeros((2, n_max), dtype=np.float32)
    for b in range(2):
        cum[b, :n[b]] = oracle.cumulative_scores(parent[b], tok[b], logits[b, 0], logits[b, 1:],
                                                 int(n[b]))
    par1, tok1, cum1, n1, lg = _run(ta, logits, parent, tok, cum, n, 4)
    assert n1.tolist() == [10, 12]
    for b in range(2):
        _check_round(parent[b], tok[b], cum[b], int(n[b]), lg[b], 4, n_max, par1[b], tok1[b],
                     cum1[b], int(n1[b]))
        for k in range(int(n[b]), int(n1[b])):
            sib = [int(tok1[b, c]) for c in range(int(n1[b])) if par1[b, c] == par1[b, k] and c != k]
            assert int(tok1[b, k]) not in sib


def test_topw_config4_rounds_on_device(ta):
    """The draft-expansion workload's four rounds, each selected on the GPU.
    The oracle runs its own four rounds from the same seeded inputs; the
    seeded candidates are separated by more than the fp32 error at every
    pick, so the two trees must be equal after every round (weights within
    the fp32 error)."""
    import torch
    c = config4_expand()
    n_max, V, w, n0 = c.n_max, c.vocab, c.w, c.n0
    rows = np.zeros((n_max + 1, V), dtype=np.float32)   # row 0: root, row 1 + i: node i
    rows[0] = c.logits_root
    rows[1:n0 + 1] = c.logits0
    for r in range(c.rounds):
        rows[n0 + r * w + 1:n0 + (r + 1) * w + 1] = c.logits_new[r]
    par = np.full(n_max, -1, dtype=np.int32)
    tok = np.zeros(n_max, dtype=np.int32)
    par[:n0], tok[:n0] = c.parent0, c.tok0
    cum0 = np.zeros(n_max, dtype=np.float32)
    cum0[:n0] = oracle.cumulative_scores(c.parent0, c.tok0, rows[0], rows[1:], n0)
    d_lg = dev_tensor(rows[None].copy())
    d_par, d_tok, d_cum = dev_tensor(par[None].copy()), dev_tensor(tok[None].copy()), \
        dev_tensor(cum0[None].copy())
    d_n = dev_tensor(np.array([n0], np.int32))
    n = n0
    for r in range(c.rounds):
        cum64 = oracle.cumulative_scores(par, tok, rows[0], rows[1:], n)
        P, T, S = oracle.select_top_w(par, tok, cum64, rows[0], rows[1:], n, w + 1)
        assert np.all(np.diff(-S) > SCORE_TOL), "seeded scores separated at every pick"
        ta.tree_expand_top_w(d_lg, d_par, d_tok, d_cum, d_n, w)
        torch.cuda.synchronize()
        assert int(d_n.item()) == n + w
        gp, gt, gc = (x.cpu().numpy()[0] for x in (d_par, d_tok, d_cum))
        assert list(zip(gp[n:n + w].tolist(), gt[n:n + w].tolist())) == \
            list(zip(P[:w].tolist(), T[:w].tolist())), f"round {r}"
        np.testing.assert_allclose(gc[n:n + w], S[:w], rtol=1e-5, atol=SCORE_TOL)
        par[n:n + w], tok[n:n + w] = P[:w], T[:w]
        np.testing.assert_array_equal(gp[:n + w], par[:n + w])
        n += w
    assert n == n0 + w * c.rounds


def _single_tree(n, V, seed):
    rng = np.random.default_rng([seed, 11])
    parent = np.array([rng.integers(-1, i) for i in range(n)], dtype=np.int32)
    tok = rng.integers(0, V, size=n).astype(np.int32)
    # siblings take distinct tokens
    for i in range(n):
        while any(int(parent[c]) == int(parent[i]) and int(tok[c]) == int(tok[i]) for c in range(i)):
            tok[i] = (tok[i] + 1) % V
    return parent, tok


@pytest.mark.parametrize("V,dtype", [(1 << 18, "f32"), (1 << 18, "bf16"), (40000, "f32"),
                                     (70001, "bf16")])
def test_topw_large_vocab(ta, V, dtype):
    """Vocabularies past one load batch per thread (rows read in several
    batches, the winners' logits read again), aligned and unaligned."""
    n_max, n = 6, 3
    parent, tok = _single_tree(n, V, 5)
    par = np.full((1, n_max), -1, np.int32)
    tk = np.zeros((1, n_max), np.int32)
    par[0, :n], tk[0, :n] = parent, tok
    logits = np.random.default_rng([V, 3]).standard_normal((1, n_max + 1, V), dtype=np.float32)
    lg = logits[0].astype(np.float64)
    if dtype == "bf16":
        import torch
        lg = torch.from_numpy(logits[0]).to(torch.bfloat16).float().numpy().astype(np.float64)
    cum = np.zeros((1, n_max), np.float32)
    cum[0, :n] = oracle.cumulative_scores(parent, tok, lg[0], lg[1:], n)
    par1, tok1, cum1, n1, lg_used = _run(ta, logits, par, tk, cum, np.array([n], np.int32), 3, dtype)
    _check_round(par[0], tk[0], cum[0], n, lg_used[0], 3, n_max, par1[0], tok1[0], cum1[0], int(n1[0]))


@pytest.mark.parametrize("V,w,dtype", [(1000, 8, "f32"), (4096, 16, "bf16"), (777, 5, "f32"),
                                     (20000, 8, "f32"), (40000, 16, "bf16")])
def test_topw_all_ties(ta, V, w, dtype):
    """Every logit equal: every thread's best logit ties, so the threshold
    step ranks hundreds of keys; the picks are the root's lowest free tokens
    in token order (equal scores: lower parent, then lower token), also for
    vocabularies of tens of thousands of tied logits."""
    n_max, n = 30, 6
    parent = np.array([-1, -1, 0, 0, 1, -1] + [-1] * (n_max - 6), np.int32)[None]
    tok = np.array([0, 2, 0, 1, 5, 3] + [0] * (n_max - 6), np.int32)[None]
    logits = np.zeros((1, n_max + 1, V), np.float32)
    cum = np.zeros((1, n_max), np.float32)
    cum[0, :n] = oracle.cumulative_scores(parent[0], tok[0], logits[0, 0].astype(np.float64),
                                          logits[0, 1:].astype(np.float64), n)
    par1, tok1, cum1, n1, _ = _run(ta, logits, parent, tok, cum, np.array([n], np.int32), w, dtype)
    assert int(n1[0]) == n + w
    free_root = [t for t in range(V) if t not in (0, 2, 3)][:w]
    assert par1[0, n:n + w].tolist() == [-1] * w
    assert tok1[0, n:n + w].tolist() == free_root
    np.testing.assert_allclose(cum1[0, n:n + w], -np.log(V), rtol=1e-6)


def test_topw_inf_logits_and_scarce_tokens(ta):
    """-inf logits score -inf but stay candidates; with fewer candidates in
    the whole tree than w, all of them are appended, best first."""
    V, n_max, n, w = 3, 10, 2, 8
    parent = np.array([[-1, 0] + [-1] * (n_max - 2)], np.int32)
    tok = np.array([[1, 2] + [0] * (n_max - 2)], np.int32)
    logits = np.array([[[0.5, 2.0, -np.inf], [1.0, -np.inf, 3.0], [0.0, -1.0, -2.0]]
                       + [[0.0, 0.0, 0.0]] * (n_max - 2)], np.float32)
    cum = np.zeros((1, n_max), np.float32)
    cum[0, :n] = oracle.cumulative_scores(parent[0], tok[0], logits[0, 0].astype(np.float64),
                                          logits[0, 1:].astype(np.float64), n)
    par1, tok1, cum1, n1, lg = _run(ta, logits, parent, tok, cum, np.array([n], np.int32), w)
    # candidates: root {0, 2}, node 0 {0, 1}, node 1 {0, 1, 2}: 7 in all
    assert int(n1[0]) == n + 7
    P, T, S = oracle.select_top_w(parent[0], tok[0], cum[0].astype(np.float64), lg[0, 0], lg[0, 1:],
                                  n, 7)
    assert par1[0, n:n + 7].tolist() == P.tolist()
    assert tok1[0, n:n + 7].tolist() == T.tolist()
    fin = np.isfinite(S)
    np.testing.assert_allclose(cum1[0, n:n + 7][fin], S[fin], rtol=1e-5, atol=2e-4)
    assert np.all(np.isneginf(cum1[0, n:n + 7][~fin]))
