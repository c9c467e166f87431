"""GPU parity of accept_sampling_path (tree verification by speculative
sampling) against the oracle (oracle/sampling.py).

The path, its length and the bonus token are integers decided by floating
point, so both sides must be given decisions that the precision of either
cannot flip: the test draws the uniforms, asks the oracle how far each
decision lay from its boundary, and redraws a sequence's uniforms while
a margin is below the bar (1e-3 for an acceptance test, 2e-5 of the mass for
the bonus draw; fp32 rounding moves these quantities by ~1e-6).  Then the
outputs must match exactly.  A statistical check on the GPU alone: over many
sequences with the same single-child tree, the first emitted token follows
the target's distribution."""
import numpy as np
import pytest

from helpers import dev_tensor, ensure_built, to_f64

import oracle

pytestmark = pytest.mark.gpu

TEST_MARGIN = 1e-3
BONUS_MARGIN = 2e-5


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _gumbel_pick(rng, logits, T):
    return int(np.argmax(logits / T + rng.gumbel(size=logits.shape[0])))


def _case(seed, B, n_max, V, T, dtype, shape="random", noise=0.5, scale=2.0):
    """Target-side trees (node 0 = the root token), draft children drawn from
    the draft's distribution at their parent (Gumbel-max on the draft row)."""
    import torch
    rng = np.random.default_rng([seed, 77])
    tgt = rng.normal(size=(B, n_max, V)).astype(np.float32) * scale
    dft = (tgt + rng.normal(size=(B, n_max, V)).astype(np.float32) * noise).astype(np.float32)
    if dtype == "bf16":
        tgt_d = torch.from_numpy(tgt).to("cuda").to(torch.bfloat16)
        dft_d = torch.from_numpy(dft).to("cuda").to(torch.bfloat16)
    else:
        tgt_d = torch.from_numpy(tgt).to("cuda")
        dft_d = torch.from_numpy(dft).to("cuda")
    tgt64, dft64 = to_f64(tgt_d), to_f64(dft_d)
    par = np.full((B, n_max), -1, np.int32)
    tok = np.zeros((B, n_max), np.int32)
    n = np.zeros(B, np.int32)
    root = np.zeros(B, np.int32)
    for b in range(B):
        nb = n_max if b % 5 else int(rng.integers(1, n_max + 1))
        n[b] = nb
        tok[b, 0] = int(rng.integers(0, V))
        for i in range(1, nb):
            if shape == "chain":
                par[b, i] = i - 1
            elif shape == "star":
                par[b, i] = 0
            else:
                par[b, i] = int(rng.integers(0, i))
            tok[b, i] = _gumbel_pick(rng, dft64[b, par[b, i]], T)
        root[b] = tok[b, 0]
    return dict(tgt=tgt_d, dft=dft_d, tgt64=tgt64, dft64=dft64, par=par, tok=tok, n=n, root=root,
                rng=rng, T=T, B=B, n_max=n_max, V=V)


def _draw_uniforms(c):
    """Uniforms (fp32) whose every oracle decision clears the margins."""
    rng, B, n_max = c["rng"], c["B"], c["n_max"]
    u = rng.uniform(size=(B, n_max)).astype(np.float32)
    ub = rng.uniform(size=B).astype(np.float32)
    want = [np.full((B, n_max), -1, np.int32), np.zeros(B, np.int32), np.zeros(B, np.int32)]
    todo = np.arange(B)
    for _ in range(80):
        res = oracle.accept_sampling_path(c["tgt64"][todo], c["dft64"][todo], c["par"][todo],
                                          c["tok"][todo], c["n"][todo], c["root"][todo],
                                          u[todo].astype(np.float64), ub[todo].astype(np.float64),
                                          c["T"], margins=True)
        tm, bm = res[3]
        ok = (tm >= TEST_MARGIN) & (bm >= BONUS_MARGIN)
        for j in range(3):
            want[j][todo[ok]] = res[j][ok]
        todo = todo[~ok]
        if todo.size == 0:
            return u, ub, tuple(want)
        u[todo] = rng.uniform(size=(todo.size, n_max)).astype(np.float32)
        ub[todo] = rng.uniform(size=todo.size).astype(np.float32)
    raise AssertionError("could not draw uniforms away from the decision boundaries")


def _run(ta, c, u, ub, n_override=None, root_override=None):
    import torch
    n = c["n"] if n_override is None else n_override
    root = c["root"] if root_override is None else root_override
    path, plen, bonus = ta.accept_sampling_path(
        c["tgt"], c["dft"], dev_tensor(c["par"]), dev_tensor(c["tok"]),
        dev_tensor(np.asarray(n, np.int32)), dev_tensor(np.asarray(root, np.int32)),
        dev_tensor(u), dev_tensor(ub), c["T"])
    torch.cuda.synchronize()
    return path.cpu().numpy(), plen.cpu().numpy(), bonus.cpu().numpy()


def _compare(got, want):
    path, plen, bonus = got
    wp, wl, wb = want
    np.testing.assert_array_equal(plen, wl)
    np.testing.assert_array_equal(path, wp)
    np.testing.assert_array_equal(bonus, wb)


CASES = [
    # seed, B, n_max, V, T, dtype, shape, noise
    (1, 16, 16, 1000, 1.0, "f32", "random", 0.5),
    (2, 16, 16, 1000, 1.0, "bf16", "random", 0.5),
    (3, 8, 64, 32000, 1.0, "bf16", "random", 0.4),
    (4, 8, 16, 32000, 0.6, "f32", "chain", 0.2),
    (5, 6, 256, 1000, 1.0, "bf16", "random", 1.0),
    (6, 6, 48, 1001, 0.8, "bf16", "star", 1.5),   # odd V: scalar loads; many rejections
    (7, 6, 32, 4097, 1.3, "f32", "star", 2.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-{c[5]}-{c[6]}-V{c[3]}")
def test_sampling_matches_oracle(ta, case):
    seed, B, n_max, V, T, dt, shape, noise = case
    c = _case(seed, B, n_max, V, T, dt, shape, noise)
    u, ub, want = _draw_uniforms(c)
    print(f"case {case}: path lengths {list(want[1])}", flush=True)
    _compare(_run(ta, c, u, ub), want)
    if shape == "star":  # the case must exercise rejections (a later child or the bonus wins)
        assert ((want[0][:, 1] > 1) | (want[1] == 1)).any()


def test_sampling_edge_cases(ta):
    c = _case(8, 6, 16, 500, 1.0, "f32")
    u, ub, _ = _draw_uniforms(c)
    # n = 0, a single root node, and a root token that node 0 does not carry
    n = c["n"].copy()
    n[0], n[1] = 0, 1
    root = c["root"].copy()
    root[2] = (root[2] + 1) % c["V"]
    want = oracle.accept_sampling_path(c["tgt64"], c["dft64"], c["par"], c["tok"], n, root,
                                       u.astype(np.float64), ub.astype(np.float64), c["T"])
    got = _run(ta, c, u, ub, n_override=n, root_override=root)
    _compare(got, want)
    assert got[1][0] == 0 and got[2][0] == root[0]
    assert got[1][1] == 1 and got[1][2] == 0 and got[2][2] == root[2]


def test_first_token_follows_the_target_distribution(ta):
    """Root + one child drawn from q, for 20000 sequences: the first emitted
    token (the child if accepted, else the bonus) must be distributed as p."""
    import torch
    rng = np.random.default_rng(99)
    B, V, T = 20000, 8, 1.0
    lp = rng.normal(size=V) * 1.2
    lq = lp + rng.normal(size=V) * 1.0
    p, q = oracle.softmax_t(lp, T), oracle.softmax_t(lq, T)
    tgt = np.broadcast_to(np.stack([lp, lp]), (B, 2, V)).astype(np.float32).copy()
    dft = np.broadcast_to(np.stack([lq, lq]), (B, 2, V)).astype(np.float32).copy()
    par = np.tile(np.array([-1, 0], np.int32), (B, 1))
    tok = np.zeros((B, 2), np.int32)
    tok[:, 1] = rng.choice(V, size=B, p=q)
    u = rng.uniform(size=(B, 2)).astype(np.float32)
    ub = rng.uniform(size=B).astype(np.float32)
    path, plen, bonus = ta.accept_sampling_path(
        dev_tensor(tgt), dev_tensor(dft), dev_tensor(par), dev_tensor(tok),
        dev_tensor(np.full(B, 2, np.int32)), dev_tensor(np.zeros(B, np.int32)), dev_tensor(u),
        dev_tensor(ub), T)
    torch.cuda.synchronize()
    plen, bonus = plen.cpu().numpy(), bonus.cpu().numpy()
    first = np.where(plen == 2, tok[:, 1], bonus)
    hist = np.bincount(first, minlength=V) / B
    sigma = np.sqrt(p * (1 - p) / B)
    assert np.all(np.abs(hist - p) < 5 * sigma + 1e-4), (hist, p)
    # the draft alone would be visibly different
    assert np.max(np.abs(q - p) / np.sqrt(p * (1 - p) / B + 1e-12)) > 10
