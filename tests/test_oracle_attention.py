"""Pins for the attention oracle against facts that do not come from it.

* chain tree == causal attention (torch's scaled_dot_product_attention, fp64)
* all-zero queries: closed-form log-sum-exp and output read back as a mask
* Figure 3 of the SwiftSpec summary (Section 3.1.3): 4 x 10 mask, t7 row
* star tree, single key, expand == verify rows, re-root invariance
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from gen import random_case


def _chain_parent(n):
    return np.arange(-1, n - 1, dtype=np.int32)


def _recursive_depth(parent, n):
    """depth[i] = 1 + depth[parent[i]] (0 above the tree), filled in index order."""
    dep = np.zeros(n, dtype=np.int64)
    for i in range(n):
        p = int(parent[i])
        dep[i] = 1 + (dep[p] if p >= 0 else 0)
    return dep


def _recursive_visible(parent, n):
    """vis(i) = vis(parent(i)) | {i}, as boolean rows."""
    vis = np.zeros((n, n), dtype=bool)
    for i in range(n):
        p = int(parent[i])
        if p >= 0:
            vis[i] = vis[p]
        vis[i, i] = True
    return vis


def _subtree_sizes(parent, n):
    """1 + descendants, accumulated leaves-first."""
    size = np.ones(n, dtype=np.int64)
    for i in range(n - 1, -1, -1):
        p = int(parent[i])
        if p >= 0:
            size[p] += size[i]
    return size


@pytest.mark.parametrize("P,n,G,Hkv,d,seed", [
    (0, 1, 1, 1, 8, 0), (0, 7, 2, 2, 16, 1), (1, 5, 4, 1, 16, 2), (9, 12, 2, 3, 8, 3),
    (33, 16, 8, 1, 32, 4), (64, 3, 3, 2, 16, 5),
])
def test_chain_equals_causal_sdpa(P, n, G, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    Hq = G * Hkv
    T = P + n
    Qfull = rng.standard_normal((T, Hq, d))
    K = rng.standard_normal((T, Hkv, d))
    V = rng.standard_normal((T, Hkv, d))
    scale = 1.0 / np.sqrt(d) * 1.3
    O, LSE = oracle.tree_attention(Qfull[P:], K, V, P, _chain_parent(n), list(range(n)), G, scale)

    q = torch.from_numpy(Qfull).permute(1, 0, 2)[None]                      # [1,Hq,T,d]
    k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    ref = ref[0].permute(1, 0, 2).numpy()[P:]
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)

    # LSE through the same library routine: an extra all-zero key at position 0
    # (score 0 for every row, visible to every row under the causal mask) whose
    # value is a unit vector in an extra channel carries 1 / (1 + sum exp(s)).
    k0 = torch.cat([torch.zeros(1, Hq, 1, d, dtype=torch.float64), k], 2)
    v_ext = torch.cat([v, torch.zeros(1, Hq, T, 1, dtype=torch.float64)], 3)
    unit = torch.zeros(1, Hq, 1, d + 1, dtype=torch.float64)
    unit[..., d] = 1.0
    v0 = torch.cat([unit, v_ext], 2)
    q0 = torch.cat([torch.zeros(1, Hq, 1, d, dtype=torch.float64), q], 2)
    r = torch.nn.functional.scaled_dot_product_attention(q0, k0, v0, is_causal=True, scale=scale)
    frac = r[0, :, 1 + P:, d].numpy()                                           # [Hq, n]
    np.testing.assert_allclose(LSE, np.log(1.0 / frac - 1.0), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("seed", range(12))
def test_zero_query_closed_form(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 14))
    P = int(rng.integers(0, 6))
    parent = np.array([rng.integers(-1, i) if i else -1 for i in range(n)], dtype=np.int32)
    G, Hkv = 2, 1
    d = max(n, 4)
    q = np.zeros((n, G * Hkv, d))
    K = rng.standard_normal((P + n, Hkv, d))
    V = np.zeros((P + n, Hkv, d))
    for j in range(n):
        V[P + j, 0, j] = 1.0
    O, LSE = oracle.tree_attention(q, K, V, P, parent, list(range(n)), G, 0.37)
    dep = _recursive_depth(parent, n)
    vis = _recursive_visible(parent, n)
    for h in range(G):
        np.testing.assert_allclose(LSE[h], np.log(P + dep), rtol=0, atol=1e-14)
        # The tree block of O is indicator(visible)/(P + depth): read the mask back.
        np.testing.assert_allclose(O[:, h, :n], vis / (P + dep)[:, None], rtol=0, atol=1e-15)
    # column counts = subtree sizes (who sees node j)
    seen_by = (O[:, 0, :n] > 0).sum(axis=0)
    np.testing.assert_array_equal(seen_by, _subtree_sizes(parent, n))


def _fig3_parents(fx, max_cases=None, seed=0):
    toks = fx["tokens"]
    idx = {t: i for i, t in enumerate(toks)}
    existing = [idx[t] for t in fx["existing"]]
    choices = []
    for i, t in enumerate(toks):
        if t in fx["fixed_parent"]:
            p = fx["fixed_parent"][t]
            choices.append([-1] if p == "root" else [idx[p]])
        elif t in fx["new_leaves"]:
            choices.append([-1] + existing)
        else:
            choices.append(list(range(-1, i)))
    allp = list(itertools.product(*choices))
    if max_cases is not None and len(allp) > max_cases:
        rng = np.random.default_rng(seed)
        allp = [allp[j] for j in rng.choice(len(allp), size=max_cases, replace=False)]
    return [np.array(p, dtype=np.int32) for p in allp]


def test_fig3_non_square_mask(golden):
    fx = golden("fig3_expand_mask.json")
    toks = fx["tokens"]
    n, P, w = len(toks), fx["prefix_len"], len(fx["new_leaves"])
    parents = _fig3_parents(fx, max_cases=400)
    assert len(parents) == 400
    d = P + n
    t7 = toks.index("t7")
    for parent in parents:
        assert oracle.is_valid_parent(parent, n)
        q = np.zeros((w, 1, d))
        K = np.zeros((P + n, 1, d))
        V = np.eye(P + n)[:, None, :]         # column j's value is the unit vector e_j
        nodes = list(range(n - w, n))
        O, LSE = oracle.tree_attention(q, K, V, P, parent, nodes, 1, 1.0)
        assert O.shape[0] == fx["mask_rows"] and O.shape[2] == fx["mask_cols"]
        row = nodes.index(t7)
        visible = np.nonzero(O[row, 0] > 0)[0].tolist()
        assert visible == fx["row_t7_visible_columns"]
        assert np.isclose(LSE[0, row], np.log(len(visible)))


def test_star_tree_sees_prefix_and_self():
    rng = np.random.default_rng(7)
    n, P, d = 9, 5, 16
    parent = np.full(n, -1, dtype=np.int32)
    q = rng.standard_normal((n, 1, d))
    K = rng.standard_normal((P + n, 1, d))
    V = rng.standard_normal((P + n, 1, d))
    O, LSE = oracle.tree_attention(q, K, V, P, parent, list(range(n)), 1, 0.25)
    for i in range(n):
        keys = np.r_[np.arange(P), P + i]
        s = 0.25 * K[keys, 0] @ q[i, 0]
        e = np.exp(s - s.max())
        np.testing.assert_allclose(O[i, 0], (e / e.sum()) @ V[keys, 0], rtol=1e-13, atol=1e-13)
        assert np.isclose(LSE[0, i], s.max() + np.log(e.sum()), rtol=1e-13)


def test_single_key():
    rng = np.random.default_rng(8)
    d = 32
    q = rng.standard_normal((1, 4, d))
    K = rng.standard_normal((1, 2, d))
    V = rng.standard_normal((1, 2, d))
    O, LSE = oracle.tree_attention(q, K, V, 0, np.array([-1]), [0], 2, 0.5)
    for h in range(4):
        np.testing.assert_allclose(O[0, h], V[0, h // 2], rtol=0, atol=0)
        assert LSE[h, 0] == pytest.approx(0.5 * q[0, h] @ K[0, h // 2], rel=1e-15)


def test_expand_rows_equal_verify_rows():
    c = random_case(11, B=3, Hq=4, Hkv=2, d=16, P_range=(0, 40), n_max=10, n_range=(4, 10),
                    dtype="f32")
    w = 3
    qe = np.stack([c.q[b, int(c.n_nodes[b]) - w: int(c.n_nodes[b])] for b in range(c.B)])
    Ov, Lv = oracle.verify(c)
    Oe, Le = oracle.expand(c, qe, w)
    for b in range(c.B):
        n = int(c.n_nodes[b])
        np.testing.assert_allclose(Oe[b], Ov[b, n - w: n], rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(Le[b], Lv[b][:, n - w: n], rtol=1e-14, atol=1e-14)


def test_paged_gather_equals_contiguous():
    c1 = random_case(12, B=3, Hq=2, Hkv=1, d=8, P_range=(0, 70), n_max=6, dtype="f32")
    c2 = random_case(12, B=3, Hq=2, Hkv=1, d=8, P_range=(0, 70), n_max=6, dtype="f32", paged=True)
    # same seed -> same tree and prefix lengths; KV values differ by layout of the
    # draw, so compare the two layouts through their own gathers and attention.
    np.testing.assert_array_equal(c1.prefix_len, c2.prefix_len)
    for b in range(3):
        T = int(c2.prefix_len[b] + c2.n_nodes[b])
        ks, vs = oracle.gather_sequence_kv(c2.k, c2.v, b, T, "f32", c2.block_table, c2.block_size)
        blocks = c2.block_table[b]
        for t in range(T):
            np.testing.assert_array_equal(ks[t], c2.k[blocks[t // 16], t % 16])
        assert np.isfinite(ks).all() and np.isfinite(vs).all()


@pytest.mark.parametrize("seed", range(6))
def test_reroot_preserves_attention_of_kept_nodes(seed):
    """Kept nodes see the same (key, value) rows before and after the re-root."""
    rng = np.random.default_rng(300 + seed)
    c = random_case(300 + seed, B=1, Hq=4, Hkv=2, d=16, P_range=(3, 20), n_max=14,
                    n_range=(6, 14), dtype="f32")
    n = int(c.n_nodes[0])
    par = c.parent[0]
    end = int(rng.integers(0, n))
    path = oracle.root_path(par, end)
    pa = np.full((1, c.n_max), -1, dtype=np.int32)
    pa[0, : len(path)] = path
    kept = oracle.descendants(par, end, n)
    O0, L0 = oracle.verify(c)
    (layers, P1, par1, n1) = oracle.tree_cache_reroot([(c.k, c.v)], c.prefix_len, c.parent,
                                                      c.n_nodes, pa, np.array([len(path)]),
                                                      np.array([True]))
    c.k, c.v = layers[0]
    q1 = np.zeros_like(c.q)
    q1[0, : len(kept)] = c.q[0, kept]
    c.q = q1
    c.prefix_len, c.parent, c.n_nodes = P1, par1, n1
    O1, L1 = oracle.verify(c)
    assert n1[0] == len(kept)
    for r, u in enumerate(kept):
        np.testing.assert_allclose(O1[0, r], O0[0, u], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L1[0][:, r], L0[0][:, u], rtol=1e-12, atol=1e-12)
