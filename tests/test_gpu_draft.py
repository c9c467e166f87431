"""GPU parity of the draft-side entry points against the oracle
(oracle/draft.py, oracle/reroot.py): tree_token_walk (bit-exact path, length,
keep flag), tree_cache_reroot_draft (bit-exact tokens, re-based weights, KV
bytes) and tree_select_subtree (bit-exact nodes, renumbered parents, tokens),
Figure 2 chained through the device re-root, and one whole draft iteration
(four top-w expansions, walk, re-root, Select) on the device against an
independent oracle chain."""
import numpy as np
import pytest

from helpers import dev_tensor, ensure_built

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _tree(rng, n, n_max, V=40, dup_siblings=False):
    par = np.full(n_max, -1, dtype=np.int32)
    tok = np.zeros(n_max, dtype=np.int32)
    for i in range(n):
        par[i] = rng.integers(-1, i) if i else -1
        used = {int(tok[c]) for c in range(i) if par[c] == par[i]}
        if dup_siblings and used and rng.random() < 0.3:
            tok[i] = rng.choice(sorted(used))
        else:
            tok[i] = rng.choice([t for t in range(V + n) if t not in used])
    return par, tok


def _walk(ta, par, tok, n, ver, m_max):
    import torch
    B = par.shape[0]
    verified = np.zeros((B, m_max), dtype=np.int32)
    vlen = np.zeros(B, dtype=np.int32)
    for b, v in enumerate(ver):
        verified[b, :min(len(v), m_max)] = v[:m_max]
        vlen[b] = len(v)
    path, plen, keep = ta.tree_token_walk(dev_tensor(par), dev_tensor(tok),
                                          dev_tensor(np.asarray(n, np.int32)), dev_tensor(verified),
                                          dev_tensor(vlen))
    torch.cuda.synchronize()
    return path.cpu().numpy(), plen.cpu().numpy(), keep.cpu().numpy()


@pytest.mark.parametrize("seed,n_max,dup", [(1, 16, False), (2, 64, False), (3, 256, False),
                                            (4, 40, True)])
def test_token_walk_random_trees(ta, seed, n_max, dup):
    rng = np.random.default_rng([seed, 50])
    B = 12
    par = np.full((B, n_max), -1, dtype=np.int32)
    tok = np.zeros((B, n_max), dtype=np.int32)
    n = np.zeros(B, dtype=np.int32)
    ver = []
    for b in range(B):
        n[b] = rng.integers(0, n_max + 1) if b % 4 else n_max
        par[b], tok[b] = _tree(rng, int(n[b]), n_max, dup_siblings=dup)
        if n[b] == 0:
            ver.append([int(rng.integers(0, 50))] if b % 2 else [])
            continue
        x = int(rng.integers(0, n[b]))
        v = [int(tok[b, u]) for u in oracle.root_path(par[b], x)]
        kind = b % 3
        if kind == 1:
            v.append(10 ** 6)                          # out of the tree
        elif kind == 2:
            kids = [c for c in range(n[b]) if par[b, c] == x]
            v.append(int(tok[b, kids[0]]) if kids else 10 ** 6)
        ver.append(v)
    m_max = max(1, max(len(v) for v in ver))
    path, plen, keep = _walk(ta, par, tok, n, ver, m_max)
    for b in range(B):
        want, wkeep = oracle.token_walk(par[b], tok[b], int(n[b]), ver[b])
        assert plen[b] == len(want) and keep[b] == int(wkeep), (b, want, wkeep)
        assert path[b, :plen[b]].tolist() == want


def test_token_walk_clamps_length(ta):
    """verified_len past m_max reads only the m_max tokens present; a
    negative length is an empty walk."""
    import torch
    par = np.array([[-1, 0, 1, 2]], dtype=np.int32)
    tok = np.array([[4, 5, 6, 7]], dtype=np.int32)
    ver = dev_tensor(np.array([[4, 5]], np.int32))
    for vlen, want in ((9, (2, 1)), (-3, (0, 1)), (1, (1, 1))):
        path, plen, keep = ta.tree_token_walk(dev_tensor(par), dev_tensor(tok),
                                              dev_tensor(np.array([4], np.int32)), ver,
                                              dev_tensor(np.array([vlen], np.int32)))
        torch.cuda.synchronize()
        assert (plen.item(), keep.item()) == want, vlen
        assert path[0, :plen.item()].tolist() == [0, 1][:plen.item()]


def test_fig2_walk_and_reroot_on_the_gpu(ta, golden):
    import torch
    fx = golden("fig2_iterations.json")
    toks = fx["tree_tokens"]
    idx = {t: i for i, t in enumerate(toks)}
    n = len(toks)
    # one parent array consistent with the figure: t3 under the root, t6
    # under t3, t9..t12 exactly the subtree of t6, the rest under the root
    par = np.full(n, -1, dtype=np.int32)
    par[idx["t6"]] = idx["t3"]
    for t in fx["under_t6"]:
        par[idx[t]] = idx["t6"]
    tok = np.array([int(t[1:]) for t in toks], dtype=np.int32)
    P, Hkv, d = 5, 1, 64
    k = torch.arange((P + n) * Hkv * d, dtype=torch.float32).reshape(1, P + n, Hkv, d).cuda()
    v = -k
    kv = ta.KVCache(k, v)
    d_par, d_tok = dev_tensor(par[None].copy()), dev_tensor(tok[None].copy())
    d_P, d_n = dev_tensor(np.array([P], np.int32)), dev_tensor(np.array([n], np.int32))
    ver = dev_tensor(np.array([[3, 6]], np.int32))
    path, plen, keep = ta.tree_token_walk(d_par, d_tok, d_n, ver, dev_tensor(np.array([2], np.int32)))
    torch.cuda.synchronize()
    assert plen.item() == 2 and keep.item() == 1
    assert path[0, :2].tolist() == [idx["t3"], idx["t6"]]
    ta.tree_cache_reroot_draft([kv], d_P, d_par, d_n, path, plen, keep, d_tok)
    torch.cuda.synchronize()
    assert d_P.item() == P + 2 and d_n.item() == len(fx["iter1"]["expected_tree"])
    # the draft's next tree is t9..t12, moved on the device with their KV rows
    m = len(fx["iter1"]["expected_tree"])
    assert d_tok.cpu().numpy()[0, :m].tolist() == [int(t[1:]) for t in fx["iter1"]["expected_tree"]]
    kk = k.cpu().numpy()[0]
    for j, t in enumerate(fx["iter1"]["expected_tree"]):
        np.testing.assert_array_equal(kv.k.cpu().numpy()[0, P + 2 + j], kk[P + idx[t]])
    # iteration 2 walks the re-rooted tree with the tokens the re-root left
    path2, plen2, keep2 = ta.tree_token_walk(d_par, d_tok, d_n,
                                             dev_tensor(np.array([[9, 16]], np.int32)),
                                             dev_tensor(np.array([2], np.int32)))
    torch.cuda.synchronize()
    assert [fx["iter1"]["expected_tree"][i] for i in path2[0, :plen2.item()].tolist()] == \
        fx["iter2"]["path"]
    assert keep2.item() == int(fx["iter2"]["keep"])
    ta.tree_cache_reroot_draft([kv], d_P, d_par, d_n, path2, plen2, keep2, d_tok)
    torch.cuda.synchronize()
    assert d_n.item() == fx["iter2"]["expected_n_nodes"] and d_P.item() == P + 3
    assert (d_tok.cpu().numpy() == -1).all()


@pytest.mark.parametrize("seed,n_max,bs,uniform", [(1, 16, 4, False), (2, 64, 16, False),
                                                   (3, 256, 64, False), (4, 256, 256, False),
                                                   (5, 40, 8, True)])
def test_select_subtree_random_trees(ta, seed, n_max, bs, uniform):
    import torch
    rng = np.random.default_rng([seed, 51])
    B = 6
    par = np.full((B, n_max), -1, dtype=np.int32)
    tok = np.zeros((B, n_max), dtype=np.int32)
    cum = np.zeros((B, n_max), dtype=np.float32)
    n = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n[b] = [n_max, 0, 1, bs // 2, int(rng.integers(1, n_max + 1)), n_max][b]
        par[b], tok[b] = _tree(rng, int(n[b]), n_max)
        V = int(tok[b].max()) + 1
        lg = np.zeros((n_max + 1, V)) if uniform else rng.standard_normal((n_max + 1, V))
        cum[b, :n[b]] = oracle.cumulative_scores(par[b], tok[b], lg[0], lg[1:], int(n[b]))
    cum[4, 0] = np.nan                                   # NaN ranks last
    sn, sp, st, sc = ta.tree_select_subtree(dev_tensor(cum), dev_tensor(par), dev_tensor(tok),
                                            dev_tensor(n), bs)
    torch.cuda.synchronize()
    sn, sp, st, sc = (x.cpu().numpy() for x in (sn, sp, st, sc))
    for b in range(B):
        c64 = cum[b].astype(np.float64)
        c64[np.isnan(c64)] = -np.inf
        nodes, new_par, toks = oracle.select_subtree(par[b], tok[b], c64, int(n[b]), bs)
        k = len(nodes)
        assert sc[b] == k
        assert sn[b, :k].tolist() == nodes.tolist()
        assert st[b, :k].tolist() == toks.tolist()
        assert sp[b, :k].tolist() == new_par.tolist()
        assert (sn[b, k:] == -1).all() and (sp[b, k:] == -1).all() and (st[b, k:] == 0).all()


def _kv_bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("seed,n_max,paged", [(1, 16, False), (2, 64, True), (3, 256, False),
                                              (4, 40, True)])
def test_reroot_draft_moves_tokens_and_weights(ta, seed, n_max, paged):
    import torch
    from gen import random_case
    c = random_case(400 + seed, B=8, Hq=2, Hkv=2, d=64, P_range=(0, 50), n_max=n_max,
                    n_range=(0, n_max), dtype="bf16", paged=paged, block_size=8)
    rng = np.random.default_rng([seed, 52])
    B = c.B
    tok = rng.integers(0, 1000, size=(B, n_max)).astype(np.int32)
    cum = (-np.abs(rng.standard_normal((B, n_max))) * 5).astype(np.float32)
    path = np.full((B, n_max), -1, dtype=np.int32)
    plen = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(c.n_nodes[b])
        if n == 0 or b == 1:
            continue                                  # k = 0 cases
        rp = oracle.root_path(c.parent[b], int(rng.integers(0, n)))
        cut = int(rng.integers(1, len(rp) + 1))
        path[b, :cut] = rp[:cut]
        plen[b] = cut
    keep = np.array([(b % 3) != 0 for b in range(B)], dtype=np.uint8)
    from helpers import DevCase
    dc = DevCase(c)
    d_tok, d_cum = dev_tensor(tok), dev_tensor(cum)
    ta.tree_cache_reroot_draft([dc.kv], dc.prefix_len, dc.parent, dc.n_nodes, dev_tensor(path),
                               dev_tensor(plen), dev_tensor(keep), d_tok, d_cum)
    torch.cuda.synchronize()
    layers, P1, par1, n1 = oracle.tree_cache_reroot([(c.k, c.v)], c.prefix_len, c.parent,
                                                    c.n_nodes, path, plen, keep.astype(bool),
                                                    c.block_table, c.block_size)
    np.testing.assert_array_equal(dc.prefix_len.cpu().numpy(), P1)
    np.testing.assert_array_equal(dc.n_nodes.cpu().numpy(), n1)
    np.testing.assert_array_equal(dc.parent.cpu().numpy(), par1)
    gt, gc = d_tok.cpu().numpy(), d_cum.cpu().numpy()
    for b in range(B):
        wt, wc = oracle.reroot_node_arrays(c.parent[b], int(c.n_nodes[b]), path[b],
                                           int(plen[b]), bool(keep[b]), tok[b], cum[b])
        np.testing.assert_array_equal(gt[b], wt)
        np.testing.assert_array_equal(gc[b].view(np.int32), wc.view(np.int32))
    kg, vg = _kv_bits(dc.k), _kv_bits(dc.v)
    kr, vr = layers[0][0].view(np.int16), layers[0][1].view(np.int16)
    for b in range(B):
        for t in range(int(P1[b] + n1[b])):
            if paged:
                blk, sl = c.block_table[b, t // c.block_size], t % c.block_size
                assert (kg[blk, sl] == kr[blk, sl]).all() and (vg[blk, sl] == vr[blk, sl]).all()
            else:
                assert (kg[b, t] == kr[b, t]).all() and (vg[b, t] == vr[b, t]).all()


SCORE_TOL = 2e-4  # fp32 log-softmax of a 32000-way row against fp64: a few 1e-6


@pytest.mark.parametrize("extend", ["keep", "absent"])
def test_draft_iteration_on_device(ta, extend):
    """SwiftSpec summary, Section 3.1.1 Algorithm 1 on the device: four
    maximum-likelihood expansions (tree_expand_top_w, Section 3.1.3), the walk
    along the verified tokens (Synchronize), the re-root that moves the KV and
    the draft's tokens and weights (Re-root, Section 3.2), then Select.  The
    oracle runs its own chain from the same seeded inputs; the seeded scores
    are separated by more than the fp32 error wherever a choice is made, so
    every step is compared exactly (weights within the fp32 error)."""
    import torch
    from gen import config4_expand
    c = config4_expand()
    n_max, V, w, n0 = c.n_max, c.vocab, c.w, c.n0
    rows = np.zeros((n_max + 1, V), dtype=np.float32)   # row 0: root, row 1 + i: node i
    rows[0] = c.logits_root
    rows[1:n0 + 1] = c.logits0
    for r in range(c.rounds):
        rows[n0 + r * w + 1: n0 + (r + 1) * w + 1] = c.logits_new[r]
    # ---- oracle chain ----
    par = np.full(n_max, -1, dtype=np.int32)
    tok = np.full(n_max, -1, dtype=np.int32)
    par[:n0], tok[:n0] = c.parent0, c.tok0
    n = n0
    for r in range(c.rounds):
        cum64 = oracle.cumulative_scores(par, tok, rows[0], rows[1:], n)
        p, t, sc = oracle.select_top_w(par, tok, cum64, rows[0], rows[1:], n, w + 1)
        assert np.all(np.diff(-sc) > SCORE_TOL), "seeded scores separated at every pick"
        par[n:n + w], tok[n:n + w] = p[:w], t[:w]
        n += w
    cum64 = oracle.cumulative_scores(par, tok, rows[0], rows[1:], n)
    # verified tokens: the root path of the node at depth >= 2 with the largest
    # subtree (the re-root then keeps that subtree), optionally followed by a
    # token outside the tree (then a new tree starts)
    deep = [i for i in range(n) if oracle.depth(par, i) >= 2]
    x = max(deep, key=lambda i: (len(oracle.descendants(par, i, n)), -i))
    verified = [int(tok[u]) for u in oracle.root_path(par, x)]
    if extend == "absent":
        verified.append(V + 7)
    o_path, o_keep = oracle.token_walk(par, tok, n, verified)
    o_layers, o_P, o_par, o_n = oracle.tree_cache_reroot(
        [(c.k, c.v)], np.array([c.P]), par[None], np.array([n]),
        np.array([o_path + [-1] * (n_max - len(o_path))]), np.array([len(o_path)]),
        np.array([o_keep]))
    o_tok, o_cum = oracle.reroot_node_arrays(par, n, o_path, len(o_path), o_keep, tok,
                                             cum64.astype(np.float32))
    o_cum64 = np.array([cum64[u] for u in oracle.descendants(par, o_path[-1], n)]) - \
        cum64[o_path[-1]] if o_keep else np.zeros(0)
    bs = 8
    nn = int(o_n[0])
    # ---- device chain ----
    d_lg = dev_tensor(rows[None].copy())
    d_par = dev_tensor(np.r_[c.parent0, np.full(n_max - n0, -1)].astype(np.int32)[None].copy())
    d_tok = dev_tensor(np.r_[c.tok0, np.full(n_max - n0, -1)].astype(np.int32)[None].copy())
    cum0 = np.full(n_max, -np.inf, dtype=np.float32)
    cum0[:n0] = oracle.cumulative_scores(c.parent0, c.tok0, rows[0], rows[1:], n0)
    d_cum = dev_tensor(cum0[None].copy())
    d_n = dev_tensor(np.array([n0], np.int32))
    d_P = dev_tensor(np.array([c.P], np.int32))
    kv = ta.KVCache(dev_tensor(c.k, "bf16"), dev_tensor(c.v, "bf16"))
    for r in range(c.rounds):
        ta.tree_expand_top_w(d_lg, d_par, d_tok, d_cum, d_n, w)
    d_ver = dev_tensor(np.array([verified], np.int32))
    path, plen, keep = ta.tree_token_walk(d_par, d_tok, d_n, d_ver,
                                          dev_tensor(np.array([len(verified)], np.int32)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_par.cpu().numpy()[0], par)
    np.testing.assert_array_equal(d_tok.cpu().numpy()[0], tok)
    np.testing.assert_allclose(d_cum.cpu().numpy()[0], cum64, rtol=1e-5, atol=SCORE_TOL)
    assert plen.item() == len(o_path) and keep.item() == int(o_keep)
    assert path.cpu().numpy()[0, :len(o_path)].tolist() == o_path
    ta.tree_cache_reroot_draft([kv], d_P, d_par, d_n, path, plen, keep, d_tok, d_cum)
    sel = ta.tree_select_subtree(d_cum, d_par, d_tok, d_n, bs)
    torch.cuda.synchronize()
    assert d_P.item() == int(o_P[0]) and d_n.item() == nn
    np.testing.assert_array_equal(d_par.cpu().numpy()[0], o_par[0])
    np.testing.assert_array_equal(d_tok.cpu().numpy()[0], o_tok)
    gcum = d_cum.cpu().numpy()[0]
    np.testing.assert_allclose(gcum[:nn], o_cum64, rtol=1e-5, atol=SCORE_TOL)
    assert np.all(np.isneginf(gcum[nn:]))
    kb = kv.k.view(torch.int16).cpu().numpy()[0]
    vb = kv.v.view(torch.int16).cpu().numpy()[0]
    end_row = int(o_P[0]) + nn
    np.testing.assert_array_equal(kb[:end_row], o_layers[0][0].view(np.int16)[0, :end_row])
    np.testing.assert_array_equal(vb[:end_row], o_layers[0][1].view(np.int16)[0, :end_row])
    # Select on the re-rooted tree (the oracle's own weights)
    o_sel = oracle.select_subtree(o_par[0], o_tok, o_cum64, nn, bs)
    order = np.sort(o_cum64)[::-1]
    if nn > bs:
        assert order[bs - 1] - order[bs] > SCORE_TOL, "seeded weights separated at the cut"
    k_sel = len(o_sel[0])
    sn, sp, st, sc = (x.cpu().numpy()[0] for x in sel)
    assert sc == k_sel
    assert sn[:k_sel].tolist() == o_sel[0].tolist()
    assert sp[:k_sel].tolist() == o_sel[1].tolist()
    assert st[:k_sel].tolist() == o_sel[2].tolist()
    if extend == "keep":
        assert o_keep and nn > bs
    else:
        assert not o_keep and nn == 0
