"""GPU parity of the draft-side entry points against the oracle
(oracle/draft.py): tree_token_walk (bit-exact path, length, keep flag) and
tree_select_subtree (bit-exact nodes, renumbered parents, tokens), including
Figure 2 chained through the GPU re-root."""
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
    ta.tree_cache_reroot([kv], d_P, d_par, d_n, path, plen, keep)
    torch.cuda.synchronize()
    assert d_P.item() == P + 2 and d_n.item() == len(fx["iter1"]["expected_tree"])
    # the kept nodes' tokens in their new order (the caller moves tok like parent)
    tok1 = np.array([int(t[1:]) for t in fx["iter1"]["expected_tree"]] + [0] * (n - 4), np.int32)
    path2, plen2, keep2 = ta.tree_token_walk(d_par, dev_tensor(tok1[None]), d_n,
                                             dev_tensor(np.array([[9, 16]], np.int32)),
                                             dev_tensor(np.array([2], np.int32)))
    torch.cuda.synchronize()
    assert [fx["iter1"]["expected_tree"][i] for i in path2[0, :plen2.item()].tolist()] == \
        fx["iter2"]["path"]
    assert keep2.item() == int(fx["iter2"]["keep"])


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
