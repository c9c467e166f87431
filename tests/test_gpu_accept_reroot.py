"""GPU parity of accept_greedy_path and tree_cache_reroot against the oracle
(bit-exact: indices, lengths, bonus tokens, parents, compacted KV bytes)."""
import numpy as np
import pytest

from helpers import DevCase, dev_tensor, ensure_built

import oracle
from gen import config1_tiny, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _accept(ta, dc, logits=None):
    import torch
    path, plen, bonus = ta.accept_greedy_path(dc.logits if logits is None else logits, dc.parent,
                                              dc.tok, dc.n_nodes, dc.root_tok)
    torch.cuda.synchronize()
    return path.cpu().numpy(), plen.cpu().numpy(), bonus.cpu().numpy()


@pytest.mark.parametrize("seed,target_side,n_max,vocab", [
    (1, False, 16, 256), (2, True, 16, 32000), (3, False, 64, 1000), (4, True, 256, 300),
    (5, False, 7, 33), (6, True, 1, 50)])
def test_accept_random(ta, seed, target_side, n_max, vocab):
    c = random_case(seed, B=9, Hq=1, Hkv=1, d=64, P_range=(0, 2), n_max=n_max, dtype="f32",
                    target_side=target_side, vocab=vocab)
    dc = DevCase(c)
    p, l, bo = _accept(ta, dc)
    pr, lr, br = oracle.accept_greedy_path(c.logits, c.parent, c.tok, c.n_nodes, c.root_tok)
    np.testing.assert_array_equal(l, lr)
    np.testing.assert_array_equal(p, pr)
    np.testing.assert_array_equal(bo, br)
    assert l.tolist() == c.planted["path_len"]


def test_accept_bf16_logits_and_ties(ta):
    import torch
    c = random_case(12, B=5, Hq=1, Hkv=1, d=64, P_range=(0, 2), n_max=10, dtype="f32",
                    vocab=600)
    # bf16 logits: round, then plant exact ties (two equal maxima) in some rows
    lg = torch.from_numpy(c.logits).to(torch.bfloat16)
    lg[:, :, 5] = 40.0
    lg[:, :, 17] = 40.0
    logits_np = lg.float().numpy()
    dc = DevCase(c)
    p, l, bo = _accept(ta, dc, lg.cuda())
    pr, lr, br = oracle.accept_greedy_path(logits_np, c.parent, c.tok, c.n_nodes, c.root_tok)
    np.testing.assert_array_equal(l, lr)
    np.testing.assert_array_equal(p, pr)
    np.testing.assert_array_equal(bo, br)


def test_accept_tiny_config(ta):
    c = config1_tiny()
    dc = DevCase(c)
    p, l, bo = _accept(ta, dc)
    pr, lr, br = oracle.accept_greedy_path(c.logits, c.parent, c.tok, c.n_nodes, c.root_tok)
    np.testing.assert_array_equal(p, pr)
    np.testing.assert_array_equal(l, lr)
    np.testing.assert_array_equal(bo, br)


def _kv_bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _reroot_case(ta, c, keep, n_layers=2, seed=0):
    """Run GPU and oracle re-root; compare metadata and every moved byte."""
    import torch
    rng = np.random.default_rng(seed)
    B = c.B
    path = np.full((B, c.n_max), -1, dtype=np.int32)
    plen = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(c.n_nodes[b])
        if n == 0:
            continue
        end = int(rng.integers(0, n))
        rp = oracle.root_path(c.parent[b], end)
        cut = int(rng.integers(0, len(rp) + 1))
        path[b, :cut] = rp[:cut]
        plen[b] = cut
    keep_np = np.array([keep if isinstance(keep, bool) else bool(rng.integers(0, 2))
                        for _ in range(B)], dtype=np.uint8)
    # extra layers are perturbed copies of layer 0 (distinct bytes per layer)
    layers_np = []
    for L in range(n_layers):
        if c.dtype == "bf16":
            kL = (c.k.astype(np.uint32) + 3 * L).astype(np.uint16)
            vL = (c.v.astype(np.uint32) + 5 * L).astype(np.uint16)
        else:
            kL = c.k + np.float32(L)
            vL = c.v - np.float32(L)
        layers_np.append((kL, vL))
    dc = DevCase(c)
    layers = [ta.KVCache(dev_tensor(k, c.dtype), dev_tensor(v, c.dtype), dc.block_table,
                         T_cap=c.T_cap if c.paged else None) for k, v in layers_np]
    d_path = dev_tensor(path)
    d_plen = dev_tensor(plen)
    d_keep = dev_tensor(keep_np)
    ta.tree_cache_reroot(layers, dc.prefix_len, dc.parent, dc.n_nodes, d_path, d_plen, d_keep)
    torch.cuda.synchronize()
    new_layers, P1, par1, n1 = oracle.tree_cache_reroot(layers_np, c.prefix_len, c.parent,
                                                        c.n_nodes, path, plen, keep_np.astype(bool),
                                                        c.block_table, c.block_size)
    np.testing.assert_array_equal(dc.prefix_len.cpu().numpy(), P1)
    np.testing.assert_array_equal(dc.n_nodes.cpu().numpy(), n1)
    np.testing.assert_array_equal(dc.parent.cpu().numpy(), par1)
    for L, ((k_ref, v_ref), lay) in enumerate(zip(new_layers, layers)):
        kg, vg = _kv_bits(lay.k), _kv_bits(lay.v)
        kr = k_ref.view(np.int16 if c.dtype == "bf16" else np.int32)
        vr = v_ref.view(np.int16 if c.dtype == "bf16" else np.int32)
        for b in range(B):
            end = int(P1[b] + n1[b])
            if c.paged:
                for t in range(end):
                    blk, s = c.block_table[b, t // c.block_size], t % c.block_size
                    assert (kg[blk, s] == kr[blk, s]).all() and (vg[blk, s] == vr[blk, s]).all()
            else:
                np.testing.assert_array_equal(kg[b, :end], kr[b, :end])
                np.testing.assert_array_equal(vg[b, :end], vr[b, :end])
    return plen, n1


@pytest.mark.parametrize("seed,dtype,d,paged,keep", [
    (1, "bf16", 128, False, True), (2, "bf16", 128, False, False), (3, "f32", 64, False, None),
    (4, "bf16", 64, True, True), (5, "f32", 128, True, None), (6, "bf16", 128, False, None)])
def test_reroot_random(ta, seed, dtype, d, paged, keep):
    c = random_case(100 + seed, B=6, Hq=4, Hkv=2, d=d, P_range=(0, 90), n_max=24,
                    n_range=(0, 24), dtype=dtype, paged=paged, block_size=8)
    _reroot_case(ta, c, keep, n_layers=3, seed=seed)


def test_reroot_max_tree_and_many_layers(ta):
    c = random_case(200, B=2, Hq=2, Hkv=1, d=128, P_range=(5, 9), n_max=256,
                    n_range=(200, 256), dtype="f32")
    _reroot_case(ta, c, True, n_layers=40, seed=3)    # > 32 layers: two move launches


def test_reroot_fig4_on_gpu(ta, golden):
    import torch
    fx = golden("fig4_reroot.json")
    toks = fx["tree_tokens"]
    idx = {t: i for i, t in enumerate(toks)}
    P, n = len(fx["prefix_tokens"]), len(toks)
    par = np.array([-1, -1, 0, 1, 1, 2, 4, 4], dtype=np.int32)   # one tree the caption allows
    assert par[idx["t12"]] == -1 and par[idx["t15"]] == idx["t12"]
    T = P + n + 2
    k = np.arange(T * 128, dtype=np.float32).reshape(1, T, 1, 128)
    v = -k
    kv = ta.KVCache(dev_tensor(k), dev_tensor(v))
    d_P = dev_tensor(np.array([P], np.int32))
    d_par = dev_tensor(par[None].copy())
    d_n = dev_tensor(np.array([n], np.int32))
    path = np.full((1, n), -1, np.int32)
    path[0, :2] = [idx[t] for t in fx["path"]]
    ta.tree_cache_reroot([kv], d_P, d_par, d_n, dev_tensor(path), dev_tensor(np.array([2], np.int32)),
                         dev_tensor(np.array([1], np.uint8)))
    torch.cuda.synchronize()
    assert d_P.item() == fx["expected_prefix_len"] and d_n.item() == fx["expected_n_nodes"]
    assert d_par.cpu().numpy()[0, :2].tolist() == fx["expected_parent"]
    kk = kv.k.cpu().numpy()
    for row, old in fx["expected_rows_old_position"].items():
        np.testing.assert_array_equal(kk[0, int(row)], k[0, old])


def _duplicate_sibling_case(seed, B, n_max, vocab):
    """Trees whose siblings often share a token (tokens drawn from a tiny
    vocabulary) and integer-valued logits (frequent argmax ties), so that
    several accepted nodes reach the maximum depth: the deepest-then-lowest-
    index rule (draft-length co-design article, Acceptance Length: the
    longest accepted path) decides between them."""
    rng = np.random.default_rng([seed, 31])
    parent = np.full((B, n_max), -1, dtype=np.int32)
    n_nodes = rng.integers(1, n_max + 1, size=B).astype(np.int32)
    for b in range(B):
        for i in range(1, int(n_nodes[b])):
            parent[b, i] = rng.integers(-1, i) if seed % 2 else rng.integers(max(-1, i - 3), i)
    tok = rng.integers(0, vocab, size=(B, n_max)).astype(np.int32)
    logits = rng.integers(-2, 3, size=(B, n_max, vocab)).astype(np.float32)
    root_tok = np.array([tok[b, 0] for b in range(B)], dtype=np.int32)
    return parent, tok, logits, root_tok, n_nodes


def _tied_deepest(parent, tok, logits, root_tok, n):
    """Number of accepted nodes at the maximum accepted depth (brute force)."""
    a = [oracle.argmax_first(logits[i]) for i in range(n)]
    depths = []
    for i in range(n):
        rp = oracle.root_path(parent, i)
        ok = tok[rp[0]] == root_tok and all(tok[y] == a[x] for x, y in zip(rp[:-1], rp[1:]))
        if ok:
            depths.append(len(rp))
    return depths.count(max(depths)) if depths else 0


@pytest.mark.parametrize("seed,n_max,vocab,ldt", [
    (1, 12, 2, "f32"), (2, 24, 2, "f32"), (3, 64, 2, "bf16"), (4, 256, 2, "f32"),
    (5, 40, 3, "bf16")])
def test_accept_duplicate_sibling_ties(ta, seed, n_max, vocab, ldt):
    import torch
    B = 48
    parent, tok, logits, root_tok, n_nodes = _duplicate_sibling_case(seed, B, n_max, vocab)
    ties = sum(_tied_deepest(parent[b], tok[b], logits[b], root_tok[b], int(n_nodes[b])) >= 2
               for b in range(B))
    assert ties >= B // 8, "the case must exercise ties between deepest accepted nodes"
    lg = torch.from_numpy(logits)
    if ldt == "bf16":
        lg = lg.to(torch.bfloat16)      # small integers: exact in bf16
    path, plen, bonus = ta.accept_greedy_path(lg.cuda(), dev_tensor(parent), dev_tensor(tok),
                                              dev_tensor(n_nodes), dev_tensor(root_tok))
    torch.cuda.synchronize()
    pr, lr, br = oracle.accept_greedy_path(logits, parent, tok, n_nodes, root_tok)
    np.testing.assert_array_equal(plen.cpu().numpy(), lr)
    np.testing.assert_array_equal(path.cpu().numpy(), pr)
    np.testing.assert_array_equal(bonus.cpu().numpy(), br)


@pytest.mark.parametrize("seed,keep", [(11, True), (12, False), (13, None)])
def test_accept_then_reroot_with_duplicate_siblings(ta, seed, keep):
    """The GPU's accepted path feeds the GPU re-root on duplicate-sibling
    trees; paths, metadata and every kept KV byte against the oracle."""
    import torch
    B, n_max, Hkv, d = 24, 48, 2, 128
    parent, tok, logits, root_tok, n_nodes = _duplicate_sibling_case(seed, B, n_max, 2)
    rng = np.random.default_rng(seed)
    P = rng.integers(0, 40, size=B).astype(np.int32)
    T_cap = int(P.max()) + n_max
    k = rng.standard_normal((B, T_cap, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, T_cap, Hkv, d), dtype=np.float32)
    keep_np = np.array([keep if keep is not None else bool(rng.integers(0, 2))
                        for _ in range(B)], dtype=np.uint8)
    d_par, d_P, d_n = dev_tensor(parent), dev_tensor(P), dev_tensor(n_nodes)
    kv = ta.KVCache(dev_tensor(k), dev_tensor(v))
    path, plen, bonus = ta.accept_greedy_path(dev_tensor(logits), d_par, dev_tensor(tok), d_n,
                                              dev_tensor(root_tok))
    ta.tree_cache_reroot([kv], d_P, d_par, d_n, path, plen, dev_tensor(keep_np))
    torch.cuda.synchronize()
    pr, lr, br = oracle.accept_greedy_path(logits, parent, tok, n_nodes, root_tok)
    np.testing.assert_array_equal(path.cpu().numpy(), pr)
    np.testing.assert_array_equal(plen.cpu().numpy(), lr)
    np.testing.assert_array_equal(bonus.cpu().numpy(), br)
    layers, P1, par1, n1 = oracle.tree_cache_reroot([(k, v)], P, parent, n_nodes, pr, lr,
                                                    keep_np.astype(bool))
    np.testing.assert_array_equal(d_P.cpu().numpy(), P1)
    np.testing.assert_array_equal(d_n.cpu().numpy(), n1)
    np.testing.assert_array_equal(d_par.cpu().numpy(), par1)
    kg, vg = _kv_bits(kv.k), _kv_bits(kv.v)
    kr, vr = layers[0][0].view(np.int32), layers[0][1].view(np.int32)
    for b in range(B):
        e = int(P1[b] + n1[b])
        np.testing.assert_array_equal(kg[b, :e], kr[b, :e])
        np.testing.assert_array_equal(vg[b, :e], vr[b, :e])
