"""The five seeded workloads at full size, in the launch configuration the
benchmark uses (automatic kernel and split choice), against the oracle.
The chain-verify attention (2.1 GB of KV) is compared in
test_gpu_fullsize.py, every block, with structured inputs beside it."""
import numpy as np
import pytest

from helpers import DevCase, assert_attn_close, dev_tensor, ensure_built, to_f64

import oracle
from gen import config2_chain, config3_tree, config4_expand, config5_paged

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _verify(ta, dc):
    import torch
    c = dc.case
    out, lse = ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


def _accept_and_reroot(ta, dc, keep):
    import torch
    c = dc.case
    path, plen, bonus = ta.accept_greedy_path(dc.logits, dc.parent, dc.tok, dc.n_nodes,
                                              dc.root_tok)
    torch.cuda.synchronize()
    pr, lr, br = oracle.accept_greedy_path(c.logits, c.parent, c.tok, c.n_nodes, c.root_tok)
    np.testing.assert_array_equal(plen.cpu().numpy(), lr)
    np.testing.assert_array_equal(path.cpu().numpy(), pr)
    np.testing.assert_array_equal(bonus.cpu().numpy(), br)
    keep_np = np.full(c.B, keep, dtype=np.uint8)
    ta.tree_cache_reroot([dc.kv], dc.prefix_len, dc.parent, dc.n_nodes, path, plen,
                         dev_tensor(keep_np))
    torch.cuda.synchronize()
    _, P1, par1, n1 = oracle.tree_cache_reroot([], c.prefix_len, c.parent, c.n_nodes, pr, lr,
                                               keep_np.astype(bool))
    np.testing.assert_array_equal(dc.prefix_len.cpu().numpy(), P1)
    np.testing.assert_array_equal(dc.n_nodes.cpu().numpy(), n1)
    np.testing.assert_array_equal(dc.parent.cpu().numpy(), par1)
    return pr, lr


def test_config3_llama70b_share(ta):
    c = config3_tree()
    dc = DevCase(c)
    O, L = _verify(ta, dc)
    Or, Lr = oracle.verify(c)
    assert_attn_close(O, L, Or, Lr, "bf16", what="config3")
    pr, lr = _accept_and_reroot(ta, dc, keep=False)
    assert lr.tolist() == c.planted["path_len"]


def test_config3_keep_subtree_compaction(ta):
    """keep=true variant: real row moves, checked byte for byte."""
    import torch
    c = config3_tree()
    dc = DevCase(c)
    pr, lr, br = oracle.accept_greedy_path(c.logits, c.parent, c.tok, c.n_nodes, c.root_tok)
    keep_np = np.ones(c.B, dtype=np.uint8)
    ta.tree_cache_reroot([dc.kv], dc.prefix_len, dc.parent, dc.n_nodes, dev_tensor(pr),
                         dev_tensor(lr), dev_tensor(keep_np))
    torch.cuda.synchronize()
    layers, P1, par1, n1 = oracle.tree_cache_reroot([(c.k, c.v)], c.prefix_len, c.parent,
                                                    c.n_nodes, pr, lr, keep_np.astype(bool))
    lk, lv = layers[0]
    kg = dc.k.view(torch.int16).cpu().numpy()
    vg = dc.v.view(torch.int16).cpu().numpy()
    for b in range(c.B):
        e = int(P1[b] + n1[b])
        np.testing.assert_array_equal(kg[b, :e], lk.view(np.int16)[b, :e])
        np.testing.assert_array_equal(vg[b, :e], lv.view(np.int16)[b, :e])
    np.testing.assert_array_equal(dc.parent.cpu().numpy(), par1)


def test_config5_paged_alternating(ta):
    c = config5_paged()
    m = c.planted["batch_size"]
    dc = DevCase(c)
    for s in (0, 1, 0):
        sl = slice(s * m, (s + 1) * m)
        bt = dc.block_table[sl].contiguous()
        kv = ta.KVCache(dc.k, dc.v, bt, T_cap=c.T_cap)
        out, lse = ta.tree_attn_verify(dc.q[sl].contiguous(), kv, dc.prefix_len[sl].contiguous(),
                                       dc.parent[sl].contiguous(), dc.n_nodes[sl].contiguous(),
                                       c.scale)
        import torch
        torch.cuda.synchronize()
        sub = _subcase(c, sl)
        Or, Lr = oracle.verify(sub)
        assert_attn_close(to_f64(out), lse.cpu().numpy(), Or, Lr, "bf16", what=f"batch {s}")
    pr, lr, br = oracle.accept_greedy_path(c.logits, c.parent, c.tok, c.n_nodes, c.root_tok)
    assert lr.tolist() == c.planted["path_len"]
    _accept_and_reroot(ta, dc, keep=False)


def _subcase(c, sl):
    import copy
    s = copy.copy(c)
    s.q = c.q[sl]
    s.prefix_len = c.prefix_len[sl]
    s.parent = c.parent[sl]
    s.n_nodes = c.n_nodes[sl]
    s.block_table = c.block_table[sl]
    s.B = s.q.shape[0]
    return s


def test_config4_draft_expansion_rounds(ta):
    import torch
    c = config4_expand()
    par = np.full(c.n_max, -1, dtype=np.int32)
    tok = np.zeros(c.n_max, dtype=np.int32)
    par[: c.n0] = c.parent0
    tok[: c.n0] = c.tok0
    rows = c.logits0.copy()
    n = c.n0
    k = dev_tensor(c.k, "bf16")
    v = dev_tensor(c.v, "bf16")
    kv = ta.KVCache(k, v)
    d_P = dev_tensor(np.array([c.P], np.int32))
    d_par = dev_tensor(par[None].copy())
    d_n = dev_tensor(np.array([n], np.int32))
    for r in range(c.rounds):
        cum = oracle.cumulative_scores(par, tok, c.logits_root, rows, n)
        p, t, _ = oracle.select_top_w(par, tok, cum, c.logits_root, rows, n, c.w)
        par[n: n + c.w] = p
        tok[n: n + c.w] = t
        n += c.w
        d_par.copy_(dev_tensor(par[None].copy()))
        d_n.fill_(n)
        q = dev_tensor(c.q_new[r], "bf16")
        out, lse = ta.tree_attn_expand(q, kv, d_P, d_par, d_n, c.scale)
        torch.cuda.synchronize()

        class _C:
            pass
        oc = _C()
        oc.B, oc.Hq, oc.d, oc.G, oc.scale, oc.dtype = 1, c.Hq, c.d, c.Hq // c.Hkv, c.scale, "bf16"
        oc.prefix_len, oc.n_nodes, oc.parent = np.array([c.P]), np.array([n]), par[None]
        oc.k, oc.v, oc.block_table, oc.block_size = c.k, c.v, None, 0
        Or, Lr = oracle.expand(oc, c.q_new[r], c.w)
        assert Or.shape[1] == 8 and c.P + n == 2048 + 64 + 8 * (r + 1)
        assert_attn_close(to_f64(out), lse.cpu().numpy(), Or, Lr, "bf16", what=f"round {r}")
        rows = np.r_[rows, c.logits_new[r]]


def test_config2_chain_accept_reroot(ta):
    """Accept and re-root on the chain-verify workload (its attention is
    compared block by block in test_gpu_fullsize.py)."""
    import torch
    c = config2_chain()
    dc = DevCase(c)
    pr, lr = _accept_and_reroot(ta, dc, keep=False)
    assert lr.tolist() == c.planted["path_len"]
    del dc
    torch.cuda.empty_cache()
