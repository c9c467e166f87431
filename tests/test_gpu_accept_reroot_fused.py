"""tree_accept_reroot (greedy acceptance and re-root in two launches) against
the same work done by accept_greedy_path then tree_cache_reroot, bit for bit:
the path outputs, prefix_len / parent / n_nodes and every byte of every
layer's cache (rows past the new end included: both move the same rows), and
against the oracle (paths, metadata, kept rows).

The fused launch's work groups each find the path themselves from a copy of
the metadata the argmax launch took, and one group per sequence rewrites the
live metadata; the cases cover several launches of layers, no layers, many
sequences, repeated calls on one workspace with changing batch sizes and
stray bytes in it, paged and contiguous caches, empty trees and ties between
deepest accepted nodes."""
import numpy as np
import pytest

from helpers import DevCase, dev_tensor, ensure_built

import oracle
from gen import random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _layers_np(c, n_layers):
    out = []
    for L in range(n_layers):
        if c.dtype == "bf16":
            out.append(((c.k.astype(np.uint32) + 3 * L).astype(np.uint16),
                        (c.v.astype(np.uint32) + 5 * L).astype(np.uint16)))
        else:
            out.append((c.k + np.float32(L), c.v - np.float32(L)))
    return out


def _device_state(ta, c, layers_np, keep_np):
    dc = DevCase(c)
    layers = [ta.KVCache(dev_tensor(k, c.dtype), dev_tensor(v, c.dtype), dc.block_table,
                         T_cap=c.T_cap if c.paged else None) for k, v in layers_np]
    return dc, layers, dev_tensor(keep_np)


def _check_case(ta, c, keep_np, n_layers, ws=None, oracle_rows=True):
    import torch
    layers_np = _layers_np(c, n_layers)
    A, la, ka = _device_state(ta, c, layers_np, keep_np)
    F, lf, kf = _device_state(ta, c, layers_np, keep_np)
    path_a, plen_a, bonus_a = ta.accept_greedy_path(A.logits, A.parent, A.tok, A.n_nodes,
                                                    A.root_tok)
    ta.tree_cache_reroot(la, A.prefix_len, A.parent, A.n_nodes, path_a, plen_a, ka)
    path_f, plen_f, bonus_f = ta.tree_accept_reroot(F.logits, F.tok, F.root_tok, lf, F.prefix_len,
                                                    F.parent, F.n_nodes, kf, workspace=ws)
    torch.cuda.synchronize()
    for x, y in ((path_a, path_f), (plen_a, plen_f), (bonus_a, bonus_f), (A.prefix_len, F.prefix_len),
                 (A.parent, F.parent), (A.n_nodes, F.n_nodes)):
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy())
    for a, f in zip(la, lf):
        np.testing.assert_array_equal(_bits(a.k), _bits(f.k))
        np.testing.assert_array_equal(_bits(a.v), _bits(f.v))
    # the oracle: greedy path, then the re-root on it
    pr, lr, br = oracle.accept_greedy_path(c.logits, c.parent, c.tok, c.n_nodes, c.root_tok)
    np.testing.assert_array_equal(path_f.cpu().numpy(), pr)
    np.testing.assert_array_equal(plen_f.cpu().numpy(), lr)
    np.testing.assert_array_equal(bonus_f.cpu().numpy(), br)
    new_layers, P1, par1, n1 = oracle.tree_cache_reroot(layers_np, c.prefix_len, c.parent,
                                                        c.n_nodes, pr, lr, keep_np.astype(bool),
                                                        c.block_table, c.block_size)
    np.testing.assert_array_equal(F.prefix_len.cpu().numpy(), P1)
    np.testing.assert_array_equal(F.n_nodes.cpu().numpy(), n1)
    np.testing.assert_array_equal(F.parent.cpu().numpy(), par1)
    if oracle_rows:
        for (k_ref, v_ref), lay in zip(new_layers, lf):
            kg, vg = _bits(lay.k), _bits(lay.v)
            kr = k_ref.view(np.int16 if c.dtype == "bf16" else np.int32)
            vr = v_ref.view(np.int16 if c.dtype == "bf16" else np.int32)
            for b in range(c.B):
                end = int(P1[b] + n1[b])
                if c.paged:
                    for t in range(end):
                        blk, s = c.block_table[b, t // c.block_size], t % c.block_size
                        assert (kg[blk, s] == kr[blk, s]).all() and (vg[blk, s] == vr[blk, s]).all()
                else:
                    np.testing.assert_array_equal(kg[b, :end], kr[b, :end])
                    np.testing.assert_array_equal(vg[b, :end], vr[b, :end])
    return lr, n1


def _keep(rng, B, keep):
    return np.array([keep if keep is not None else bool(rng.integers(0, 2)) for _ in range(B)],
                    dtype=np.uint8)


@pytest.mark.parametrize("seed,dtype,d,paged,keep,n_layers", [
    (1, "bf16", 128, False, True, 1), (2, "bf16", 128, False, False, 3),
    (3, "f32", 64, False, None, 2), (4, "bf16", 64, True, True, 1),
    (5, "f32", 128, True, None, 3), (6, "bf16", 128, False, None, 0),
    (7, "bf16", 128, True, None, 33)])
def test_fused_matches_two_calls(ta, seed, dtype, d, paged, keep, n_layers):
    print(f"case seed={seed} {dtype} d={d} paged={paged} layers={n_layers}", flush=True)
    c = random_case(500 + seed, B=7, Hq=4, Hkv=2, d=d, P_range=(0, 90), n_max=24,
                    n_range=(0, 24), dtype=dtype, paged=paged, block_size=8, target_side=True,
                    vocab=300)
    lr, n1 = _check_case(ta, c, _keep(np.random.default_rng(seed), c.B, keep), n_layers)
    assert (lr > 0).any()


def test_fused_many_sequences_and_full_trees(ta):
    """512 sequences (many groups per count), then trees of 256 nodes."""
    c = random_case(601, B=512, Hq=2, Hkv=1, d=64, P_range=(0, 40), n_max=12, n_range=(0, 12),
                    dtype="bf16", target_side=True, vocab=64)
    _check_case(ta, c, _keep(np.random.default_rng(1), c.B, None), 2, oracle_rows=False)
    c = random_case(602, B=3, Hq=8, Hkv=8, d=128, P_range=(0, 20), n_max=256,
                    n_range=(200, 256), dtype="bf16", target_side=True, vocab=40)
    _check_case(ta, c, _keep(np.random.default_rng(2), c.B, True), 2)


def test_fused_repeated_calls_share_one_workspace(ta):
    """Five calls in a row on one workspace, with batch sizes that shrink and
    grow, after stray bytes were written into it: nothing carries over from
    one call to the next."""
    import torch
    ws = ta.Workspace()
    ws.get(1 << 16, torch.device("cuda")).fill_(0x5A)  # stray bytes
    for i, B in enumerate((9, 4, 9, 16, 1)):
        c = random_case(700 + i, B=B, Hq=4, Hkv=2, d=128, P_range=(10, 200), n_max=32,
                        n_range=(1, 32), dtype="bf16", target_side=True, vocab=500)
        _check_case(ta, c, _keep(np.random.default_rng(i), B, None), 2, ws=ws)


def test_fused_duplicate_sibling_ties(ta):
    """Ties between deepest accepted nodes (tokens from {0, 1}, small-integer
    logits in columns 0 and 1 only): every group of a sequence must pick the
    same path."""
    from test_gpu_accept_reroot import _tied_deepest
    rng = np.random.default_rng([77, 1])
    c = random_case(703, B=24, Hq=2, Hkv=2, d=64, P_range=(0, 30), n_max=40, n_range=(1, 40),
                    dtype="f32", target_side=True, vocab=64)
    c.tok = rng.integers(0, 2, size=c.tok.shape).astype(np.int32)
    c.root_tok = c.tok[:, 0].copy()
    lg = np.full(c.logits.shape, -10.0, dtype=np.float32)
    lg[:, :, :2] = rng.integers(-2, 3, size=lg[:, :, :2].shape)
    c.logits = lg
    ties = sum(_tied_deepest(c.parent[b], c.tok[b], c.logits[b], c.root_tok[b], int(c.n_nodes[b])) >= 2
               for b in range(c.B))
    assert ties >= c.B // 8, "the case must exercise ties between deepest accepted nodes"
    _check_case(ta, c, _keep(rng, c.B, None), 2)
