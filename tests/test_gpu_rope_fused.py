"""RoPE fused into the attention call (tree_attn_verify_rope,
tree_attn_expand_rope; SwiftSpec summary, Section 3.3: the masked attention
takes the position embedding) against the same work done in two calls,
tree_rope_append then tree_attn_verify / tree_attn_expand, and against the
float64 oracle.

* The cache rows the call writes (rotated keys, values) equal the two-call
  path's bit for bit: both use the same rotation arithmetic.
* Outputs: where the call falls back to those two launches (paged caches,
  fp32, too many query slots per tile) they are identical; where the
  streaming kernel rotates on load, the tree positions are attended as tiles
  of their own, so fp32 sums run in another order and the softmax weights
  round to bf16 against another running maximum: outputs agree within
  FUSED_ATOL (two bf16 roundings of weights and outputs, 2^-7 relative, on
  outputs below 0.3) and LSE within FUSED_LSE: each path is within the
  derived 1e-4 of the exact log-sum-exp (fp32 sums of a few hundred terms per
  split, exponentials within an ulp; test_gpu_fullsize.py), so the two within
  twice that.
* Against the oracle (rotation in float64, rounded to the cache dtype, then
  explicit-mask attention): the stated float bars.
"""
import numpy as np
import pytest

from helpers import DevCase, assert_attn_close, dev_tensor, ensure_built, to_f64

import oracle
from gen import config2_chain, random_case

pytestmark = pytest.mark.gpu

BASE = 10000.0
FUSED_ATOL = 4e-3
FUSED_LSE = 2e-4


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _raw(rng, shape, dtype):
    import torch
    a = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        return torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return a


def _f64(a, dtype):
    return oracle.bf16_to_f64(a) if dtype == "bf16" else np.asarray(a, np.float64)


def _round_to(a64, dtype):
    """float64 values rounded to the storage dtype, back as float64."""
    import torch
    t = torch.from_numpy(np.asarray(a64, np.float64))
    if dtype == "bf16":
        return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    return t.to(torch.float32).to(torch.float64).numpy()


def _run_both(ta, c, q, kn, vn, w):
    """(fused outputs, two-call outputs, both caches after) for one case."""
    import torch
    dt = c.dtype
    A, Bc = DevCase(c), DevCase(c)
    dq, dk, dv = dev_tensor(q, dt), dev_tensor(kn, dt), dev_tensor(vn, dt)
    if w:
        of, lf = ta.tree_attn_expand_rope(dq, dk, dv, A.kv, A.prefix_len, A.parent, A.n_nodes,
                                          c.scale, base=BASE)
        qo = ta.tree_rope_append(dq, dk, dv, Bc.kv, Bc.prefix_len, Bc.parent, Bc.n_nodes,
                                 base=BASE, expand=True)
        ou, lu = ta.tree_attn_expand(qo, Bc.kv, Bc.prefix_len, Bc.parent, Bc.n_nodes, c.scale)
    else:
        of, lf = ta.tree_attn_verify_rope(dq, dk, dv, A.kv, A.prefix_len, A.parent, A.n_nodes,
                                          c.scale, base=BASE)
        qo = ta.tree_rope_append(dq, dk, dv, Bc.kv, Bc.prefix_len, Bc.parent, Bc.n_nodes,
                                 base=BASE)
        ou, lu = ta.tree_attn_verify(qo, Bc.kv, Bc.prefix_len, Bc.parent, Bc.n_nodes, c.scale)
    torch.cuda.synchronize()
    return (of, lf, ou, lu, A, Bc)


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _rows(c, w):
    """[B][n_q] mask of query rows that hold a node."""
    n_q = w if w else c.n_max
    m = np.zeros((c.B, n_q), bool)
    for b in range(c.B):
        n = int(c.n_nodes[b])
        for s in range(n_q):
            node = n - n_q + s if w else s
            m[b, s] = 0 <= node < n
    return m


CASES = [
    # (seed, B, Hq, Hkv, d, P_range, n_max, n_range, dtype, paged, w, fused)
    (1, 4, 16, 2, 128, (100, 6000), 16, None, "bf16", False, 0, True),     # G 8, splits
    (2, 3, 32, 8, 128, (0, 3000), 40, (1, 40), "bf16", False, 0, True),    # G 4, two tree tiles
    (3, 2, 16, 2, 64, (500, 9000), 24, (6, 24), "bf16", False, 6, True),   # d 64, expand
    (4, 3, 64, 8, 128, (30, 34), 16, None, "bf16", False, 0, True),        # P at a tile edge
    (5, 2, 32, 4, 128, (0, 0), 20, (1, 20), "bf16", False, 0, True),       # no prefix at all
    (6, 2, 64, 8, 128, (2000, 8000), 16, None, "bf16", True, 0, False),    # paged: two calls
    (7, 2, 8, 1, 64, (0, 300), 12, None, "f32", False, 0, False),          # fp32: two calls
    (8, 2, 8, 4, 128, (100, 2000), 64, (1, 64), "bf16", False, 0, False),  # G 2, 128 rows
    (9, 2, 16, 2, 128, (3000, 9000), 200, (150, 200), "bf16", False, 8, True),  # big tree, expand
]


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_fused_rope_matches_two_calls_and_oracle(ta, case):
    seed, B, Hq, Hkv, d, P_range, n_max, n_range, dtype, paged, w, fused = case
    print(f"case seed={seed} {dtype} d={d} G={Hq // Hkv} paged={paged} w={w}", flush=True)
    c = random_case(300 + seed, B, Hq, Hkv, d, P_range=P_range, n_max=n_max, n_range=n_range,
                    dtype=dtype, paged=paged)
    if w:
        c.n_nodes = np.maximum(c.n_nodes, 1).astype(np.int32)
    rng = np.random.default_rng([seed, 61])
    n_q = w if w else n_max
    q = _raw(rng, (B, n_q, Hq, d), dtype)
    kn, vn = _raw(rng, (B, n_q, Hkv, d), dtype), _raw(rng, (B, n_q, Hkv, d), dtype)
    of, lf, ou, lu, A, Bc = _run_both(ta, c, q, kn, vn, w)
    rows = _rows(c, w)
    # the cache: identical bits wherever a sequence's rows are defined
    for b in range(B):
        end = int(c.prefix_len[b] + c.n_nodes[b])
        ka, kb, va, vb = _bits(A.k), _bits(Bc.k), _bits(A.v), _bits(Bc.v)
        for t in range(end):
            if paged:
                blk, o = c.block_table[b, t // c.block_size], t % c.block_size
                assert (ka[blk, o] == kb[blk, o]).all() and (va[blk, o] == vb[blk, o]).all(), (b, t)
            else:
                assert (ka[b, t] == kb[b, t]).all() and (va[b, t] == vb[b, t]).all(), (b, t)
    Of, Ou = to_f64(of), to_f64(ou)
    Lf, Lu = lf.cpu().numpy().astype(np.float64), lu.cpu().numpy().astype(np.float64)
    if not fused:
        np.testing.assert_array_equal(_bits(of)[rows], _bits(ou)[rows])
        np.testing.assert_array_equal(Lf.transpose(0, 2, 1)[rows], Lu.transpose(0, 2, 1)[rows])
    else:
        err = np.abs(Of[rows] - Ou[rows]).max()
        lerr = np.abs(Lf.transpose(0, 2, 1)[rows] - Lu.transpose(0, 2, 1)[rows]).max()
        assert err <= FUSED_ATOL and lerr <= FUSED_LSE, (err, lerr)
    # oracle: rotation in float64, stored in the cache dtype, then attention
    q_ref, new_rows = oracle.rope_append(_f64(q, dtype), _f64(kn, dtype), _f64(vn, dtype),
                                         c.prefix_len, c.parent, c.n_nodes, n_q, bool(w), BASE)
    k64 = _f64(c.k, dtype).copy()
    v64 = _f64(c.v, dtype).copy()
    for b in range(B):
        for t, (kr, vr) in new_rows[b].items():
            if paged:
                idx = (int(c.block_table[b, t // c.block_size]), t % c.block_size)
            else:
                idx = (b, t)
            k64[idx] = _round_to(kr, dtype)
            v64[idx] = vr
    oc = type("OC", (), {})()
    oc.B, oc.Hq, oc.d, oc.G, oc.scale, oc.dtype = B, Hq, d, Hq // Hkv, c.scale, "f32"
    oc.prefix_len, oc.n_nodes, oc.parent = c.prefix_len, c.n_nodes, c.parent
    oc.k, oc.v = k64.astype(np.float32) if dtype == "f32" else k64, v64
    oc.block_table, oc.block_size = c.block_table, c.block_size
    qr = _round_to(np.nan_to_num(q_ref), dtype)
    if dtype == "bf16":
        oc.k, oc.v, qr = oc.k.astype(np.float32), oc.v.astype(np.float32), qr.astype(np.float32)
    if w:
        Or, Lr = oracle.expand(oc, qr, w)
    else:
        oc.q = qr
        Or, Lr = oracle.verify(oc)
    assert_attn_close(Of, Lf, Or, Lr, dtype, rows_mask=rows, what=f"fused rope seed {seed}")


def test_fused_rope_chain_verify_full_size(ta):
    """The chain-verify workload's shapes (2.1 GB of KV, 16 chains of 16
    nodes, 128 rows per KV head) with RoPE fused in, against the two calls."""
    import torch
    c = config2_chain()
    rng = np.random.default_rng(62)
    q = _raw(rng, c.q.shape, "bf16")
    kn = _raw(rng, (c.B, c.n_max, c.Hkv, c.d), "bf16")
    vn = _raw(rng, (c.B, c.n_max, c.Hkv, c.d), "bf16")
    of, lf, ou, lu, A, Bc = _run_both(ta, c, q, kn, vn, 0)
    for b in range(c.B):
        P = int(c.prefix_len[b])
        assert torch.equal(A.k[b, P:P + 16], Bc.k[b, P:P + 16])
        assert torch.equal(A.v[b, P:P + 16], Bc.v[b, P:P + 16])
    err = (of.float() - ou.float()).abs().max().item()
    lerr = (lf - lu).abs().max().item()
    assert err <= FUSED_ATOL and lerr <= FUSED_LSE, (err, lerr)
    del A, Bc
    torch.cuda.empty_cache()
