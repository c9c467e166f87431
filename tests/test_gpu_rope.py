"""GPU parity of tree_rope_append against the float64 oracle (oracle/rope.py):
the rotated query rows, the cache rows the append writes (rotated keys,
values copied bit for bit) and nothing else, for contiguous and paged caches,
fp32 and bf16, d 64 and 128, verify and expand slots; then RoPE + append +
verify end to end against the oracle's attention on rotated inputs."""
import numpy as np
import pytest

from helpers import DevCase, assert_attn_close, dev_tensor, ensure_built, to_f64

import oracle
from gen import random_case

pytestmark = pytest.mark.gpu

BASE = 10000.0


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _f64(a, dtype):
    return oracle.bf16_to_f64(a) if dtype == "bf16" else np.asarray(a, np.float64)


def _cache_row(c, kv_arr, b, t):
    """[Hkv][d] cache row of sequence b at position t (contiguous or paged)."""
    if c.block_table is None:
        return kv_arr[b, t]
    blk = int(c.block_table[b, t // c.block_size])
    return kv_arr[blk, t % c.block_size]


def _tol(dtype):
    return (dict(rtol=1e-5, atol=1e-6) if dtype == "f32" else dict(rtol=1e-2, atol=1e-2))


CASES = [
    # (seed, B, Hq, Hkv, d, P_range, n_max, dtype, paged, expand_w)
    (1, 3, 8, 2, 64, (0, 300), 12, "f32", False, 0),
    (2, 4, 16, 2, 128, (100, 40000), 16, "bf16", False, 0),
    (3, 3, 8, 1, 128, (1, 700), 10, "f32", True, 0),
    (4, 2, 64, 8, 128, (5000, 12000), 16, "bf16", True, 4),
    (5, 3, 6, 3, 64, (0, 50), 20, "f32", False, 3),
]


def _unaligned(t):
    """A copy of t whose data starts one element past a 16-byte boundary."""
    import torch
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    view = flat[1:].view(t.shape)
    view.copy_(t)
    return view


MODES = [(CASES[0], "plain"), (CASES[1], "plain"), (CASES[2], "plain"), (CASES[3], "plain"),
         (CASES[4], "plain"), (CASES[1], "unaligned"), (CASES[2], "unaligned"),
         (CASES[3], "in_place")]


@pytest.mark.parametrize("case,mode", MODES, ids=[f"seed{c[0]}-{m}" for c, m in MODES])
def test_rope_append_matches_oracle(ta, case, mode):
    """Aligned rows take the 16-byte vector kernel; an input one element off a
    16-byte boundary takes the element-wise one; in place, q_out is q."""
    import torch
    seed, B, Hq, Hkv, d, P_range, n_max, dtype, paged, w = case
    c = random_case(seed, B, Hq, Hkv, d, P_range=P_range, n_max=n_max, dtype=dtype, paged=paged)
    print(f"case seed={seed} {dtype} d={d} paged={paged} w={w}", flush=True)
    rng = np.random.default_rng([seed, 60])
    n_q = w if w else n_max
    raw = lambda shape: rng.standard_normal(shape, dtype=np.float32)  # noqa: E731
    q = raw((B, n_q, Hq, d))
    kn, vn = raw((B, n_q, Hkv, d)), raw((B, n_q, Hkv, d))
    if dtype == "bf16":
        import torch as _t
        conv = lambda a: _t.from_numpy(a).to(_t.bfloat16).view(_t.int16).numpy().view(np.uint16)  # noqa: E731
        q, kn, vn = conv(q), conv(kn), conv(vn)
    dc = DevCase(c)
    k_before = to_f64(dc.k)
    dq, dk, dv = dev_tensor(q, dtype), dev_tensor(kn, dtype), dev_tensor(vn, dtype)
    if mode == "unaligned":
        dq = _unaligned(dq)
        assert dq.data_ptr() % 16 != 0
    qo = ta.tree_rope_append(dq, dk, dv, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, base=BASE,
                             expand=bool(w), q_out=dq if mode == "in_place" else None)
    if mode == "in_place":
        assert qo.data_ptr() == dq.data_ptr()
    torch.cuda.synchronize()
    qo, k_after, v_after = to_f64(qo), to_f64(dc.k), to_f64(dc.v)
    q_ref, rows = oracle.rope_append(_f64(q, dtype), _f64(kn, dtype), _f64(vn, dtype),
                                     c.prefix_len, c.parent, c.n_nodes, n_q, bool(w), BASE)
    valid = ~np.isnan(q_ref[:, :, 0, 0])
    np.testing.assert_allclose(qo[valid], q_ref[valid], **_tol(dtype))
    vn64 = _f64(vn, dtype)
    for b in range(B):
        for t, (kr, vr) in rows[b].items():
            np.testing.assert_allclose(_cache_row(c, k_after, b, t), kr, **_tol(dtype))
            np.testing.assert_array_equal(_cache_row(c, v_after, b, t), vr)
        # a row the append does not own keeps its contents
        P = int(c.prefix_len[b])
        if P > 0:
            np.testing.assert_array_equal(_cache_row(c, k_after, b, P - 1),
                                          _cache_row(c, k_before, b, P - 1))


def test_rope_append_then_verify(ta):
    """Un-rotated queries and new keys through RoPE + append + verify, against
    the oracle's attention on inputs rotated in float64."""
    import torch
    c = random_case(71, 3, 16, 2, 128, P_range=(200, 3000), n_max=12, dtype="f32")
    dc = DevCase(c)
    B, n_max = c.B, c.n_max
    kn = np.zeros((B, n_max, c.Hkv, c.d), np.float32)
    vn = np.zeros_like(kn)
    for b in range(B):
        P, n = int(c.prefix_len[b]), int(c.n_nodes[b])
        kn[b, :n] = c.k[b, P:P + n]
        vn[b, :n] = c.v[b, P:P + n]
    qo = ta.tree_rope_append(dc.q, dev_tensor(kn), dev_tensor(vn), dc.kv, dc.prefix_len,
                             dc.parent, dc.n_nodes, base=BASE)
    out, lse = ta.tree_attn_verify(qo, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale)
    torch.cuda.synchronize()
    q_ref, rows = oracle.rope_append(c.q.astype(np.float64), kn.astype(np.float64),
                                     vn.astype(np.float64), c.prefix_len, c.parent, c.n_nodes,
                                     n_max, False, BASE)
    c.q = np.nan_to_num(q_ref).astype(np.float64)
    c.k = c.k.astype(np.float64)
    for b in range(B):
        for t, (kr, _) in rows[b].items():
            c.k[b, t] = kr
    Or, Lr = oracle.verify(c)
    assert_attn_close(to_f64(out), lse.cpu().numpy(), Or, Lr, "f32", what="rope + verify")
