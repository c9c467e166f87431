"""Seeded sweep of attention shapes against the oracle: contiguous and
paged caches, verify and expand, ragged lengths (empty trees, prefixes
shorter than a tile), one to four row groups and several row tiles, head
sizes 64 and 128, block sizes 1 to 32, bf16 and fp32.  Every case runs the
automatic kernel choice; bf16 cases also run the register-prefetch MFMA
kernel (the fallback for paged splits with many blocks).  Each case is
drawn from its seed alone and printed before it runs."""
import numpy as np
import pytest

from helpers import DevCase, assert_attn_close, ensure_built, to_f64

import oracle
from gen import random_case

pytestmark = pytest.mark.gpu

SEEDS = list(range(300, 348))


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _draw(seed):
    rng = np.random.default_rng([seed, 99])
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    d = int(rng.choice([64, 128]))
    n_max = int(rng.choice([1, 3, 6, 8, 16, 33]))
    B = int(rng.integers(1, 7))
    p_hi = int(rng.choice([0, 20, 300, 1500, 3000]))
    paged = bool(rng.integers(0, 2))
    block = int(rng.choice([1, 8, 16, 32])) if paged else 16
    target = bool(rng.integers(0, 2))
    expand_w = int(rng.integers(1, n_max + 1)) if rng.integers(0, 3) == 0 else 0
    dtype = "f32" if rng.integers(0, 4) == 0 else "bf16"
    return dict(B=B, Hq=Hkv * G, Hkv=Hkv, d=d, P_range=(0, p_hi), n_max=n_max,
                n_range=(0, n_max), target_side=target, paged=paged, block_size=block,
                expand_w=expand_w, dtype=dtype)


# every case through the automatic choice; bf16 cases also through kernel 2
CASES = [(seed, 0) for seed in SEEDS] + [(seed, 2) for seed in SEEDS
                                         if _draw(seed)["dtype"] == "bf16"]


@pytest.mark.parametrize("seed,kernel", CASES, ids=[f"seed{s}-k{k}" for s, k in CASES])
def test_random_shapes(ta, seed, kernel):
    import torch
    s = _draw(seed)
    w = s.pop("expand_w")
    print(f"case seed={seed} kernel={kernel} {s} expand_w={w}", flush=True)
    c = random_case(seed, **s)
    dc = DevCase(c)
    if w == 0:
        out = torch.full_like(dc.q, float("nan"))
        lse = torch.full((c.B, c.Hq, c.n_max), float("nan"), dtype=torch.float32,
                         device=dc.q.device)
        ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale,
                            out=out, lse=lse, kernel=kernel)
        torch.cuda.synchronize()
        Or, Lr = oracle.verify(c)
    else:
        qe = dc.q[:, :w].contiguous()
        out = torch.full_like(qe, float("nan"))
        lse = torch.full((c.B, c.Hq, w), float("nan"), dtype=torch.float32, device=qe.device)
        ta.tree_attn_expand(qe, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale, out=out,
                            lse=lse, kernel=kernel)
        torch.cuda.synchronize()
        Or, Lr = oracle.expand(c, c.q[:, :w], w)
    O, L = to_f64(out), lse.cpu().numpy().astype(np.float64)
    # rows of absent nodes are left unwritten (NaN) on both sides
    written = ~np.isnan(Or)
    np.testing.assert_array_equal(~np.isnan(O), written)
    assert_attn_close(O, L, Or, Lr, c.dtype, what=f"sweep seed{seed} kernel{kernel}")


def _draw_path(seed):
    rng = np.random.default_rng([seed, 77])
    n_max = int(rng.choice([1, 5, 16, 40, 100, 256]))
    # siblings carry distinct tokens, so the vocabulary exceeds the node count
    vocab = max(int(rng.choice([7, 300, 5000, 32000])), n_max + 1)
    B = int(rng.integers(1, 9))
    while B > 1 and B * n_max * vocab > (1 << 24):
        B -= 1
    return dict(B=B, n_max=n_max, vocab=vocab, target=bool(rng.integers(0, 2)),
                paged=bool(rng.integers(0, 2)), d=int(rng.choice([64, 128])),
                kv_dtype=str(rng.choice(["f32", "bf16"])), bf16_logits=bool(rng.integers(0, 2)),
                keep=int(rng.integers(0, 2)), P_hi=int(rng.choice([0, 40, 300])))


@pytest.mark.parametrize("seed", list(range(400, 432)))
def test_random_accept_then_reroot(ta, seed):
    """The GPU's accepted path feeds the GPU re-root, as in a decode step;
    both steps must match the oracle bit for bit (path, length, bonus token;
    prefix length, node count, parents and every KV byte up to the new end)."""
    import torch
    from helpers import dev_tensor
    s = _draw_path(seed)
    print(f"case seed={seed} {s}", flush=True)
    c = random_case(seed, B=s["B"], Hq=2, Hkv=1, d=s["d"], P_range=(0, s["P_hi"]),
                    n_max=s["n_max"], n_range=(0, s["n_max"]), dtype=s["kv_dtype"],
                    target_side=s["target"], paged=s["paged"], block_size=8, vocab=s["vocab"])
    dc = DevCase(c)
    logits_np = c.logits
    d_logits = dc.logits
    if s["bf16_logits"]:
        lg = torch.from_numpy(c.logits).to(torch.bfloat16)
        logits_np = lg.float().numpy()
        d_logits = lg.cuda()
    path, plen, bonus = ta.accept_greedy_path(d_logits, dc.parent, dc.tok, dc.n_nodes, dc.root_tok)
    keep = torch.full((c.B,), s["keep"], dtype=torch.uint8, device=dc.q.device)
    ta.tree_cache_reroot([dc.kv], dc.prefix_len, dc.parent, dc.n_nodes, path, plen, keep)
    torch.cuda.synchronize()
    pr, lr, br = oracle.accept_greedy_path(logits_np, c.parent, c.tok, c.n_nodes, c.root_tok)
    np.testing.assert_array_equal(plen.cpu().numpy(), lr)
    np.testing.assert_array_equal(path.cpu().numpy(), pr)
    np.testing.assert_array_equal(bonus.cpu().numpy(), br)
    (new_kv,), P1, par1, n1 = oracle.tree_cache_reroot(
        [(c.k, c.v)], c.prefix_len, c.parent, c.n_nodes, pr, lr,
        np.full(c.B, bool(s["keep"])), c.block_table, c.block_size)
    np.testing.assert_array_equal(dc.prefix_len.cpu().numpy(), P1)
    np.testing.assert_array_equal(dc.n_nodes.cpu().numpy(), n1)
    np.testing.assert_array_equal(dc.parent.cpu().numpy(), par1)
    bits = np.int16 if c.dtype == "bf16" else np.int32
    kg = dc.kv.k.view(torch.int16 if c.dtype == "bf16" else torch.int32).cpu().numpy()
    vg = dc.kv.v.view(torch.int16 if c.dtype == "bf16" else torch.int32).cpu().numpy()
    kr, vr = new_kv[0].view(bits), new_kv[1].view(bits)
    for b in range(c.B):
        end = int(P1[b] + n1[b])
        if c.paged:
            for t in range(end):
                blk, o = c.block_table[b, t // c.block_size], t % c.block_size
                assert (kg[blk, o] == kr[blk, o]).all() and (vg[blk, o] == vr[blk, o]).all(), (b, t)
        else:
            np.testing.assert_array_equal(kg[b, :end], kr[b, :end])
            np.testing.assert_array_equal(vg[b, :end], vr[b, :end])
