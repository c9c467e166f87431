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
