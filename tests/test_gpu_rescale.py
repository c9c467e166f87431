"""GPU parity of the attention kernels when a row's running maximum jumps.

The streaming kernel keeps each row's online softmax against a running
maximum that is raised lazily: a tile whose maximum passes it by a moderate
amount rescales the state after the tile's P.V, and one that passes it by a
lot takes its exponentials against a reference raised within the tile, so
that the state so far drops below fp32 resolution next to it.  (The units
and register-prefetch kernels rescale before every larger maximum.)  Random
inputs rarely move the maximum by more than a few units, so
these cases plant keys along the one direction every query takes: scores
then jump by set amounts at set positions (moderate jumps between tiles, and
jumps of 80 to 110 log2 units inside a split and in the tree tail).  The
reference is the float64 oracle on the same bf16 inputs.

The log-sum-exp bar here is tighter than the general bf16 bar: its only
rounding is fp32 (scores, exponentials and sums), so a tile dropped, counted
twice or taken against the wrong reference moves it far past 1e-3 + 1e-4
|LSE|, while the output keeps the bf16 bar (its p are rounded to bf16 for
P.V)."""
import numpy as np
import pytest

from helpers import BF16_ATOL, BF16_RTOL, DevCase, ensure_built, to_f64

import oracle
from gen import bf16_bits_from_f32, random_case

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634

# (tile index in the prefix or "tree" for a tree node's key, score in log2 units)
PLANTS = {
    "moderate": [(2, 10.0), (9, 16.0), (17, 27.0), (30, 24.0), ("tree", 30.0)],
    "huge": [(2, 10.0), (9, 90.0), (17, 200.0), (30, 150.0), ("tree", 280.0)],
}


def _bf16(x):
    bits = bf16_bits_from_f32(np.asarray(x, dtype=np.float32))
    return bits, (bits.astype(np.uint32) << 16).view(np.float32)


def _planted_case(seed, paged, pattern):
    c = random_case(seed, B=3, Hq=8, Hkv=2, d=128, P_range=(1100, 1400), n_max=16, n_range=(8, 16),
                    dtype="bf16", target_side=True, paged=paged)
    rng = np.random.default_rng([seed, 99])
    u = rng.standard_normal(c.d)
    u /= np.linalg.norm(u)
    q_bits, u_b = _bf16(u)
    c.q[...] = q_bits                      # every row and head takes the direction u
    k = (c.k.astype(np.uint32) << 16).view(np.float32) * np.float32(0.1)
    c.k[...] = bf16_bits_from_f32(k)       # background scores near 0
    unit = float(np.dot(u_b.astype(np.float64), u_b.astype(np.float64))) * c.scale * LOG2E
    for b in range(c.B):
        P, n = int(c.prefix_len[b]), int(c.n_nodes[b])
        for tile, score in PLANTS[pattern]:
            if tile == "tree":
                t = P + int(rng.integers(1, n))        # a node other than the root
            else:
                t = tile * 32 + int(rng.integers(0, 32))
                assert t < P
            bits, _ = _bf16(u * (score / unit))
            for h in range(c.Hkv):
                if paged:
                    blk = int(c.block_table[b, t // c.block_size])
                    c.k[blk, t % c.block_size, h] = bits
                else:
                    c.k[b, t, h] = bits
    return c


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


@pytest.mark.parametrize("pattern", sorted(PLANTS))
@pytest.mark.parametrize("paged,chunk,kernel", [(False, 0, 0), (False, 256, 0), (False, 128, 0),
                                                (True, 0, 0), (True, 256, 3), (False, 0, 2)],
                         ids=["stream", "stream256", "stream128", "units", "paged-stream",
                              "mfma"])
def test_score_jumps(ta, pattern, paged, chunk, kernel):
    import torch
    c = _planted_case(17, paged, pattern)
    print(f"case pattern={pattern} paged={paged} chunk={chunk} kernel={kernel}", flush=True)
    dc = DevCase(c)
    out = torch.full_like(dc.q, float("nan"))
    lse = torch.full((c.B, c.Hq, c.n_max), float("nan"), dtype=torch.float32, device=dc.q.device)
    ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale, out=out,
                        lse=lse, chunk_tokens=chunk, kernel=kernel)
    torch.cuda.synchronize()
    O, L = to_f64(out), lse.cpu().numpy().astype(np.float64)
    Or, Lr = oracle.verify(c)
    for b in range(c.B):
        n = int(c.n_nodes[b])
        o, orf = O[b, :n], Or[b, :n]
        l, lrf = L[b, :, :n], Lr[b, :, :n]
        assert np.isfinite(o).all() and np.isfinite(l).all(), f"b={b}: non-finite results"
        eo = np.abs(o - orf) - (BF16_ATOL + BF16_RTOL * np.abs(orf))
        assert eo.max() <= 0, f"b={b}: output off by {np.abs(o - orf).max():.3e}"
        el = np.abs(l - lrf) - (1e-3 + 1e-4 * np.abs(lrf))
        assert el.max() <= 0, f"b={b}: LSE off by {np.abs(l - lrf).max():.3e}"
    # the planted jumps reach the results: the LSE sits near the largest score a row sees
    top = max(s for _, s in PLANTS[pattern]) / LOG2E
    assert np.nanmax(Lr) > 0.9 * top
