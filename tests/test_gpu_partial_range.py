"""GPU parity when the value rows are very large or very small.

A split's partial output reaches the combine in fp16 under a power-of-two
scale chosen per row (the bf16 MFMA kernels).  These cases scale every value
by 2^100 or by 2^-118, far outside fp16's range (largest 65504, smallest
normal 2^-14) yet inside bf16's, and force splits, so that a partial state
that overflowed, flushed to zero or lost its scale would show.  The output
of attention is linear in V: the stated bf16 bars hold with their absolute
part scaled by the same factor; the log-sum-exp does not depend on V.  The
reference is the float64 oracle on the same bf16 inputs."""
import numpy as np
import pytest

from helpers import BF16_ATOL, BF16_RTOL, DevCase, ensure_built, to_f64

import oracle
from gen import bf16_bits_from_f32, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


@pytest.mark.parametrize("log2_scale", [100, -118])
@pytest.mark.parametrize("paged,chunk,kernel", [(False, 256, 3), (True, 0, 4), (False, 256, 2)],
                         ids=["stream", "units", "mfma"])
def test_value_range(ta, log2_scale, paged, chunk, kernel):
    import torch
    c = random_case(23, B=3, Hq=8, Hkv=2, d=128, P_range=(900, 1300), n_max=16, n_range=(6, 16),
                    dtype="bf16", target_side=True, paged=paged)
    scale = 2.0 ** log2_scale
    v = (c.v.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * scale
    c.v[...] = bf16_bits_from_f32(v.astype(np.float32))
    print(f"case 2^{log2_scale} paged={paged} chunk={chunk} kernel={kernel}", flush=True)
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
        assert np.isfinite(o).all(), f"b={b}: non-finite outputs"
        assert np.abs(orf).max() > 1e-3 * scale, "the scaled values reach the outputs"
        eo = np.abs(o - orf) - (BF16_ATOL * scale + BF16_RTOL * np.abs(orf))
        assert eo.max() <= 0, f"b={b}: output off by {np.abs(o - orf).max() / scale:.3e} x scale"
        l, lrf = L[b, :, :n], Lr[b, :, :n]
        assert np.all(np.abs(l - lrf) <= BF16_ATOL + BF16_RTOL * np.abs(lrf)), f"b={b}: LSE"
