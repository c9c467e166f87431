"""GPU parity of tree_attn_verify / tree_attn_expand against the float64 oracle
(small seeded cases spanning several KV tiles, splits and a ragged tail)."""
import numpy as np
import pytest

from helpers import DevCase, assert_attn_close, ensure_built, to_f64

import oracle
from gen import config1_tiny, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _run_verify(ta, dc, chunk=0, kernel=0):
    import torch
    c = dc.case
    out = torch.full_like(dc.q, float("nan"))
    lse = torch.full((c.B, c.Hq, c.n_max), float("nan"), dtype=torch.float32, device=dc.q.device)
    ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale, out=out,
                        lse=lse, chunk_tokens=chunk, kernel=kernel)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


def _check_unwritten(O, L, c, q_nodes_of):
    for b in range(c.B):
        n = int(c.n_nodes[b])
        for r, node in enumerate(q_nodes_of(n)):
            if not (0 <= node < n):
                assert np.isnan(O[b, r]).all() and np.isnan(L[b, :, r]).all(), (b, r)


@pytest.mark.parametrize("chunk", [0, 64, 128])
def test_tiny_fp32_verify_and_expand(ta, chunk):
    import torch
    c = config1_tiny()
    dc = DevCase(c)
    O, L = _run_verify(ta, dc, chunk)
    Or, Lr = oracle.verify(c)
    assert_attn_close(O, L, Or, Lr, "f32", what="verify")
    w = c.planted["expand_w"]
    qe = dc.q[:, c.n_max - w:].contiguous()
    out, lse = ta.tree_attn_expand(qe, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale,
                                   chunk_tokens=chunk)
    torch.cuda.synchronize()
    Oer, Ler = oracle.expand(c, c.q[:, c.n_max - w:], w)
    assert Oer.shape[1] == 4 and c.prefix_len[0] + c.n_nodes[0] == 144   # the 4 x 144 mask
    assert_attn_close(to_f64(out), lse.cpu().numpy(), Oer, Ler, "f32", what="expand")


CASES = [
    # (seed, B, Hq, Hkv, d, P_range, n_max, dtype, target_side, paged, chunk)
    (1, 3, 8, 1, 64, (0, 300), 16, "f32", False, False, 64),
    (2, 4, 8, 2, 128, (0, 300), 16, "bf16", False, False, 0),
    (3, 4, 16, 2, 128, (100, 700), 8, "bf16", True, False, 128),
    (4, 2, 4, 4, 64, (0, 200), 12, "bf16", False, True, 64),
    (5, 5, 6, 3, 128, (1, 520), 20, "f32", True, True, 192),
    (6, 2, 64, 8, 128, (60, 400), 16, "bf16", True, False, 64),
    (7, 3, 32, 8, 128, (0, 257), 40, "bf16", False, False, 0),
    (8, 2, 2, 1, 128, (0, 5), 256, "bf16", False, False, 64),   # maximum tree size
]


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_random_verify(ta, case):
    seed, B, Hq, Hkv, d, P_range, n_max, dtype, target_side, paged, chunk = case
    c = random_case(seed, B, Hq, Hkv, d, P_range=P_range, n_max=n_max, dtype=dtype,
                    target_side=target_side, paged=paged)
    print(f"case seed={seed} B={B} Hq={Hq} Hkv={Hkv} d={d} n_max={n_max} {dtype} paged={paged}",
          flush=True)
    dc = DevCase(c)
    O, L = _run_verify(ta, dc, chunk)
    Or, Lr = oracle.verify(c)
    assert_attn_close(O, L, Or, Lr, dtype, what=f"seed{seed}")
    _check_unwritten(O, L, c, lambda n: range(c.n_max))


BOTH_KERNELS = [
    # (seed, B, Hq, Hkv, d, P_range, n_max, target_side, paged, chunk)
    (21, 3, 8, 1, 128, (0, 700), 16, True, False, 128),     # 128 rows: 4 row groups
    (22, 4, 16, 2, 128, (50, 900), 8, True, False, 0),      # 64 rows: 2 groups x 2 token halves
    (23, 5, 64, 8, 128, (10, 600), 6, True, True, 128),     # 48 rows, paged
    (24, 2, 32, 8, 128, (0, 400), 8, False, False, 256),    # 32 rows: 4 token quarters
    (25, 3, 12, 1, 64, (0, 500), 8, False, False, 64),      # 96 rows: 3 groups, d = 64
    (26, 2, 16, 1, 128, (100, 300), 20, False, True, 0),    # 320 rows: 3 row tiles
    (27, 2, 8, 1, 128, (700, 900), 8, True, True, 0),       # paged, 1-position blocks
]


@pytest.mark.parametrize("case", BOTH_KERNELS, ids=[f"seed{c[0]}" for c in BOTH_KERNELS])
@pytest.mark.parametrize("kernel", [1, 2, 3, 4])
def test_bf16_both_kernels(ta, case, kernel):
    seed, B, Hq, Hkv, d, P_range, n_max, target_side, paged, chunk = case
    c = random_case(seed, B, Hq, Hkv, d, P_range=P_range, n_max=n_max, dtype="bf16",
                    target_side=target_side, paged=paged, block_size=1 if seed == 27 else 16)
    print(f"case seed={seed} kernel={kernel} rows={n_max * Hq // Hkv} d={d} paged={paged}",
          flush=True)
    dc = DevCase(c)
    O, L = _run_verify(ta, dc, chunk, kernel)
    Or, Lr = oracle.verify(c)
    assert_attn_close(O, L, Or, Lr, "bf16", what=f"seed{seed} kernel{kernel}")
    _check_unwritten(O, L, c, lambda n: range(c.n_max))


@pytest.mark.parametrize("w", [1, 3, 8])
def test_random_expand(ta, w):
    import torch
    c = random_case(40 + w, 3, 8, 2, 128, P_range=(0, 200), n_max=12, n_range=(1, 12),
                    dtype="bf16")
    dc = DevCase(c)
    qe_np = c.q[:, :w]
    qe = dc.q[:, :w].contiguous()
    out = torch.full_like(qe, float("nan"))
    lse = torch.full((c.B, c.Hq, w), float("nan"), dtype=torch.float32, device=qe.device)
    ta.tree_attn_expand(qe, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale, out=out,
                        lse=lse, chunk_tokens=64)
    torch.cuda.synchronize()
    O, L = to_f64(out), lse.cpu().numpy()
    Or, Lr = oracle.expand(c, qe_np, w)
    assert_attn_close(O, L, Or, Lr, "bf16", what=f"expand w={w}")
    _check_unwritten(O, L, c, lambda n: [n - w + r for r in range(w)])


@pytest.mark.parametrize("w", [1, 8])
def test_units_kernel_expand(ta, w):
    """Expansion rows through the units kernel (kernel 4)."""
    import torch
    c = random_case(60 + w, 5, 32, 8, 128, P_range=(0, 1500), n_max=24, n_range=(1, 24),
                    dtype="bf16", paged=True)
    dc = DevCase(c)
    qe = dc.q[:, :w].contiguous()
    out = torch.full_like(qe, float("nan"))
    lse = torch.full((c.B, c.Hq, w), float("nan"), dtype=torch.float32, device=qe.device)
    ta.tree_attn_expand(qe, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale, out=out,
                        lse=lse, kernel=4)
    torch.cuda.synchronize()
    O, L = to_f64(out), lse.cpu().numpy()
    Or, Lr = oracle.expand(c, c.q[:, :w], w)
    assert_attn_close(O, L, Or, Lr, "bf16", what=f"units expand w={w}")
    _check_unwritten(O, L, c, lambda n: [n - w + r for r in range(w)])


@pytest.mark.parametrize("seed", [90, 91])
def test_units_kernel_mixed_lengths(ta, seed):
    """Paged batch with lengths from 0 to ~6000 (jobs of 1 to ~190 tiles):
    ranges cut jobs at arbitrary tiles, some groups hold several whole jobs."""
    c = random_case(seed, 12, 16, 4, 128, P_range=(0, 6000), n_max=10, dtype="bf16",
                    target_side=seed == 91, paged=True)
    dc = DevCase(c)
    O, L = _run_verify(ta, dc, 0, 4)
    Or, Lr = oracle.verify(c)
    assert_attn_close(O, L, Or, Lr, "bf16", what=f"units mixed seed{seed}")
    _check_unwritten(O, L, c, lambda n: range(c.n_max))


@pytest.mark.parametrize("case", [
    # (seed, B, Hq, Hkv, d, P_range, n_max, block_size)
    (92, 8, 64, 8, 128, (3500, 4500), 6, 1),   # 1-position blocks: ranges set up in batches
    (93, 6, 16, 2, 64, (0, 3000), 8, 16),      # 64 rows, d = 64: 4 KiB ring halves
    (95, 3, 4, 2, 128, (0, 2000), 256, 16),    # maximum tree: 512 rows, four 128-row tiles
], ids=["many-batches", "d64", "max-tree"])
def test_units_kernel_batches_and_shapes(ta, case):
    """Units kernel on ranges that need several set-up batches (1-position
    blocks), 64-dimensional heads, and the maximum tree (256 nodes, whose
    tree pieces fill the row-mask table in several batches)."""
    seed, B, Hq, Hkv, d, P_range, n_max, bsz = case
    c = random_case(seed, B, Hq, Hkv, d, P_range=P_range, n_max=n_max, dtype="bf16",
                    target_side=True, paged=True, block_size=bsz)
    print(f"case seed={seed} units kernel d={d} n_max={n_max} block_size={bsz}", flush=True)
    dc = DevCase(c)
    O, L = _run_verify(ta, dc, 0, 4)
    Or, Lr = oracle.verify(c)
    assert_attn_close(O, L, Or, Lr, "bf16", what=f"units kernel seed{seed}")
    _check_unwritten(O, L, c, lambda n: range(c.n_max))


def test_split_count_invariance(ta):
    c = random_case(77, 2, 16, 2, 128, P_range=(900, 1100), n_max=8, dtype="bf16",
                    target_side=True)
    dc = DevCase(c)
    ref = None
    for chunk in (64, 256, 1024, 2048):
        O, L = _run_verify(ta, dc, chunk)
        if ref is None:
            ref = (O, L)
            Or, Lr = oracle.verify(c)
            assert_attn_close(O, L, Or, Lr, "bf16", what=f"chunk {chunk}")
        else:
            # unwritten padding rows stay NaN in both; written rows agree closely
            np.testing.assert_array_equal(np.isnan(O), np.isnan(ref[0]))
            assert np.nanmax(np.abs(O - ref[0])) < 4e-3 and np.nanmax(np.abs(L - ref[1])) < 1e-4


@pytest.mark.parametrize("kernel", [3, 4])
def test_combine_ignores_stale_workspace(ta, kernel):
    """The combine launch fetches its first partial states before it knows a
    sequence's split count; slots past a short sequence's last split hold
    whatever an earlier call left (here NaN bytes) and must not reach the
    result."""
    import torch
    c = random_case(94, 6, 16, 2, 128, P_range=(40, 3000), n_max=8, dtype="bf16",
                    target_side=True, paged=kernel == 4)
    dc = DevCase(c)
    ws = ta.Workspace()
    for rep in range(2):
        out = torch.full_like(dc.q, float("nan"))
        lse = torch.full((c.B, c.Hq, c.n_max), float("nan"), dtype=torch.float32,
                         device=dc.q.device)
        ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale, out=out,
                            lse=lse, workspace=ws, chunk_tokens=64, kernel=kernel)
        torch.cuda.synchronize()
        if rep == 0:
            ws.buf.view(torch.float32)[: ws.buf.numel() // 4].fill_(float("nan"))
            torch.cuda.synchronize()
    Or, Lr = oracle.verify(c)
    assert_attn_close(to_f64(out), lse.cpu().numpy().astype(np.float64), Or, Lr, "bf16",
                      what=f"stale workspace kernel{kernel}")


def test_repeated_calls_are_deterministic_and_reset_counters(ta):
    c = random_case(78, 3, 8, 2, 128, P_range=(300, 900), n_max=16, dtype="bf16")
    dc = DevCase(c)
    O1, L1 = _run_verify(ta, dc, 64)
    for _ in range(3):
        O2, L2 = _run_verify(ta, dc, 64)
        np.testing.assert_array_equal(O1, O2)
        np.testing.assert_array_equal(L1, L2)


def test_zero_prefix_and_empty_trees(ta):
    c = random_case(79, 4, 8, 2, 64, P_range=(0, 0), n_max=6, n_range=(0, 6), dtype="f32")
    c.n_nodes[1] = 0
    dc = DevCase(c)
    O, L = _run_verify(ta, dc, 0)
    Or, Lr = oracle.verify(c)
    assert_attn_close(O, L, Or, Lr, "f32", what="P=0")
    assert np.isnan(O[1]).all()


def test_workspace_reuse_across_plans(ta):
    """One workspace serves calls with different plans (split counts, tiles)."""
    ws = ta.Workspace()
    cases = [random_case(80 + i, 2 + i, 8, 2, 128, P_range=(300, 900 + 300 * i), n_max=8 + 4 * i,
                         dtype="bf16") for i in range(3)]
    for rep in range(2):
        for i, c in enumerate(cases):
            dc = DevCase(c)
            import torch
            out, lse = ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes,
                                           c.scale, workspace=ws, chunk_tokens=64 * (i + 1))
            torch.cuda.synchronize()
            Or, Lr = oracle.verify(c)
            assert_attn_close(to_f64(out), lse.cpu().numpy(), Or, Lr, "bf16",
                              what=f"rep {rep} case {i}")


def test_default_workspace_is_per_stream(ta):
    """Calls on two streams without an explicit workspace get one workspace
    each (so they cannot race on partial results) and the same outputs."""
    import torch
    from tree_masked_verify_attn_amd import _lib
    c = random_case(77, B=3, Hq=16, Hkv=2, d=128, P_range=(3000, 5000), n_max=8, dtype="bf16")
    dc = DevCase(c)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        o1, l1 = ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale)
    with torch.cuda.stream(s2):
        o2, l2 = ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale)
    torch.cuda.synchronize()
    keys = {k for k in _lib._default_ws if k[1] in (s1.cuda_stream, s2.cuda_stream)}
    assert len(keys) == 2
    bufs = [_lib._default_ws[k].buf for k in keys]
    assert bufs[0].data_ptr() != bufs[1].data_ptr()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
