"""The whole hot path captured in one HIP graph (torch.cuda.CUDAGraph on the
library's stream): every replay must reproduce the eager results bit for bit.

The entry points take sizes from device memory and allocate nothing, so a
decode step can be captured once and replayed.  Each replay here follows
eager work of the program itself (restoring the inputs the re-root rewrote)
and a synchronisation, and every replay is checked, not just the last."""
import numpy as np
import pytest

from helpers import DevCase, dev_tensor, ensure_built

from gen import random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _bits(t):
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    return t.cpu().numpy()


@pytest.mark.parametrize("paged,fused", [(False, False), (True, False), (False, True),
                                         (True, True)])
def test_step_graph_replays_match_eager(ta, paged, fused):
    """fused: greedy accept + re-root through tree_accept_reroot (two
    launches, its copy of the metadata in the shared workspace), else
    accept_greedy_path then tree_cache_reroot."""
    import torch
    c = random_case(41 + int(paged), B=5, Hq=16, Hkv=2, d=128, P_range=(0, 1500), n_max=24,
                    dtype="bf16", paged=paged, vocab=3000)
    dc = DevCase(c)
    w = 4
    q_exp = dc.q[:, -w:].contiguous()
    keep = dev_tensor(np.array([1, 0, 1, 1, 0], dtype=np.uint8))
    ws = ta.Workspace(dc.q.device)
    pristine = {name: getattr(dc, name).clone() for name in ("k", "v", "prefix_len", "parent",
                                                             "n_nodes")}

    def restore():
        for name, t in pristine.items():
            getattr(dc, name).copy_(t)

    out = torch.empty_like(dc.q)
    lse = torch.empty((c.B, c.Hq, c.n_max), dtype=torch.float32, device=dc.q.device)
    out_x = torch.empty_like(q_exp)
    lse_x = torch.empty((c.B, c.Hq, w), dtype=torch.float32, device=dc.q.device)
    path = torch.empty((c.B, c.n_max), dtype=torch.int32, device=dc.q.device)
    plen = torch.empty((c.B,), dtype=torch.int32, device=dc.q.device)
    bonus = torch.empty((c.B,), dtype=torch.int32, device=dc.q.device)
    # a small split so that the combine launch is part of the graph too
    opts = {"chunk_tokens": 256}

    def step():
        ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale, out=out,
                            lse=lse, workspace=ws, **opts)
        ta.tree_attn_expand(q_exp, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale,
                            out=out_x, lse=lse_x, workspace=ws, **opts)
        if fused:
            ta.tree_accept_reroot(dc.logits, dc.tok, dc.root_tok, [dc.kv], dc.prefix_len,
                                  dc.parent, dc.n_nodes, keep, path, plen, bonus, workspace=ws)
        else:
            ta.accept_greedy_path(dc.logits, dc.parent, dc.tok, dc.n_nodes, dc.root_tok, path,
                                  plen, bonus)
            ta.tree_cache_reroot([dc.kv], dc.prefix_len, dc.parent, dc.n_nodes, path, plen, keep)

    def results():
        torch.cuda.synchronize()
        return [_bits(t) for t in (out, lse, out_x, lse_x, path, plen, bonus, dc.k, dc.v,
                                   dc.prefix_len, dc.parent, dc.n_nodes)]

    def poison():  # rows a call does not write keep this value in both runs
        for t in (out, lse, out_x, lse_x, path, plen, bonus):
            t.fill_(-7)

    step()  # eager warm-up (loads the library, sizes the workspace)
    restore()
    poison()
    step()
    want = results()
    assert want[5].tolist() == c.planted["path_len"]

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        poison()
        restore()
        torch.cuda.synchronize()
        g.replay()
        got = results()
        for i, (a, b) in enumerate(zip(got, want)):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}, result {i}")
    del g
