"""tree_attn_verify_noalloc: the same results as tree_attn_verify from the
library's fixed per-GPU scratch array, with nothing allocated by the call.

Two calls in a row on each layout, the second with a smaller input, so the
second reads an array that still holds the first call's partial results:
both must equal tree_attn_verify's outputs bit for bit (same kernels, same
plan) and the oracle within the bf16 bars."""
import ctypes

import numpy as np
import pytest

from helpers import DevCase, assert_attn_close, ensure_built, to_f64

import oracle
from gen import random_case


@pytest.fixture(scope="module")
def ta():
    ensure_built()
    import tree_masked_verify_attn_amd as m
    return m


def _both(ta, dc):
    """(noalloc outputs, verify outputs) of one case, outputs preallocated."""
    import torch
    c = dc.case
    out_a = torch.full_like(dc.q, float("nan"))
    lse_a = torch.full((c.B, c.Hq, c.n_max), float("nan"), device=dc.q.device)
    ta.tree_attn_verify_noalloc(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes, c.scale,
                                out=out_a, lse=lse_a)
    torch.cuda.synchronize()
    out_b, lse_b = ta.tree_attn_verify(dc.q, dc.kv, dc.prefix_len, dc.parent, dc.n_nodes,
                                       c.scale, workspace=ta.Workspace(dc.q.device))
    torch.cuda.synchronize()
    return (out_a, lse_a), (out_b, lse_b)


def _check(ta, c, what):
    import torch
    dc = DevCase(c)
    (oa, la), (ob, lb) = _both(ta, dc)
    rows = np.zeros((c.B, c.n_max), bool)
    for b in range(c.B):
        rows[b, : int(c.n_nodes[b])] = True
    ia = oa.view(torch.int16).cpu().numpy()[rows]
    ib = ob.view(torch.int16).cpu().numpy()[rows]
    np.testing.assert_array_equal(ia, ib, err_msg=f"{what}: outputs differ from tree_attn_verify")
    la_n = la.cpu().numpy().transpose(0, 2, 1)[rows]
    lb_n = lb.cpu().numpy().transpose(0, 2, 1)[rows]
    np.testing.assert_array_equal(la_n.view(np.int32), lb_n.view(np.int32),
                                  err_msg=f"{what}: LSE differs from tree_attn_verify")
    Or, Lr = oracle.verify(c)
    assert_attn_close(to_f64(oa), la.cpu().numpy().astype(np.float64), Or, Lr, "bf16", what=what)


@pytest.mark.gpu
@pytest.mark.parametrize("paged", [False, True])
def test_noalloc_matches_verify_on_two_calls(ta, paged):
    # first call: long prefixes, so the plan splits (the scratch array is used)
    big = random_case(901 + paged, B=6, Hq=16, Hkv=2, d=128, P_range=(2000, 6000), n_max=16,
                      dtype="bf16", paged=paged)
    small = random_case(903 + paged, B=2, Hq=16, Hkv=2, d=128, P_range=(700, 1200), n_max=9,
                        dtype="bf16", paged=paged)
    assert ta.tree_attn_workspace_bytes(big.B, big.n_max, big.Hq, big.Hkv, big.d, ta.TA_BF16,
                                        big.T_cap) > 0
    _check(ta, big, f"first call (paged={paged})")
    _check(ta, small, f"second, smaller call (paged={paged})")


def test_noalloc_rejects_plans_beyond_the_scratch_array():
    """Host-side: a plan that needs more than TA_NOALLOC_SCRATCH_BYTES is
    refused before any device call (fake pointers; nothing is launched)."""
    from tree_masked_verify_attn_amd import _lib
    lib = ensure_built()
    B, n_max, Hq, Hkv, d, T_cap = 16, 16, 64, 8, 128, 32768
    opts = _lib.ta_attn_opts(0, 3)      # split plan of a paged cache: 16 splits per job
    need = lib.tree_attn_workspace_bytes(B, n_max, Hq, Hkv, d, _lib.TA_BF16, T_cap,
                                         ctypes.byref(opts))
    assert need > (72 << 20)
    kv = _lib.ta_kv(0x1000, 0x2000, 0x3000, 16, T_cap // 16, 4096, T_cap)
    st = lib.tree_attn_verify_noalloc(0x4000, kv, 0x5000, 0x6000, 0x7000, B, n_max, Hq, Hkv, d,
                                      _lib.TA_BF16, ctypes.c_float(0.1), 0x8000, 0x9000,
                                      ctypes.byref(opts), None)
    assert st == _lib.TA_ERR_SCRATCH
    assert "72 MiB" in lib.ta_status_string(st).decode()
    # host-checkable argument errors come first, as for tree_attn_verify
    st = lib.tree_attn_verify_noalloc(None, kv, 0x5000, 0x6000, 0x7000, B, n_max, Hq, Hkv, d,
                                      _lib.TA_BF16, ctypes.c_float(0.1), 0x8000, 0x9000, None,
                                      None)
    assert st == _lib.TA_ERR_INVALID_ARG
