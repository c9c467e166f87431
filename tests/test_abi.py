"""The C-ABI library loads, exports every declared symbol, and rejects
host-checkable bad arguments before touching a device (no compute here)."""
import ctypes
import os
import re

import pytest

from helpers import ROOT, ensure_built

import tree_masked_verify_attn_amd as ta
from tree_masked_verify_attn_amd import _lib


def test_header_declares_exactly_the_bound_symbols():
    hdr = open(os.path.join(ROOT, "include", "tree_attn.h")).read()
    declared = set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(\w+)\(", hdr, re.M))
    assert declared == set(_lib.EXPORTED_SYMBOLS)


def test_library_exports_every_symbol():
    lib = ensure_built()
    for name in _lib.EXPORTED_SYMBOLS:
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for name in _lib.EXPORTED_SYMBOLS:
        assert re.search(rf"\bT {name}$", out, re.M), name
    assert ta.ta_version() == "0.1.0"
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert ta.ta_status_string(st).startswith("TA_")


def _kv(T_cap=64, paged=False):
    if paged:
        return _lib.ta_kv(0x1000, 0x2000, 0x3000, 16, 4, 8, T_cap)
    return _lib.ta_kv(0x1000, 0x2000, None, 0, 0, 0, T_cap)


def _verify(lib, **kw):
    a = dict(q=0x4000, kv=_kv(), P=0x5000, par=0x6000, n=0x7000, B=2, n_max=16, Hq=8, Hkv=2,
             d=128, dt=ta.TA_BF16, scale=0.1, out=0x8000, lse=0x9000, ws=0xa000, wsb=1 << 30)
    a.update(kw)
    return lib.tree_attn_verify(a["q"], a["kv"], a["P"], a["par"], a["n"], a["B"], a["n_max"],
                                a["Hq"], a["Hkv"], a["d"], a["dt"], ctypes.c_float(a["scale"]),
                                a["out"], a["lse"], a["ws"], a["wsb"], None, None)


def test_invalid_arguments_are_rejected_on_the_host():
    lib = ensure_built()
    assert _verify(lib, Hq=7) == _lib.TA_ERR_INVALID_ARG          # Hq % Hkv != 0
    assert _verify(lib, d=96) == _lib.TA_ERR_UNSUPPORTED
    assert _verify(lib, dt=7) == _lib.TA_ERR_UNSUPPORTED
    assert _verify(lib, n_max=257) == _lib.TA_ERR_TREE_TOO_LARGE
    assert _verify(lib, q=None) == _lib.TA_ERR_INVALID_ARG
    assert _verify(lib, scale=0.0) == _lib.TA_ERR_INVALID_ARG
    assert _verify(lib, kv=_lib.ta_kv(0x1000, None, None, 0, 0, 0, 64)) == _lib.TA_ERR_INVALID_ARG
    # paged capacity larger than the block table can address
    assert _verify(lib, kv=_lib.ta_kv(0x1000, 0x2000, 0x3000, 16, 4, 8, 65)) == \
        _lib.TA_ERR_INVALID_ARG
    assert _verify(lib, B=0) == _lib.TA_OK                        # nothing to do
    # a split-kernel plan that does not split needs no workspace; the units
    # kernel (automatic for paged bf16 caches, so part of the layout-independent
    # answer) always needs one: its stream table and two partial slots per group
    need = ta.tree_attn_workspace_bytes(1, 16, 8, 2, 128, ta.TA_BF16, 64, chunk_tokens=64,
                                        kernel=3)
    assert need == 0
    units = ta.tree_attn_workspace_bytes(1, 16, 8, 2, 128, ta.TA_BF16, 64, kernel=4)
    assert units > 0
    assert ta.tree_attn_workspace_bytes(1, 16, 8, 2, 128, ta.TA_BF16, 64) >= units
    # (kernel 3 for both layouts: the query then sizes exactly the plan the
    # contiguous call below runs)
    need = ta.tree_attn_workspace_bytes(2, 16, 8, 2, 128, ta.TA_BF16, 4096, chunk_tokens=256,
                                        kernel=3)
    assert need > 0
    opts = _lib.ta_attn_opts(256, 0)
    st = lib.tree_attn_verify(0x4000, _kv(4096), 0x5000, 0x6000, 0x7000, 2, 16, 8, 2, 128,
                              ta.TA_BF16, ctypes.c_float(0.1), 0x8000, None, None, 0,
                              ctypes.byref(opts), None)
    assert st == _lib.TA_ERR_WORKSPACE
    st = lib.tree_attn_verify(0x4000, _kv(4096), 0x5000, 0x6000, 0x7000, 2, 16, 8, 2, 128,
                              ta.TA_BF16, ctypes.c_float(0.1), 0x8000, None, 0xa000, need - 1,
                              ctypes.byref(opts), None)
    assert st == _lib.TA_ERR_WORKSPACE
    bad = _lib.ta_attn_opts(100, 0)                               # not a multiple of 64
    st = lib.tree_attn_verify(0x4000, _kv(4096), 0x5000, 0x6000, 0x7000, 2, 16, 8, 2, 128,
                              ta.TA_BF16, ctypes.c_float(0.1), 0x8000, None, 0xa000, 1 << 30,
                              ctypes.byref(bad), None)
    assert st == _lib.TA_ERR_UNSUPPORTED
    # expand: w must lie in [1, n_max]
    st = lib.tree_attn_expand(0x4000, _kv(), 0x5000, 0x6000, 0x7000, 2, 17, 16, 8, 2, 128,
                              ta.TA_BF16, ctypes.c_float(0.1), 0x8000, None, 0xa000, 1 << 30,
                              None, None)
    assert st == _lib.TA_ERR_INVALID_ARG
    # accept
    st = lib.accept_greedy_path(0x1000, ta.TA_F32, 0x2000, 0x3000, 0x4000, 0x5000, 2, 300, 10,
                                0x6000, 0x7000, 0x8000, None)
    assert st == _lib.TA_ERR_TREE_TOO_LARGE
    st = lib.accept_greedy_path(0x1000, 5, 0x2000, 0x3000, 0x4000, 0x5000, 2, 16, 10, 0x6000,
                                0x7000, 0x8000, None)
    assert st == _lib.TA_ERR_UNSUPPORTED
    st = lib.accept_greedy_path(None, ta.TA_F32, 0x2000, 0x3000, 0x4000, 0x5000, 2, 16, 10,
                                0x6000, 0x7000, 0x8000, None)
    assert st == _lib.TA_ERR_INVALID_ARG
    # re-root
    arr = (_lib.ta_kv * 1)(_kv())
    st = lib.tree_cache_reroot(arr, 1, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 2, 16, 2,
                               80, ta.TA_BF16, None)
    assert st == _lib.TA_ERR_UNSUPPORTED
    st = lib.tree_cache_reroot(arr, 1, None, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 2, 16, 2,
                               128, ta.TA_BF16, None)
    assert st == _lib.TA_ERR_INVALID_ARG
    arr2 = (_lib.ta_kv * 1)(_lib.ta_kv(0x1001, 0x2000, None, 0, 0, 0, 64))   # misaligned
    st = lib.tree_cache_reroot(arr2, 1, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 2, 16, 2,
                               128, ta.TA_BF16, None)
    assert st == _lib.TA_ERR_INVALID_ARG


def test_top_w_host_side_validation():
    """tree_expand_top_w rejects bad sizes before touching device memory."""
    lib = ensure_built()
    call = lambda B=2, n_max=16, V=100, w=4, dt=ta.TA_F32, ws=0xa000, wsb=1 << 20: \
        lib.tree_expand_top_w(0x1000, dt, 0x2000, 0x3000, 0x4000, 0x5000, B, n_max, V, w, ws,
                              wsb, None)  # noqa: E731
    assert call(w=0) == _lib.TA_ERR_INVALID_ARG
    assert call(w=17) == _lib.TA_ERR_UNSUPPORTED
    assert call(V=(1 << 18) + 1) == _lib.TA_ERR_UNSUPPORTED
    assert call(n_max=257) == _lib.TA_ERR_TREE_TOO_LARGE
    assert call(dt=9) == _lib.TA_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.TA_ERR_WORKSPACE
    need = ta.tree_expand_top_w_workspace_bytes(2, 16, 4)
    assert need == 2 * 17 * 4 * 8
    assert call(wsb=need - 1) == _lib.TA_ERR_WORKSPACE
    assert call(B=0) == _lib.TA_OK
    with pytest.raises(ta.TreeAttnError):
        ta.tree_expand_top_w_workspace_bytes(1, 16, 0)


def test_workspace_query_rejects_bad_sizes():
    ensure_built()
    with pytest.raises(ta.TreeAttnError):
        ta.tree_attn_workspace_bytes(1, 4, 6, 4, 128, ta.TA_BF16, 100)
    assert ta.tree_attn_workspace_bytes(0, 4, 8, 4, 128, ta.TA_BF16, 100) == 0


def test_binding_refuses_host_memory_for_device_arguments():
    """Host tensors never reach the library as device pointers."""
    import torch
    ws = ta.Workspace()
    with pytest.raises(ValueError):
        ws.get(1024, "cpu")
    with pytest.raises(ValueError):
        _lib._need(torch.zeros(4), "workspace")
    with pytest.raises(ValueError):
        ta.KVCache(torch.zeros(1, 4, 1, 64), torch.zeros(1, 4, 1, 64))


def test_draft_side_host_side_validation():
    """tree_token_walk / tree_select_subtree reject bad sizes and null
    pointers before any launch (no GPU needed for these paths)."""
    lib = ensure_built()
    P = 0x1000

    def walk(B=2, n_max=16, m_max=8, ptrs=(P,) * 8):
        return lib.tree_token_walk(*ptrs[:5], B, n_max, m_max, *ptrs[5:], None)

    assert walk(B=0) == _lib.TA_OK
    assert walk(B=-1) == _lib.TA_ERR_INVALID_ARG
    assert walk(n_max=0) == _lib.TA_ERR_INVALID_ARG
    assert walk(n_max=257) == _lib.TA_ERR_TREE_TOO_LARGE
    assert walk(m_max=0) == _lib.TA_ERR_INVALID_ARG
    assert walk(m_max=1025) == _lib.TA_ERR_UNSUPPORTED
    for i in range(8):
        ptrs = [P] * 8
        ptrs[i] = None
        assert walk(ptrs=tuple(ptrs)) == _lib.TA_ERR_INVALID_ARG, i

    def select(B=2, n_max=16, bs=4, ptrs=(P,) * 8):
        return lib.tree_select_subtree(*ptrs[:4], B, n_max, bs, *ptrs[4:], None)

    assert select(B=0) == _lib.TA_OK
    assert select(bs=0) == _lib.TA_ERR_INVALID_ARG
    assert select(bs=17) == _lib.TA_ERR_INVALID_ARG
    assert select(n_max=257, bs=4) == _lib.TA_ERR_TREE_TOO_LARGE
    for i in range(8):
        ptrs = [P] * 8
        ptrs[i] = None
        assert select(ptrs=tuple(ptrs)) == _lib.TA_ERR_INVALID_ARG, i


def test_rope_append_host_side_validation():
    lib = ensure_built()
    P = 0x4000

    def call(B=2, n_q=16, n_max=16, expand=0, Hq=8, Hkv=2, d=128, dt=ta.TA_BF16, base=1e4,
             ptrs=(P,) * 7, kv=None):
        kv = kv if kv is not None else _kv()
        return lib.tree_rope_append(ptrs[0], ptrs[1], ptrs[2], ptrs[3], kv, ptrs[4], ptrs[5],
                                    ptrs[6], B, n_q, n_max, expand, Hq, Hkv, d, dt,
                                    ctypes.c_float(base), None)

    assert call(B=0) == _lib.TA_OK
    assert call(Hq=7) == _lib.TA_ERR_INVALID_ARG
    assert call(d=96) == _lib.TA_ERR_UNSUPPORTED
    assert call(dt=7) == _lib.TA_ERR_UNSUPPORTED
    assert call(n_max=257, n_q=16) == _lib.TA_ERR_TREE_TOO_LARGE
    assert call(n_q=17) == _lib.TA_ERR_INVALID_ARG
    assert call(expand=2) == _lib.TA_ERR_INVALID_ARG
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert call(base=bad) == _lib.TA_ERR_INVALID_ARG, bad
    assert call(kv=_lib.ta_kv(0x1000, None, None, 0, 0, 0, 64)) == _lib.TA_ERR_INVALID_ARG
    for i in range(7):
        ptrs = [P] * 7
        ptrs[i] = None
        assert call(ptrs=tuple(ptrs)) == _lib.TA_ERR_INVALID_ARG, i


def test_accept_sampling_host_side_validation():
    lib = ensure_built()
    P = 0x4000
    ws_need = lib.accept_sampling_workspace_bytes(4, 16)
    assert ws_need == 4 * 16 * 16
    assert lib.accept_sampling_workspace_bytes(4, 257) == ctypes.c_size_t(-1).value
    assert lib.accept_sampling_workspace_bytes(-1, 16) == ctypes.c_size_t(-1).value

    def call(B=4, n_max=16, V=1000, dt=ta.TA_BF16, T=1.0, ptrs=(P,) * 13, ws=P, ws_bytes=ws_need):
        return lib.accept_sampling_path(ptrs[0], ptrs[1], dt, ptrs[2], ptrs[3], ptrs[4], ptrs[5],
                                        ptrs[6], ptrs[7], ctypes.c_float(T), B, n_max, V, ptrs[8],
                                        ptrs[9], ptrs[10], ws, ws_bytes, None)

    assert call(B=0) == _lib.TA_OK
    assert call(B=-1) == _lib.TA_ERR_INVALID_ARG
    assert call(V=0) == _lib.TA_ERR_INVALID_ARG
    assert call(n_max=257) == _lib.TA_ERR_TREE_TOO_LARGE
    assert call(dt=5) == _lib.TA_ERR_UNSUPPORTED
    for bad in (0.0, -1.0, float("nan"), float("inf"), 1e-45):
        assert call(T=bad) == _lib.TA_ERR_INVALID_ARG, bad
    for i in range(11):
        ptrs = [P] * 13
        ptrs[i] = None
        assert call(ptrs=tuple(ptrs)) == _lib.TA_ERR_INVALID_ARG, i
    assert call(ws=None) == _lib.TA_ERR_WORKSPACE
    assert call(ws_bytes=ws_need - 1) == _lib.TA_ERR_WORKSPACE
    assert call(ws=P + 8) == _lib.TA_ERR_WORKSPACE


def _accept_reroot(lib, **kw):
    a = dict(lg=0x1000, ldt=ta.TA_F32, tok=0x2000, rt=0x3000, arr=(_lib.ta_kv * 1)(_kv()), nl=1,
             P=0x4000, par=0x5000, n=0x6000, keep=0x7000, B=2, n_max=16, V=10, Hkv=2, d=128,
             dt=ta.TA_BF16, path=0x8000, plen=0x9000, bonus=0xa000, ws=0xb000, wsb=1 << 20)
    a.update(kw)
    return lib.tree_accept_reroot(a["lg"], a["ldt"], a["tok"], a["rt"], a["arr"], a["nl"], a["P"],
                                  a["par"], a["n"], a["keep"], a["B"], a["n_max"], a["V"],
                                  a["Hkv"], a["d"], a["dt"], a["path"], a["plen"], a["bonus"],
                                  a["ws"], a["wsb"], None)


def test_accept_reroot_host_side_validation():
    """tree_accept_reroot checks what accept_greedy_path and tree_cache_reroot
    check, plus its workspace, before any launch."""
    lib = ensure_built()
    need = ta.tree_accept_reroot_workspace_bytes(2, 16)
    # argmax per node, copies of parent, prefix_len and n_nodes, each on a
    # 256-byte boundary
    assert need == 4 * 256
    assert ta.tree_accept_reroot_workspace_bytes(100, 256) == 2 * 102400 + 2 * 512
    assert lib.tree_accept_reroot_workspace_bytes(-1, 16) == ctypes.c_size_t(-1).value
    assert lib.tree_accept_reroot_workspace_bytes(2, 257) == ctypes.c_size_t(-1).value
    assert _accept_reroot(lib, n_max=300) == _lib.TA_ERR_TREE_TOO_LARGE
    assert _accept_reroot(lib, ldt=5) == _lib.TA_ERR_UNSUPPORTED
    assert _accept_reroot(lib, dt=9) == _lib.TA_ERR_UNSUPPORTED
    assert _accept_reroot(lib, d=80) == _lib.TA_ERR_UNSUPPORTED
    assert _accept_reroot(lib, lg=None) == _lib.TA_ERR_INVALID_ARG
    assert _accept_reroot(lib, keep=None) == _lib.TA_ERR_INVALID_ARG
    assert _accept_reroot(lib, bonus=None) == _lib.TA_ERR_INVALID_ARG
    assert _accept_reroot(lib, nl=-1) == _lib.TA_ERR_INVALID_ARG
    assert _accept_reroot(lib, V=0) == _lib.TA_ERR_INVALID_ARG
    assert _accept_reroot(lib, arr=None) == _lib.TA_ERR_INVALID_ARG
    mis = (_lib.ta_kv * 1)(_lib.ta_kv(0x1001, 0x2000, None, 0, 0, 0, 64))
    assert _accept_reroot(lib, arr=mis) == _lib.TA_ERR_INVALID_ARG
    assert _accept_reroot(lib, ws=None) == _lib.TA_ERR_WORKSPACE
    assert _accept_reroot(lib, wsb=need - 1) == _lib.TA_ERR_WORKSPACE
    assert _accept_reroot(lib, ws=0xb004) == _lib.TA_ERR_WORKSPACE   # not 16-byte aligned
    assert _accept_reroot(lib, B=0, ws=None) == _lib.TA_OK           # nothing to do
    assert _accept_reroot(lib, nl=0, arr=None, B=0) == _lib.TA_OK
