"""ctypes binding of libtreeattn.so (the C ABI declared in include/tree_attn.h).

Argument marshalling only: tensors are checked for shape, dtype, device and
contiguity, their device pointers and torch's current HIP stream are passed
to the library, and status codes become exceptions.  Every step of the hot
path runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtreeattn.so")

TA_OK = 0
TA_ERR_INVALID_ARG = -1
TA_ERR_UNSUPPORTED = -2
TA_ERR_TREE_TOO_LARGE = -3
TA_ERR_WORKSPACE = -4
TA_ERR_HIP = -5
TA_ERR_SCRATCH = -6
TA_F32 = 0
TA_BF16 = 1
TA_MAX_NODES = 256

#: Every symbol include/tree_attn.h declares.
EXPORTED_SYMBOLS = (
    "tree_attn_workspace_bytes",
    "tree_attn_verify",
    "tree_attn_expand",
    "tree_attn_verify_noalloc",
    "tree_attn_verify_rope",
    "tree_attn_expand_rope",
    "accept_greedy_path",
    "accept_sampling_path",
    "accept_sampling_workspace_bytes",
    "tree_cache_reroot",
    "tree_cache_reroot_draft",
    "tree_accept_reroot",
    "tree_accept_reroot_workspace_bytes",
    "tree_expand_top_w",
    "tree_expand_top_w_workspace_bytes",
    "tree_rope_append",
    "tree_token_walk",
    "tree_select_subtree",
    "ta_status_string",
    "ta_version",
    "ta_last_error",
)


class TreeAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class ta_kv(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("T_cap", ctypes.c_int32),
    ]


class ta_attn_opts(ctypes.Structure):
    _fields_ = [("chunk_tokens", ctypes.c_int32), ("kernel", ctypes.c_int32)]


_lib = None
_lib_lock = threading.Lock()


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtreeattn.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the HIP library first "
                "(python -m tree_masked_verify_attn_amd.build)")
        # torch brings its own HIP runtime (soname libamdhip64.so.7, requested by
        # torch under another name).  Loading torch first makes libtreeattn bind
        # to that same runtime by soname; the other order would put two HIP
        # runtimes in the process, and the second one finds no device.
        import torch  # noqa: F401
        lib = ctypes.CDLL(path)
        c_int, c_size, vp, f32 = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
        lib.tree_attn_workspace_bytes.argtypes = [c_int] * 7 + [ctypes.POINTER(ta_attn_opts)]
        lib.tree_attn_workspace_bytes.restype = c_size
        attn = [vp, ta_kv, vp, vp, vp]
        lib.tree_attn_verify.argtypes = attn + [c_int] * 6 + [f32, vp, vp, vp, c_size,
                                                              ctypes.POINTER(ta_attn_opts), vp]
        lib.tree_attn_verify.restype = c_int
        lib.tree_attn_expand.argtypes = attn + [c_int] * 7 + [f32, vp, vp, vp, c_size,
                                                              ctypes.POINTER(ta_attn_opts), vp]
        lib.tree_attn_expand.restype = c_int
        lib.tree_attn_verify_noalloc.argtypes = attn + [c_int] * 6 + [
            f32, vp, vp, ctypes.POINTER(ta_attn_opts), vp]
        lib.tree_attn_verify_noalloc.restype = c_int
        rope_head = [vp, vp, vp, ta_kv, vp, vp, vp]
        lib.tree_attn_verify_rope.argtypes = rope_head + [c_int] * 6 + [
            f32, f32, vp, vp, vp, c_size, ctypes.POINTER(ta_attn_opts), vp]
        lib.tree_attn_verify_rope.restype = c_int
        lib.tree_attn_expand_rope.argtypes = rope_head + [c_int] * 7 + [
            f32, f32, vp, vp, vp, c_size, ctypes.POINTER(ta_attn_opts), vp]
        lib.tree_attn_expand_rope.restype = c_int
        lib.accept_greedy_path.argtypes = [vp, c_int, vp, vp, vp, vp, c_int, c_int, c_int, vp, vp,
                                           vp, vp]
        lib.accept_greedy_path.restype = c_int
        lib.accept_sampling_path.argtypes = [vp, vp, c_int] + [vp] * 6 + [f32] + [c_int] * 3 + \
            [vp] * 4 + [c_size, vp]
        lib.accept_sampling_path.restype = c_int
        lib.accept_sampling_workspace_bytes.argtypes = [c_int, c_int]
        lib.accept_sampling_workspace_bytes.restype = c_size
        lib.tree_cache_reroot.argtypes = [ctypes.POINTER(ta_kv), c_int, vp, vp, vp, vp, vp, vp,
                                          c_int, c_int, c_int, c_int, c_int, vp]
        lib.tree_cache_reroot.restype = c_int
        lib.tree_cache_reroot_draft.argtypes = [ctypes.POINTER(ta_kv), c_int] + [vp] * 8 + \
            [c_int] * 5 + [vp]
        lib.tree_cache_reroot_draft.restype = c_int
        lib.tree_accept_reroot.argtypes = [vp, c_int, vp, vp, ctypes.POINTER(ta_kv), c_int] + \
            [vp] * 4 + [c_int] * 6 + [vp] * 4 + [c_size, vp]
        lib.tree_accept_reroot.restype = c_int
        lib.tree_accept_reroot_workspace_bytes.argtypes = [c_int, c_int]
        lib.tree_accept_reroot_workspace_bytes.restype = c_size
        lib.tree_expand_top_w.argtypes = [vp, c_int, vp, vp, vp, vp, c_int, c_int, c_int, c_int,
                                          vp, c_size, vp]
        lib.tree_expand_top_w.restype = c_int
        lib.tree_expand_top_w_workspace_bytes.argtypes = [c_int, c_int, c_int]
        lib.tree_expand_top_w_workspace_bytes.restype = c_size
        lib.tree_rope_append.argtypes = [vp] * 4 + [ta_kv] + [vp] * 3 + [c_int] * 8 + [f32, vp]
        lib.tree_rope_append.restype = c_int
        lib.tree_token_walk.argtypes = [vp] * 5 + [c_int] * 3 + [vp] * 4
        lib.tree_token_walk.restype = c_int
        lib.tree_select_subtree.argtypes = [vp] * 4 + [c_int] * 3 + [vp] * 5
        lib.tree_select_subtree.restype = c_int
        lib.ta_status_string.argtypes = [c_int]
        lib.ta_status_string.restype = ctypes.c_char_p
        lib.ta_version.argtypes = []
        lib.ta_version.restype = ctypes.c_char_p
        lib.ta_last_error.argtypes = []
        lib.ta_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(status: int):
    if status != TA_OK:
        lib = load_library()
        msg = lib.ta_status_string(status).decode()
        if status == TA_ERR_HIP:
            msg += ": " + lib.ta_last_error().decode()
        raise TreeAttnError(status, msg)


def ta_status_string(status: int) -> str:
    return load_library().ta_status_string(status).decode()


def ta_version() -> str:
    return load_library().ta_version().decode()


def ta_last_error() -> str:
    return load_library().ta_last_error().decode()


# ----------------------------------------------------------------------------
# tensor marshalling
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TA_F32
    if t.dtype == torch.bfloat16:
        return TA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _need(t, name, dtype=None, ndim=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class KVCache:
    """One layer's K/V cache.

    Contiguous: ``k``, ``v`` are ``[B][T_cap][Hkv][d]``.  Paged: ``k``, ``v``
    are ``[num_blocks][block_size][Hkv][d]`` and ``block_table`` is
    ``[B][max_blocks]`` int32; ``T_cap`` defaults to ``max_blocks * block_size``.
    """

    def __init__(self, k, v, block_table=None, T_cap: Optional[int] = None):
        torch = _torch()
        _need(k, "k", ndim=4)
        _need(v, "v", dtype=k.dtype, ndim=4, device=k.device)
        if tuple(k.shape) != tuple(v.shape):
            raise ValueError("k and v must have the same shape")
        self.k, self.v = k, v
        self.block_table = block_table
        if block_table is not None:
            _need(block_table, "block_table", dtype=torch.int32, ndim=2, device=k.device)
            self.block_size = int(k.shape[1])
            self.max_blocks = int(block_table.shape[1])
            self.num_blocks = int(k.shape[0])
            self.T_cap = int(T_cap) if T_cap is not None else self.max_blocks * self.block_size
        else:
            self.block_size = self.max_blocks = self.num_blocks = 0
            self.T_cap = int(k.shape[1]) if T_cap is None else int(T_cap)
        self.Hkv = int(k.shape[2])
        self.d = int(k.shape[3])

    @property
    def dtype(self):
        return self.k.dtype

    def struct(self) -> ta_kv:
        return ta_kv(self.k.data_ptr(), self.v.data_ptr(), _ptr(self.block_table),
                     self.block_size, self.max_blocks, self.num_blocks, self.T_cap)


def _opts(chunk_tokens: int = 0, kernel: int = 0):
    if not chunk_tokens and not kernel:
        return None
    return ctypes.byref(ta_attn_opts(int(chunk_tokens), int(kernel)))


def tree_attn_workspace_bytes(B: int, n_q: int, Hq: int, Hkv: int, d: int, dtype: int,
                              T_cap: int, chunk_tokens: int = 0, kernel: int = 0) -> int:
    n = load_library().tree_attn_workspace_bytes(B, n_q, Hq, Hkv, d, dtype, T_cap,
                                                 _opts(chunk_tokens, kernel))
    if n == ctypes.c_size_t(-1).value:
        raise TreeAttnError(TA_ERR_INVALID_ARG, "invalid sizes for a workspace query")
    return int(n)


class Workspace:
    """A device buffer for split-KV partial results, reused across attention calls.

    It grows when a plan needs more room; its contents need no initialisation.
    Calls sharing one workspace must be ordered (one stream).
    """

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, device=None, stream=None):
        """The buffer (at least ``nbytes``) on ``device`` (default: the one given at
        construction); always device memory, never host memory.  ``stream``
        (a torch stream) is the stream the call runs on: a buffer that is
        replaced is marked as used there, so that the caching allocator does
        not hand its memory out while a queued kernel may still read it."""
        torch = _torch()
        if nbytes == 0:
            return None
        dev = torch.device(device if device is not None else self.device)
        if dev.type != "cuda":
            raise ValueError("a workspace must live in GPU memory")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != dev:
            if self.buf is not None and stream is not None and self.buf.device == dev:
                self.buf.record_stream(stream)
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
        return self.buf


# Implicit workspaces, one per (device, stream): calls on different streams
# never share one.
_default_ws = {}


def _torch_stream(stream, device):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device)
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _workspace_for(device, nbytes, stream=None):
    ts = _torch_stream(stream, device)
    key = (str(device), int(ts.cuda_stream))
    ws = _default_ws.get(key)
    if ws is None:
        ws = _default_ws[key] = Workspace(device)
    return ws.get(nbytes, stream=ts)


def _attention(fn_name, q, kv: KVCache, prefix_len, parent, n_nodes, scale, out, lse, workspace,
               w, chunk_tokens, kernel, stream, with_lse, rope=None):
    """Marshals one attention call; ``fn_name`` is "verify", "expand" or
    "verify_noalloc" (no workspace: the library's fixed scratch array);
    ``rope`` = (k_new, v_new, base) selects the RoPE-fused entry points."""
    torch = _torch()
    lib = load_library()
    _need(q, "q", dtype=kv.dtype, ndim=4, device=kv.k.device)
    dev = kv.k.device
    _need(prefix_len, "prefix_len", dtype=torch.int32, ndim=1, device=dev)
    _need(parent, "parent", dtype=torch.int32, ndim=2, device=dev)
    _need(n_nodes, "n_nodes", dtype=torch.int32, ndim=1, device=dev)
    B, n_q, Hq, d = (int(x) for x in q.shape)
    n_max = int(parent.shape[1])
    if parent.shape[0] != B or prefix_len.shape[0] != B or n_nodes.shape[0] != B:
        raise ValueError("batch size mismatch between q and prefix_len/parent/n_nodes")
    if d != kv.d:
        raise ValueError("head dim of q and kv differ")
    if kv.block_table is not None and kv.block_table.shape[0] != B:
        raise ValueError("block_table must have one row per sequence")
    if kv.block_table is None and kv.k.shape[0] != B:
        raise ValueError("contiguous k/v must have one row per sequence")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", dtype=q.dtype, device=dev)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must have q's shape")
    if lse is None and with_lse:
        lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", dtype=torch.float32, device=dev)
        if tuple(lse.shape) != (B, Hq, n_q):
            raise ValueError("lse must be [B][Hq][n_q]")
    common = (q.data_ptr(), kv.struct(), prefix_len.data_ptr(), parent.data_ptr(),
              n_nodes.data_ptr())
    if fn_name == "verify_noalloc":
        if n_q != n_max:
            raise ValueError("verify queries must be [B][n_max][Hq][d]")
        st = lib.tree_attn_verify_noalloc(*common, B, n_max, Hq, kv.Hkv, d, dt,
                                          ctypes.c_float(scale), out.data_ptr(), _ptr(lse),
                                          _opts(chunk_tokens, kernel), _stream(stream))
        _check(st)
        return out, lse
    nbytes = tree_attn_workspace_bytes(B, n_q, Hq, kv.Hkv, d, dt, kv.T_cap, chunk_tokens, kernel)
    if workspace is None:
        ws = _workspace_for(dev, nbytes, stream)
    else:
        ws = (workspace.get(nbytes, dev, _torch_stream(stream, dev))
              if isinstance(workspace, Workspace) else workspace)
    if ws is not None:
        _need(ws, "workspace", device=dev)   # device memory of this call's GPU only
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    tail = (ctypes.c_float(scale), out.data_ptr(), _ptr(lse), _ptr(ws), ws_bytes,
            _opts(chunk_tokens, kernel), _stream(stream))
    if rope is not None:
        k_new, v_new, base = rope
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            _need(t, name, dtype=q.dtype, ndim=4, device=dev)
            if tuple(t.shape) != (B, n_q, kv.Hkv, d):
                raise ValueError(f"{name} must be [B][n_q][Hkv][d] = {(B, n_q, kv.Hkv, d)}")
        if out.data_ptr() in (q.data_ptr(), k_new.data_ptr(), v_new.data_ptr()):
            raise ValueError("out must not alias q, k_new or v_new")
        rtail = (ctypes.c_float(scale), ctypes.c_float(base)) + tail[1:]
        head = (q.data_ptr(), k_new.data_ptr(), v_new.data_ptr()) + common[1:]
        if fn_name == "verify":
            if n_q != n_max:
                raise ValueError("verify queries must be [B][n_max][Hq][d]")
            st = lib.tree_attn_verify_rope(*head, B, n_max, Hq, kv.Hkv, d, dt, *rtail)
        else:
            st = lib.tree_attn_expand_rope(*head, B, w, n_max, Hq, kv.Hkv, d, dt, *rtail)
        _check(st)
        return out, lse
    if fn_name == "verify":
        if n_q != n_max:
            raise ValueError("verify queries must be [B][n_max][Hq][d]")
        st = lib.tree_attn_verify(*common, B, n_max, Hq, kv.Hkv, d, dt, *tail)
    else:
        st = lib.tree_attn_expand(*common, B, w, n_max, Hq, kv.Hkv, d, dt, *tail)
    _check(st)
    return out, lse


def tree_attn_verify(q, kv: KVCache, prefix_len, parent, n_nodes, scale: float, out=None,
                     lse=None, workspace=None, chunk_tokens: int = 0, kernel: int = 0,
                     stream=None, with_lse: bool = True):
    """Verification attention over every tree node; returns ``(out, lse)``."""
    return _attention("verify", q, kv, prefix_len, parent, n_nodes, scale, out, lse, workspace,
                      0, chunk_tokens, kernel, stream, with_lse)


def tree_attn_verify_noalloc(q, kv: KVCache, prefix_len, parent, n_nodes, scale: float, out=None,
                             lse=None, chunk_tokens: int = 0, kernel: int = 0, stream=None,
                             with_lse: bool = True):
    """tree_attn_verify without a workspace: the library keeps the split
    partial results in its fixed per-GPU scratch array and allocates nothing
    (pass ``out`` and ``lse`` to allocate nothing on this side either).
    Calls that overlap in time on one GPU race on that array."""
    return _attention("verify_noalloc", q, kv, prefix_len, parent, n_nodes, scale, out, lse,
                      None, 0, chunk_tokens, kernel, stream, with_lse)


def tree_attn_verify_rope(q, k_new, v_new, kv: KVCache, prefix_len, parent, n_nodes, scale: float,
                          base: float = 10000.0, out=None, lse=None, workspace=None,
                          chunk_tokens: int = 0, kernel: int = 0, stream=None,
                          with_lse: bool = True):
    """Verification attention with RoPE fused in: rotates ``q`` and the new
    nodes' keys ``k_new`` to their tree positions, writes keys and values
    ``v_new`` to cache rows P + node, attends; returns ``(out, lse)``."""
    return _attention("verify", q, kv, prefix_len, parent, n_nodes, scale, out, lse, workspace,
                      0, chunk_tokens, kernel, stream, with_lse, rope=(k_new, v_new, float(base)))


def tree_attn_expand_rope(q, k_new, v_new, kv: KVCache, prefix_len, parent, n_nodes, scale: float,
                          base: float = 10000.0, out=None, lse=None, workspace=None,
                          chunk_tokens: int = 0, kernel: int = 0, stream=None,
                          with_lse: bool = True):
    """Expansion attention for the ``w = q.shape[1]`` newest nodes with RoPE
    fused in (their keys and values appended as by tree_rope_append)."""
    return _attention("expand", q, kv, prefix_len, parent, n_nodes, scale, out, lse, workspace,
                      int(q.shape[1]), chunk_tokens, kernel, stream, with_lse,
                      rope=(k_new, v_new, float(base)))


def tree_attn_expand(q, kv: KVCache, prefix_len, parent, n_nodes, scale: float, out=None,
                     lse=None, workspace=None, chunk_tokens: int = 0, kernel: int = 0,
                     stream=None, with_lse: bool = True):
    """Expansion attention for the ``w = q.shape[1]`` newest nodes; returns ``(out, lse)``."""
    return _attention("expand", q, kv, prefix_len, parent, n_nodes, scale, out, lse, workspace,
                      int(q.shape[1]), chunk_tokens, kernel, stream, with_lse)


def accept_greedy_path(logits, parent, tok, n_nodes, root_tok, path=None, path_len=None,
                       bonus=None, stream=None):
    """Greedy longest accepted path; returns ``(path, path_len, bonus)`` int32 tensors."""
    torch = _torch()
    lib = load_library()
    _need(logits, "logits", ndim=3)
    dev = logits.device
    _need(parent, "parent", dtype=torch.int32, ndim=2, device=dev)
    _need(tok, "tok", dtype=torch.int32, ndim=2, device=dev)
    _need(n_nodes, "n_nodes", dtype=torch.int32, ndim=1, device=dev)
    _need(root_tok, "root_tok", dtype=torch.int32, ndim=1, device=dev)
    B, n_max, V = (int(x) for x in logits.shape)
    if tuple(parent.shape) != (B, n_max) or tuple(tok.shape) != (B, n_max):
        raise ValueError("parent/tok must be [B][n_max] matching logits")
    if path is None:
        path = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(path, "path", dtype=torch.int32, ndim=2, device=dev)
    _need(path_len, "path_len", dtype=torch.int32, ndim=1, device=dev)
    _need(bonus, "bonus", dtype=torch.int32, ndim=1, device=dev)
    if tuple(path.shape) != (B, n_max) or path_len.shape[0] != B or bonus.shape[0] != B:
        raise ValueError("path must be [B][n_max], path_len and bonus [B]")
    st = lib.accept_greedy_path(logits.data_ptr(), _dtype_code(logits), parent.data_ptr(),
                                tok.data_ptr(), n_nodes.data_ptr(), root_tok.data_ptr(), B, n_max,
                                V, path.data_ptr(), path_len.data_ptr(), bonus.data_ptr(),
                                _stream(stream))
    _check(st)
    return path, path_len, bonus


def accept_sampling_workspace_bytes(B: int, n_max: int) -> int:
    n = load_library().accept_sampling_workspace_bytes(B, n_max)
    if n == ctypes.c_size_t(-1).value:
        raise TreeAttnError(TA_ERR_INVALID_ARG, "invalid sizes for a sampling workspace query")
    return int(n)


def accept_sampling_path(target_logits, draft_logits, parent, tok, n_nodes, root_tok, u_accept,
                         u_bonus, temperature: float, path=None, path_len=None, bonus=None,
                         workspace=None, stream=None):
    """Tree verification by speculative sampling; returns ``(path, path_len,
    bonus)`` int32 tensors.  ``u_accept [B][n_max]`` and ``u_bonus [B]`` are
    fp32 uniforms in [0, 1) drawn by the caller."""
    torch = _torch()
    lib = load_library()
    _need(target_logits, "target_logits", ndim=3)
    dev = target_logits.device
    _need(draft_logits, "draft_logits", dtype=target_logits.dtype, ndim=3, device=dev)
    _need(parent, "parent", dtype=torch.int32, ndim=2, device=dev)
    _need(tok, "tok", dtype=torch.int32, ndim=2, device=dev)
    _need(n_nodes, "n_nodes", dtype=torch.int32, ndim=1, device=dev)
    _need(root_tok, "root_tok", dtype=torch.int32, ndim=1, device=dev)
    _need(u_accept, "u_accept", dtype=torch.float32, ndim=2, device=dev)
    _need(u_bonus, "u_bonus", dtype=torch.float32, ndim=1, device=dev)
    B, n_max, V = (int(x) for x in target_logits.shape)
    if tuple(draft_logits.shape) != (B, n_max, V):
        raise ValueError("draft_logits must have target_logits' shape")
    for t, name in ((parent, "parent"), (tok, "tok"), (u_accept, "u_accept")):
        if tuple(t.shape) != (B, n_max):
            raise ValueError(f"{name} must be [B][n_max] matching the logits")
    if n_nodes.shape[0] != B or root_tok.shape[0] != B or u_bonus.shape[0] != B:
        raise ValueError("n_nodes, root_tok and u_bonus must be [B]")
    if path is None:
        path = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(path, "path", dtype=torch.int32, ndim=2, device=dev)
    _need(path_len, "path_len", dtype=torch.int32, ndim=1, device=dev)
    _need(bonus, "bonus", dtype=torch.int32, ndim=1, device=dev)
    if tuple(path.shape) != (B, n_max) or path_len.shape[0] != B or bonus.shape[0] != B:
        raise ValueError("path must be [B][n_max], path_len and bonus [B]")
    nbytes = accept_sampling_workspace_bytes(B, n_max)
    if workspace is None:
        ws = _workspace_for(dev, nbytes, stream)
    else:
        ws = (workspace.get(nbytes, dev, _torch_stream(stream, dev))
              if isinstance(workspace, Workspace) else workspace)
    if ws is not None:
        _need(ws, "workspace", device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.accept_sampling_path(target_logits.data_ptr(), draft_logits.data_ptr(),
                                  _dtype_code(target_logits), parent.data_ptr(), tok.data_ptr(),
                                  n_nodes.data_ptr(), root_tok.data_ptr(), u_accept.data_ptr(),
                                  u_bonus.data_ptr(), ctypes.c_float(float(temperature)), B,
                                  n_max, V, path.data_ptr(), path_len.data_ptr(),
                                  bonus.data_ptr(), _ptr(ws), ws_bytes, _stream(stream))
    _check(st)
    return path, path_len, bonus


def _reroot(kv_layers, prefix_len, parent, n_nodes, path, path_len, keep_subtree, tok, cum,
            stream, draft):
    torch = _torch()
    lib = load_library()
    dev = parent.device
    _need(prefix_len, "prefix_len", dtype=torch.int32, ndim=1, device=dev)
    _need(parent, "parent", dtype=torch.int32, ndim=2, device=dev)
    _need(n_nodes, "n_nodes", dtype=torch.int32, ndim=1, device=dev)
    _need(path, "path", dtype=torch.int32, ndim=2, device=dev)
    _need(path_len, "path_len", dtype=torch.int32, ndim=1, device=dev)
    _need(keep_subtree, "keep_subtree", dtype=torch.uint8, ndim=1, device=dev)
    B, n_max = (int(x) for x in parent.shape)
    if draft:
        _need(tok, "tok", dtype=torch.int32, ndim=2, device=dev)
        if tuple(tok.shape) != (B, n_max):
            raise ValueError("tok must be [B][n_max] like parent")
        if cum is not None:
            _need(cum, "cum", dtype=torch.float32, ndim=2, device=dev)
            if tuple(cum.shape) != (B, n_max):
                raise ValueError("cum must be [B][n_max] like parent")
    layers: List[KVCache] = list(kv_layers)
    if layers:
        Hkv, d, dtype = layers[0].Hkv, layers[0].d, layers[0].dtype
        for L in layers:
            if (L.Hkv, L.d, L.dtype) != (Hkv, d, dtype) or L.k.device != dev:
                raise ValueError("all layers must share Hkv, d, dtype and device")
        dt = _dtype_code(layers[0].k)
    else:
        Hkv, d, dt = 1, 128, TA_BF16
    arr = (ta_kv * max(1, len(layers)))(*[L.struct() for L in layers])
    head = (arr, len(layers), prefix_len.data_ptr(), parent.data_ptr(), n_nodes.data_ptr(),
            path.data_ptr(), path_len.data_ptr(), keep_subtree.data_ptr())
    if draft:
        st = lib.tree_cache_reroot_draft(*head, tok.data_ptr(), _ptr(cum), B, n_max, Hkv, d, dt,
                                         _stream(stream))
    else:
        st = lib.tree_cache_reroot(*head, B, n_max, Hkv, d, dt, _stream(stream))
    _check(st)


def tree_cache_reroot(kv_layers: Sequence[KVCache], prefix_len, parent, n_nodes, path, path_len,
                      keep_subtree, stream=None):
    """In-place re-root of every layer's cache and of prefix_len/parent/n_nodes."""
    _reroot(kv_layers, prefix_len, parent, n_nodes, path, path_len, keep_subtree, None, None,
            stream, False)


def tree_cache_reroot_draft(kv_layers: Sequence[KVCache], prefix_len, parent, n_nodes, path,
                            path_len, keep_subtree, tok, cum=None, stream=None):
    """tree_cache_reroot that also moves the draft's per-node tokens ``tok``
    and (re-based to the new root) cumulative scores ``cum``, in place."""
    _reroot(kv_layers, prefix_len, parent, n_nodes, path, path_len, keep_subtree, tok, cum,
            stream, True)


def tree_accept_reroot_workspace_bytes(B: int, n_max: int) -> int:
    n = load_library().tree_accept_reroot_workspace_bytes(B, n_max)
    if n == ctypes.c_size_t(-1).value:
        raise TreeAttnError(TA_ERR_INVALID_ARG, "invalid sizes for an accept + re-root workspace query")
    return int(n)


def tree_accept_reroot(logits, tok, root_tok, kv_layers: Sequence[KVCache], prefix_len, parent,
                       n_nodes, keep_subtree, path=None, path_len=None, bonus=None,
                       workspace=None, stream=None):
    """accept_greedy_path, then tree_cache_reroot on the path it finds (two
    launches).  Returns ``(path, path_len, bonus)``; the caches and
    prefix_len / parent / n_nodes are updated in place.  ``workspace``
    defaults to the one kept per (device, stream)."""
    torch = _torch()
    lib = load_library()
    _need(logits, "logits", ndim=3)
    dev = logits.device
    _need(tok, "tok", dtype=torch.int32, ndim=2, device=dev)
    _need(root_tok, "root_tok", dtype=torch.int32, ndim=1, device=dev)
    _need(prefix_len, "prefix_len", dtype=torch.int32, ndim=1, device=dev)
    _need(parent, "parent", dtype=torch.int32, ndim=2, device=dev)
    _need(n_nodes, "n_nodes", dtype=torch.int32, ndim=1, device=dev)
    _need(keep_subtree, "keep_subtree", dtype=torch.uint8, ndim=1, device=dev)
    B, n_max, V = (int(x) for x in logits.shape)
    if tuple(parent.shape) != (B, n_max) or tuple(tok.shape) != (B, n_max):
        raise ValueError("parent/tok must be [B][n_max] matching logits")
    if path is None:
        path = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if bonus is None:
        bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    _need(path, "path", dtype=torch.int32, ndim=2, device=dev)
    _need(path_len, "path_len", dtype=torch.int32, ndim=1, device=dev)
    _need(bonus, "bonus", dtype=torch.int32, ndim=1, device=dev)
    if tuple(path.shape) != (B, n_max) or path_len.shape[0] != B or bonus.shape[0] != B:
        raise ValueError("path must be [B][n_max], path_len and bonus [B]")
    layers: List[KVCache] = list(kv_layers)
    if layers:
        Hkv, d, dtype = layers[0].Hkv, layers[0].d, layers[0].dtype
        for L in layers:
            if (L.Hkv, L.d, L.dtype) != (Hkv, d, dtype) or L.k.device != dev:
                raise ValueError("all layers must share Hkv, d, dtype and device")
        dt = _dtype_code(layers[0].k)
    else:
        Hkv, d, dt = 1, 128, TA_BF16
    arr = (ta_kv * max(1, len(layers)))(*[L.struct() for L in layers])
    nbytes = tree_accept_reroot_workspace_bytes(B, n_max)
    if workspace is None:
        ws = _workspace_for(dev, nbytes, stream)
    else:
        ws = workspace.get(nbytes, dev, _torch_stream(stream, dev))
    st = lib.tree_accept_reroot(logits.data_ptr(), _dtype_code(logits), tok.data_ptr(),
                                root_tok.data_ptr(), arr, len(layers), prefix_len.data_ptr(),
                                parent.data_ptr(), n_nodes.data_ptr(), keep_subtree.data_ptr(), B,
                                n_max, V, Hkv, d, dt, path.data_ptr(), path_len.data_ptr(),
                                bonus.data_ptr(), _ptr(ws), nbytes if ws is not None else 0,
                                _stream(stream))
    _check(st)
    return path, path_len, bonus


def tree_expand_top_w_workspace_bytes(B: int, n_max: int, w: int) -> int:
    n = load_library().tree_expand_top_w_workspace_bytes(B, n_max, w)
    if n == ctypes.c_size_t(-1).value:
        raise TreeAttnError(TA_ERR_INVALID_ARG, "invalid sizes for a top-w workspace query")
    return int(n)


def tree_expand_top_w(logits, parent, tok, cum, n_nodes, w: int, workspace=None, stream=None):
    """Append the ``w`` best new leaves (in place: parent, tok, cum, n_nodes).

    ``logits`` is ``[B][n_max + 1][V]`` (row 0: after the root, row 1 + i:
    after node i), fp32 or bf16; ``cum`` is the fp32 cumulative score of each
    node.  Returns ``n_nodes``.
    """
    torch = _torch()
    lib = load_library()
    _need(logits, "logits", ndim=3)
    dev = logits.device
    _need(parent, "parent", dtype=torch.int32, ndim=2, device=dev)
    _need(tok, "tok", dtype=torch.int32, ndim=2, device=dev)
    _need(cum, "cum", dtype=torch.float32, ndim=2, device=dev)
    _need(n_nodes, "n_nodes", dtype=torch.int32, ndim=1, device=dev)
    B, rows, V = (int(x) for x in logits.shape)
    n_max = int(parent.shape[1])
    if rows != n_max + 1:
        raise ValueError("logits must be [B][n_max + 1][V]")
    for t, name in ((parent, "parent"), (tok, "tok"), (cum, "cum")):
        if tuple(t.shape) != (B, n_max):
            raise ValueError(f"{name} must be [B][n_max]")
    if n_nodes.shape[0] != B:
        raise ValueError("n_nodes must be [B]")
    nbytes = tree_expand_top_w_workspace_bytes(B, n_max, int(w))
    if workspace is None:
        ws = _workspace_for(dev, nbytes, stream)
    else:
        ws = (workspace.get(nbytes, dev, _torch_stream(stream, dev))
              if isinstance(workspace, Workspace) else workspace)
    if ws is not None:
        _need(ws, "workspace", device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib.tree_expand_top_w(logits.data_ptr(), _dtype_code(logits), parent.data_ptr(),
                               tok.data_ptr(), cum.data_ptr(), n_nodes.data_ptr(), B, n_max, V,
                               int(w), _ptr(ws), ws_bytes, _stream(stream))
    _check(st)
    return n_nodes


def tree_token_walk(parent, tok, n_nodes, verified, verified_len, path=None, path_len=None,
                    keep=None, stream=None):
    """Walk the draft tree along the verified tokens; returns ``(path,
    path_len, keep)``, the re-root arguments of ``tree_cache_reroot``."""
    torch = _torch()
    lib = load_library()
    _need(parent, "parent", dtype=torch.int32, ndim=2)
    dev = parent.device
    _need(tok, "tok", dtype=torch.int32, ndim=2, device=dev)
    _need(n_nodes, "n_nodes", dtype=torch.int32, ndim=1, device=dev)
    _need(verified, "verified", dtype=torch.int32, ndim=2, device=dev)
    _need(verified_len, "verified_len", dtype=torch.int32, ndim=1, device=dev)
    B, n_max = (int(x) for x in parent.shape)
    m_max = int(verified.shape[1])
    if tuple(tok.shape) != (B, n_max) or n_nodes.shape[0] != B:
        raise ValueError("tok must be [B][n_max] and n_nodes [B]")
    if verified.shape[0] != B or verified_len.shape[0] != B:
        raise ValueError("verified must be [B][m_max] and verified_len [B]")
    if path is None:
        path = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if keep is None:
        keep = torch.empty((B,), dtype=torch.uint8, device=dev)
    _need(path, "path", dtype=torch.int32, ndim=2, device=dev)
    _need(path_len, "path_len", dtype=torch.int32, ndim=1, device=dev)
    _need(keep, "keep", dtype=torch.uint8, ndim=1, device=dev)
    if tuple(path.shape) != (B, n_max) or path_len.shape[0] != B or keep.shape[0] != B:
        raise ValueError("path must be [B][n_max], path_len and keep [B]")
    st = lib.tree_token_walk(parent.data_ptr(), tok.data_ptr(), n_nodes.data_ptr(),
                             verified.data_ptr(), verified_len.data_ptr(), B, n_max, m_max,
                             path.data_ptr(), path_len.data_ptr(), keep.data_ptr(), _stream(stream))
    _check(st)
    return path, path_len, keep


def tree_select_subtree(cum, parent, tok, n_nodes, bs: int, sel_node=None, sel_parent=None,
                        sel_tok=None, sel_n=None, stream=None):
    """The subtree of ``bs`` nodes to send; returns ``(sel_node, sel_parent,
    sel_tok, sel_n)`` ([B][bs], [B][bs], [B][bs], [B])."""
    torch = _torch()
    lib = load_library()
    _need(cum, "cum", dtype=torch.float32, ndim=2)
    dev = cum.device
    _need(parent, "parent", dtype=torch.int32, ndim=2, device=dev)
    _need(tok, "tok", dtype=torch.int32, ndim=2, device=dev)
    _need(n_nodes, "n_nodes", dtype=torch.int32, ndim=1, device=dev)
    B, n_max = (int(x) for x in cum.shape)
    bs = int(bs)
    if tuple(parent.shape) != (B, n_max) or tuple(tok.shape) != (B, n_max) or n_nodes.shape[0] != B:
        raise ValueError("parent/tok must be [B][n_max] like cum, n_nodes [B]")
    outs = []
    for t, name, shape in ((sel_node, "sel_node", (B, bs)), (sel_parent, "sel_parent", (B, bs)),
                           (sel_tok, "sel_tok", (B, bs)), (sel_n, "sel_n", (B,))):
        if t is None:
            t = torch.empty(shape, dtype=torch.int32, device=dev)
        _need(t, name, dtype=torch.int32, ndim=len(shape), device=dev)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
        outs.append(t)
    st = lib.tree_select_subtree(cum.data_ptr(), parent.data_ptr(), tok.data_ptr(),
                                 n_nodes.data_ptr(), B, n_max, bs, outs[0].data_ptr(),
                                 outs[1].data_ptr(), outs[2].data_ptr(), outs[3].data_ptr(),
                                 _stream(stream))
    _check(st)
    return tuple(outs)


def tree_rope_append(q, k_new, v_new, kv: "KVCache", prefix_len, parent, n_nodes,
                     base: float = 10000.0, expand: bool = False, q_out=None, stream=None):
    """RoPE of the query rows and the new nodes' keys at their tree positions,
    and the append of those keys and values to the cache; returns the rotated
    queries (``q_out``, which may be ``q`` itself)."""
    torch = _torch()
    lib = load_library()
    _need(q, "q", ndim=4)
    dev = q.device
    B, n_q, Hq, d = (int(x) for x in q.shape)
    _need(k_new, "k_new", dtype=q.dtype, ndim=4, device=dev)
    _need(v_new, "v_new", dtype=q.dtype, ndim=4, device=dev)
    if tuple(k_new.shape) != (B, n_q, kv.Hkv, d) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new and v_new must be [B][n_q][Hkv][d]")
    if kv.dtype != q.dtype or kv.d != d:
        raise ValueError("the cache must match q in dtype and head size")
    _need(prefix_len, "prefix_len", dtype=torch.int32, ndim=1, device=dev)
    _need(parent, "parent", dtype=torch.int32, ndim=2, device=dev)
    _need(n_nodes, "n_nodes", dtype=torch.int32, ndim=1, device=dev)
    n_max = int(parent.shape[1])
    if parent.shape[0] != B or prefix_len.shape[0] != B or n_nodes.shape[0] != B:
        raise ValueError("prefix_len, parent and n_nodes must have B rows")
    if q_out is None:
        q_out = torch.empty_like(q)
    _need(q_out, "q_out", dtype=q.dtype, ndim=4, device=dev)
    if tuple(q_out.shape) != tuple(q.shape):
        raise ValueError("q_out must have the shape of q")
    st = lib.tree_rope_append(q.data_ptr(), q_out.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                              kv.struct(), prefix_len.data_ptr(), parent.data_ptr(),
                              n_nodes.data_ptr(), B, n_q, n_max, int(bool(expand)), Hq, kv.Hkv,
                              d, _dtype_code(q), ctypes.c_float(base), _stream(stream))
    _check(st)
    return q_out
