"""Benchmark of the tree-verify hot path on one MI355X.

Default workload, ``chain_verify``: batch 16, Hq=64, Hkv=8, d=128, bf16,
prefix 32768 per sequence, D = 15 chain drafts -> 128 query rows per KV head.
One step = one pass of the whole path over one batch:

    tree_attn_verify -> tree_accept_reroot (greedy accept + re-root, 2 launches)

followed by restoring the three tiny per-sequence arrays the re-root rewrote
(prefix_len, parent, n_nodes: one small elementwise kernel), so that every
step sees the same input.  All inputs are resident in HBM before timing
starts.  The KV cache is 2.15 GB per call, far beyond the 256 MB Infinity
Cache, so every step reads it cold.

By default the K timed steps are captured once in a HIP graph and replayed
(the entry points read every size from device memory and allocate nothing, so
a decode loop can do the same); ``--eager`` issues every call from Python
inside the timed region instead.

Other workloads (``--workload``), each printing the same kind of line:

  paged_alternating  two batches of 32 requests, prefix ~ U[512, 8192], paged
                     KV in 16-token blocks, chain k = 5, Hq=64, Hkv=8, d=128;
                     step s runs the path on batch s mod 2 while the other
                     batch's blocks stay resident (1.14 GB of KV in all).
  tree_verify_l70b   batch 8, Hq=16, Hkv=2, d=128, prefix 4096, 8-node random
                     trees; step s reads KV copy s mod 16 (16 layers' worth,
                     538 MB), so no step finds its KV in the Infinity Cache.
  draft_expand       batch 1, Hq=32, Hkv=8, d=128, prefix 2048, a 64-node tree
                     grown by 4 rounds of 8 new leaves; each round selects the
                     leaves on the device (tree_expand_top_w over the root's
                     and every node's 32000-way distribution) and attends them
                     (tree_attn_expand), on KV copy s mod 64 (563 MB in all);
                     then the walk along the verified tokens, the re-root of
                     the KV rows, tokens and weights, and the choice of the
                     bs = 8 nodes to send (tree_token_walk,
                     tree_cache_reroot_draft, tree_select_subtree).

Prints one JSON line (metric, value = microseconds per step, roofline of the
attention call, CPU-oracle baseline on a bounded sample).  Without
--workload the line is chain_verify's, and the other three workloads are
timed after it in the same process and reported under "other_workloads"
(their step, attention call and HBM fraction; not part of value).

    python bench.py [--workload W] [--steps K] [--warmup W] [--eager] [--no-cpu-baseline] [--no-others]
    python bench.py --copy-calib     # plain device copy of known size (PMC scaling)
"""
from __future__ import annotations

import argparse
import copy
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD's published peak
METRIC = "tree-verify attention µs/step + achieved KV-read GB/s (% of MI355X HBM peak)"
WORKLOADS = ("chain_verify", "paged_alternating", "tree_verify_l70b", "draft_expand")
OTHER_WORKLOADS = WORKLOADS[1:]  # timed beside the default workload's line


def r_phase0(r):
    """Name of a result's first phase (the attention calls)."""
    return "verify" if "verify_us" in r else "expand"
PHASE_REPS = 5                  # timed replays of each single-phase graph
MIN_TIMED_CALLS = 50            # individually timed calls per phase (per-call percentiles)


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"verify_attn_{workload}_traffic.txt")


def kernel_source_hash() -> str:
    """Hash of the attention kernel sources (ties PMC traffic to a kernel version)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_masked_verify_attn_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.startswith("attn_") or f in ("ta_device.h", "ta_internal.h", "stream_common.h",
                                          "partial_f16.h", "rope_common.h", "api.cpp"):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per attention call from the committed PMC summary, if it still
    describes the current kernel sources; else None."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attn_bytes(prefix_len, n_nodes, n_rows, Hq, Hkv, d, eb=2) -> dict:
    """Bytes an attention call must move: K and V once per (sequence, KV head)
    over P + n positions, Q in, O out, LSE out (n_rows query rows per sequence)."""
    kv = sum(2 * (int(p) + int(n)) * Hkv * d * eb for p, n in zip(prefix_len, n_nodes))
    rows = sum(int(r) for r in n_rows)
    q = rows * Hq * d * eb
    return {"kv": kv, "q": q, "o": q, "lse": rows * Hq * 4, "total": kv + 2 * q + rows * Hq * 4}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def _subcase(c, sl):
    """The requests ``sl`` of a case, as a case of their own (host arrays only)."""
    s = copy.copy(c)
    for name in ("q", "prefix_len", "parent", "n_nodes", "tok", "root_tok", "logits",
                 "block_table"):
        val = getattr(c, name)
        if val is not None:
            setattr(s, name, val[sl])
    if c.block_table is None:
        s.k, s.v = c.k[sl], c.v[sl]
    s.B = s.q.shape[0]
    return s


def cpu_verify_step(c, budget_s: float) -> dict:
    """Time the oracle (as it stands) on a bounded sample of one verify step of
    case ``c`` (attention blocks, then accept and re-root) and scale it to
    microseconds per full step."""
    import numpy as np

    import oracle
    pairs = [(b, hk) for b in range(c.B) for hk in range(c.Hkv)]
    order = np.random.default_rng(0).permutation(len(pairs))
    t_attn, done = 0.0, 0
    for j in order:
        b, hk = pairs[j]
        t0 = time.perf_counter()
        oracle.verify(c, batches=[b], heads=list(range(hk * c.G, (hk + 1) * c.G)))
        t_attn += time.perf_counter() - t0
        done += 1
        if t_attn >= budget_s:
            break
    nb = min(4, c.B)
    t0 = time.perf_counter()
    pr, lr, _ = oracle.accept_greedy_path(c.logits[:nb], c.parent[:nb], c.tok[:nb],
                                          c.n_nodes[:nb], c.root_tok[:nb])
    t_acc = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.tree_cache_reroot([], c.prefix_len[:nb], c.parent[:nb], c.n_nodes[:nb], pr, lr,
                             np.zeros(nb, dtype=bool))
    t_rr = time.perf_counter() - t0
    per_step = t_attn / done * len(pairs) + (t_acc + t_rr) / nb * c.B
    return {"value": per_step * 1e6, "unit": "us/step", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{done} of {len(pairs)} (sequence, KV head) attention blocks "
                      f"({t_attn:.1f} s) + accept/re-root of {nb} of {c.B} sequences, "
                      f"scaled to one full step",
            "host_cpus": len(os.sched_getaffinity(0))}


# ----------------------------------------------------------------------------
# workloads: each builds device inputs once and exposes step(i, marks)
# ----------------------------------------------------------------------------

class _Up:
    def __init__(self, dev):
        self.dev = dev

    def __call__(self, arr, bf16=False):
        import numpy as np
        import torch
        t = torch.from_numpy(np.ascontiguousarray(arr.view(np.int16) if bf16 else arr)).to(self.dev)
        return t.view(torch.bfloat16) if bf16 else t


class _VerifyBatch:
    """Device arrays of one verify batch: attention, accept and re-root."""

    def __init__(self, ta, up, c, kv, q):
        import numpy as np
        import torch
        dev = up.dev
        self.ta, self.torch, self.c, self.kv, self.q = ta, torch, c, kv, q
        # prefix_len, parent and n_nodes share one buffer so that a single
        # kernel restores all three after the re-root has rewritten them
        B, nm = c.B, c.n_max
        i32 = lambda x: up(np.ascontiguousarray(x, dtype=np.int32)).view(-1)  # noqa: E731
        self.meta0 = torch.cat([i32(c.prefix_len), i32(c.parent), i32(c.n_nodes)])
        self.meta = self.meta0.clone()
        self.P = self.meta[:B]
        self.par = self.meta[B:B + B * nm].view(B, nm)
        self.n = self.meta[B + B * nm:]
        self.tok, self.root_tok, self.logits = up(c.tok), up(c.root_tok), up(c.logits)
        self.keep = torch.zeros(c.B, dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(q)
        self.lse = torch.empty((c.B, c.Hq, c.n_max), dtype=torch.float32, device=dev)
        self.path = torch.empty((c.B, c.n_max), dtype=torch.int32, device=dev)
        self.plen = torch.empty((c.B,), dtype=torch.int32, device=dev)
        self.bonus = torch.empty((c.B,), dtype=torch.int32, device=dev)
        self.bytes = attn_bytes(c.prefix_len, c.n_nodes, c.n_nodes, c.Hq, c.Hkv, c.d)

    def phase(self, j, ws, opts, kv=None, q=None, logits=None):
        """Phase j of one step: 0 verify attention, 1 greedy accept + re-root
        (tree_accept_reroot) + restore."""
        ta = self.ta
        kv = self.kv if kv is None else kv
        if j == 0:
            ta.tree_attn_verify(self.q if q is None else q, kv, self.P, self.par, self.n,
                                self.c.scale, out=self.out, lse=self.lse, workspace=ws, **opts)
        else:
            ta.tree_accept_reroot(self.logits if logits is None else logits, self.tok,
                                  self.root_tok, [kv], self.P, self.par, self.n, self.keep,
                                  self.path, self.plen, self.bonus, workspace=ws)
            self.restore()

    def restore(self):
        # an elementwise kernel, not a device copy, so that it graph-captures
        # as a kernel node
        self.torch.add(self.meta0, 0, out=self.meta)

    def two_calls(self, kv=None, logits=None):
        """The same accept + re-root as accept_greedy_path then
        tree_cache_reroot (four launches), timed beside the step."""
        ta = self.ta
        kv = self.kv if kv is None else kv
        ta.accept_greedy_path(self.logits if logits is None else logits, self.par, self.tok,
                              self.n, self.root_tok, self.path, self.plen, self.bonus)
        ta.tree_cache_reroot([kv], self.P, self.par, self.n, self.path, self.plen, self.keep)
        self.restore()


class _Workload:
    def extras(self):
        """Calls timed beside the step (name -> fn(i, ws, opts)); none by default."""
        return {}

    def step(self, i, ws, marks, opts):
        for j in range(len(self.phases)):
            if marks is not None:
                marks[j].record()
            self.phase(i, j, ws, opts)
        if marks is not None:
            marks[len(self.phases)].record()


class ChainVerify(_Workload):
    phases = ("verify", "accept_reroot")

    def __init__(self, ta, up):
        from gen import config2_chain
        c = self.c = config2_chain()
        self.batch = _VerifyBatch(ta, up, c, ta.KVCache(up(c.k, True), up(c.v, True)),
                                  up(c.q, True))
        self._rope = None
        self._samp = None
        self.config = {"workload": "chain_verify", "batch": c.B, "Hq": c.Hq, "Hkv": c.Hkv,
                       "head_dim": c.d, "prefix": int(c.prefix_len[0]), "D": c.n_max - 1,
                       "rows_per_kv_head": c.G * c.n_max, "vocab": c.vocab,
                       "step": "verify + accept/re-root (+ restore of 3 tiny arrays)"}

    def phase(self, i, j, ws, opts):
        self.batch.phase(j, ws, opts)

    def extras(self):
        """RoPE at the tree positions and the KV append of the 16 nodes per
        sequence (tree_rope_append), and the verify call with RoPE fused in
        (tree_attn_verify_rope), timed beside the step: the workload's queries
        and tree keys stand in for un-rotated ones, and the rotated keys
        overwrite the tree rows (so these run after everything else)."""
        import torch
        bt, c = self.batch, self.c
        if self._rope is None:
            k_new = torch.stack([bt.kv.k[b, int(c.prefix_len[b]):int(c.prefix_len[b]) + c.n_max]
                                 for b in range(c.B)]).contiguous()
            v_new = torch.stack([bt.kv.v[b, int(c.prefix_len[b]):int(c.prefix_len[b]) + c.n_max]
                                 for b in range(c.B)]).contiguous()
            self._rope = (k_new, v_new, torch.empty_like(bt.q))
        k_new, v_new, q_out = self._rope

        def rope(i, ws, opts):
            bt.ta.tree_rope_append(bt.q, k_new, v_new, bt.kv, bt.P, bt.par, bt.n, q_out=q_out)

        if self._samp is None:
            # Sampling verification of the same trees at temperature 1: the
            # draft's logits are the target's plus seeded Gaussian noise
            # (sd 1), the uniforms seeded; outputs go to their own arrays.
            g = torch.Generator(device=bt.logits.device).manual_seed(4242)
            dft = (bt.logits.float() + torch.randn(bt.logits.shape, generator=g,
                                                   device=bt.logits.device)).to(bt.logits.dtype)
            u = torch.rand(bt.tok.shape, generator=g, device=bt.logits.device)
            ub = torch.rand(bt.tok.shape[0], generator=g, device=bt.logits.device)
            ws_s = torch.empty(bt.ta.accept_sampling_workspace_bytes(*bt.tok.shape),
                               dtype=torch.uint8, device=bt.logits.device)
            outs = (torch.empty_like(bt.path), torch.empty_like(bt.plen),
                    torch.empty_like(bt.bonus))
            self._samp = (dft, u, ub, ws_s, outs)
        dft, u, ub, ws_s, outs = self._samp

        def sampling(i, ws, opts):
            bt.ta.accept_sampling_path(bt.logits, dft, bt.par, bt.tok, bt.n, bt.root_tok, u, ub,
                                       1.0, *outs, workspace=ws_s)
        out_r = torch.empty_like(bt.q)
        lse_r = torch.empty((c.B, c.Hq, c.n_max), dtype=torch.float32, device=bt.q.device)

        def verify_rope(i, ws, opts):
            # the verify call with RoPE fused in (rotation on load, tree rows
            # staged and written by the attention kernel)
            bt.ta.tree_attn_verify_rope(bt.q, k_new, v_new, bt.kv, bt.P, bt.par, bt.n, c.scale,
                                        out=out_r, lse=lse_r, workspace=ws, **opts)
        return {"rope_append": rope, "accept_sampling": sampling, "verify_rope": verify_rope,
                "accept_then_reroot": lambda i, ws, opts: bt.two_calls()}

    def attn_bytes(self, i):
        return self.batch.bytes

    def check(self):
        if self.batch.plen.cpu().tolist() != self.c.planted["path_len"]:
            raise RuntimeError("accepted lengths differ from the planted ones")

    def cpu_baseline(self, budget):
        return cpu_verify_step(self.c, budget)


class PagedAlternating(_Workload):
    phases = ("verify", "accept_reroot")

    def __init__(self, ta, up):
        from gen import config5_paged
        c = self.c = config5_paged()
        m = self.m = c.planted["batch_size"]
        k, v = up(c.k, True), up(c.v, True)
        self.batches = []
        for s in range(2):
            sub = _subcase(c, slice(s * m, (s + 1) * m))
            kv = ta.KVCache(k, v, up(sub.block_table), T_cap=c.T_cap)
            self.batches.append(_VerifyBatch(ta, up, sub, kv, up(sub.q, True)))
        self.ran = set()
        self.config = {"workload": "paged_alternating", "batch": m, "resident_requests": c.B,
                       "Hq": c.Hq, "Hkv": c.Hkv, "head_dim": c.d, "prefix": "U[512,8192]",
                       "block_size": c.block_size, "k": c.n_max - 1, "vocab": c.vocab,
                       "step": "verify + accept/re-root of batch (step mod 2)"}

    def phase(self, i, j, ws, opts):
        self.ran.add(i % 2)
        self.batches[i % 2].phase(j, ws, opts)

    def extras(self):
        """accept_greedy_path then tree_cache_reroot (four launches) on the
        step's batch, timed beside the step."""
        return {"accept_then_reroot": lambda i, ws, opts: self.batches[i % 2].two_calls()}

    def attn_bytes(self, i):
        return self.batches[i % 2].bytes

    def check(self):
        for s, bt in enumerate(self.batches):
            if s not in self.ran:
                continue
            want = self.c.planted["path_len"][s * self.m:(s + 1) * self.m]
            if bt.plen.cpu().tolist() != want:
                raise RuntimeError(f"batch {s}: accepted lengths differ from the planted ones")

    def cpu_baseline(self, budget):
        return cpu_verify_step(self.batches[0].c, budget)


class TreeVerifyL70b(_Workload):
    """Rotates over COPIES sets of (K, V, Q, logits) so that nothing a step
    reads is left in the Infinity Cache by the previous steps."""
    phases = ("verify", "accept_reroot")
    COPIES = 16

    def __init__(self, ta, up):
        from gen import config3_tree
        c = self.c = config3_tree()
        k, v, q, lg = up(c.k, True), up(c.v, True), up(c.q, True), up(c.logits)
        self.kvs = [ta.KVCache(k.clone(), v.clone()) for _ in range(self.COPIES)]
        self.qs = [q.clone() for _ in range(self.COPIES)]
        self.lgs = [lg.clone() for _ in range(self.COPIES)]
        del k, v, q, lg
        self.batch = _VerifyBatch(ta, up, c, self.kvs[0], self.qs[0])
        self.config = {"workload": "tree_verify_l70b", "batch": c.B, "Hq": c.Hq, "Hkv": c.Hkv,
                       "head_dim": c.d, "prefix": int(c.prefix_len[0]), "tree_nodes": c.n_max,
                       "vocab": c.vocab, "kv_copies": self.COPIES,
                       "step": "verify + accept/re-root (+ restore of 3 tiny arrays)"}

    def phase(self, i, j, ws, opts):
        c = i % self.COPIES
        self.batch.phase(j, ws, opts, kv=self.kvs[c], q=self.qs[c], logits=self.lgs[c])

    def extras(self):
        """accept_greedy_path then tree_cache_reroot (four launches), timed
        beside the step."""
        def two(i, ws, opts):
            c = i % self.COPIES
            self.batch.two_calls(kv=self.kvs[c], logits=self.lgs[c])
        return {"accept_then_reroot": two}

    def attn_bytes(self, i):
        return self.batch.bytes

    def check(self):
        if self.batch.plen.cpu().tolist() != self.c.planted["path_len"]:
            raise RuntimeError("accepted lengths differ from the planted ones")

    def cpu_baseline(self, budget):
        return cpu_verify_step(self.c, budget)


class DraftExpand(_Workload):
    """One draft-side iteration over a 64-node draft tree, all on the device
    (SwiftSpec summary, Section 3.1.1 Algorithm 1).  Four expansion rounds:
    tree_expand_top_w appends the w = 8 best leaves (maximum-likelihood
    expansion over the 32000-way rows of the root and every node), then
    tree_attn_expand attends the new leaves over prefix + tree.  Then
    tree_token_walk along the target's verified tokens, tree_cache_reroot_draft
    (the walked path joins the prefix, the subtree under its last node moves
    forward with its KV rows, tokens and re-based weights) and
    tree_select_subtree of the bs = 8 nodes to send, on the re-rooted tree.
    The verified tokens are the root path of the grown tree's node at depth
    >= 2 with the largest subtree (so the re-root keeps a subtree), fixed once
    the first step has run.  The tree state (parents, tokens, weights, sizes,
    prefix length) is restored after the step by one elementwise kernel, so
    every step grows the same tree; the rows the re-root moved stay moved in
    that step's KV copy (a permutation of tree rows, which changes no later
    step's work).  Phases (HIP-graph mode): "expand" = the 4 attention calls,
    on the trees the rounds produce; "topw" = one restore + the 4 selections;
    "walk_reroot_select" = one copy of the grown tree's state, then the walk,
    the re-root and the selection.  With --eager the phases are not separated
    (the whole step is "expand")."""
    phases = ("expand", "topw", "walk_reroot_select")
    COPIES = 64
    BS = 8       # nodes sent to the target per iteration
    M_VER = 8    # room for the verified tokens

    def __init__(self, ta, up):
        import numpy as np
        import torch
        from gen import config4_expand
        e = self.e = config4_expand()
        self.ta, self.torch = ta, torch
        k, v = up(e.k, True), up(e.v, True)
        self.kvs = [ta.KVCache(k.clone(), v.clone()) for _ in range(self.COPIES)]
        del k, v
        nm = e.n_max
        # draft distributions: row 0 after the root, row 1 + i after node i (the
        # new leaves' rows are drawn up front; a round only reads existing nodes)
        lg = np.zeros((1, nm + 1, e.vocab), dtype=np.float32)
        lg[0, 0] = e.logits_root
        lg[0, 1:e.n0 + 1] = e.logits0
        for r in range(e.rounds):
            lg[0, e.n0 + 1 + r * e.w:e.n0 + 1 + (r + 1) * e.w] = e.logits_new[r]
        self.logits = up(lg)
        # tree state in one int32 buffer (parent, tok, cum bits, n, prefix
        # length) so that one kernel restores it
        par = np.full(nm, -1, dtype=np.int32)
        tok = np.full(nm, -1, dtype=np.int32)
        cum = np.full(nm, -np.inf, dtype=np.float32)
        par[:e.n0], tok[:e.n0] = e.parent0, e.tok0
        cum[:e.n0] = self._cum0(e)
        meta = np.concatenate([par, tok, cum.view(np.int32), np.array([e.n0, e.P], np.int32)])
        self.meta0 = up(meta)
        self.meta = self.meta0.clone()
        self.meta_grown = None
        self.par = self.meta[0:nm].view(1, nm)
        self.tok = self.meta[nm:2 * nm].view(1, nm)
        self.cum = self.meta[2 * nm:3 * nm].view(torch.float32).view(1, nm)
        self.n = self.meta[3 * nm:3 * nm + 1]
        self.P = self.meta[3 * nm + 1:3 * nm + 2]
        self.qs = [up(e.q_new[r], True) for r in range(e.rounds)]
        self.outs = [torch.empty_like(q) for q in self.qs]
        self.lses = [torch.empty((1, e.Hq, e.w), dtype=torch.float32, device=up.dev)
                     for _ in self.qs]
        self.snaps = None   # per-round (parent, n) after its selection, for the expand phase
        i32 = dict(dtype=torch.int32, device=up.dev)
        self.verified = torch.zeros((1, self.M_VER), **i32)
        self.vlen = torch.zeros((1,), **i32)
        self.walk_out = (torch.empty((1, nm), **i32), torch.empty((1,), **i32),
                         torch.empty((1,), dtype=torch.uint8, device=up.dev))
        self.sel_out = (torch.empty((1, self.BS), **i32), torch.empty((1, self.BS), **i32),
                        torch.empty((1, self.BS), **i32), torch.empty((1,), **i32))
        self.topw_ws = ta.Workspace(up.dev)
        b = [attn_bytes([e.P], [e.n0 + e.w * (r + 1)], [e.w], e.Hq, e.Hkv, e.d)
             for r in range(e.rounds)]
        self.bytes = {key: sum(x[key] for x in b) for key in b[0]}
        self.config = {"workload": "draft_expand", "batch": 1, "Hq": e.Hq, "Hkv": e.Hkv,
                       "head_dim": e.d, "prefix": e.P, "tree_nodes": f"{e.n0}->{e.n_max}",
                       "w": e.w, "rounds": e.rounds, "vocab": e.vocab, "kv_copies": self.COPIES,
                       "bs": self.BS,
                       "step": "4 rounds of top-w selection + expansion attention, then the walk "
                               "along the verified tokens, the re-root (KV, tokens, weights) "
                               "and the size-bs subtree selection (+ tree restore)"}

    @staticmethod
    def _cum0(e):
        """Cumulative scores of the initial tree (fp32 of the fp64 sums), the
        caller-kept state the selection extends."""
        import numpy as np
        lsm_root = e.logits_root.astype(np.float64)
        lsm_root = lsm_root - (lsm_root.max() + np.log(np.exp(lsm_root - lsm_root.max()).sum()))
        cum = np.zeros(e.n0, dtype=np.float64)
        for i in range(e.n0):
            p = int(e.parent0[i])
            if p < 0:
                cum[i] = lsm_root[int(e.tok0[i])]
            else:
                row = e.logits0[p].astype(np.float64)
                lsm = row - (row.max() + np.log(np.exp(row - row.max()).sum()))
                cum[i] = cum[p] + lsm[int(e.tok0[i])]
        return cum.astype(np.float32)

    def _round(self, r, kv, ws, opts):
        self.ta.tree_expand_top_w(self.logits, self.par, self.tok, self.cum, self.n, self.e.w,
                                  workspace=self.topw_ws)
        self.ta.tree_attn_expand(self.qs[r], kv, self.P, self.par, self.n, self.e.scale,
                                 out=self.outs[r], lse=self.lses[r], workspace=ws, **opts)

    def _restore(self, src=None):
        self.torch.add(self.meta0 if src is None else src, 0, out=self.meta)

    def _draft_side(self, kv):
        path, plen, keep = self.walk_out
        self.ta.tree_token_walk(self.par, self.tok, self.n, self.verified, self.vlen, *self.walk_out)
        self.ta.tree_cache_reroot_draft([kv], self.P, self.par, self.n, path, plen, keep,
                                        self.tok, self.cum)
        self.ta.tree_select_subtree(self.cum, self.par, self.tok, self.n, self.BS, *self.sel_out)

    def step(self, i, ws, marks, opts):
        kv = self.kvs[i % self.COPIES]
        if marks is not None:
            marks[0].record()
        for r in range(self.e.rounds):
            self._round(r, kv, ws, opts)
        self._draft_side(kv)
        self._restore()
        if marks is not None:
            marks[1].record()
            marks[2].record()

    def _snapshots(self, ws, opts):
        """Each round's tree after its selection, and the grown tree's whole
        state (from one eager pass)."""
        torch = self.torch
        self._restore()
        snaps = []
        for r in range(self.e.rounds):
            self.ta.tree_expand_top_w(self.logits, self.par, self.tok, self.cum, self.n,
                                      self.e.w, workspace=self.topw_ws)
            snaps.append((self.par.clone(), self.n.clone()))
        self.meta_grown = self.meta.clone()
        self._restore()
        torch.cuda.synchronize()
        return snaps

    def phase(self, i, j, ws, opts):
        if self.snaps is None:
            raise RuntimeError("draft_expand phases need check() (after warm-up) first")
        kv = self.kvs[i % self.COPIES]
        if j == 0:
            for r, (par, n) in enumerate(self.snaps):
                self.ta.tree_attn_expand(self.qs[r], kv, self.P, par, n, self.e.scale,
                                         out=self.outs[r], lse=self.lses[r], workspace=ws, **opts)
        elif j == 1:
            self._restore()
            for r in range(self.e.rounds):
                self.ta.tree_expand_top_w(self.logits, self.par, self.tok, self.cum, self.n,
                                          self.e.w, workspace=self.topw_ws)
        else:
            self._restore(self.meta_grown)
            self._draft_side(kv)

    def attn_bytes(self, i):
        return self.bytes

    def check(self):
        torch = self.torch
        for o, l in zip(self.outs, self.lses):
            if not (torch.isfinite(o.float()).all() and torch.isfinite(l).all()):
                raise RuntimeError("non-finite expansion output")
        if self.snaps is None:
            self.snaps = self._snapshots(None, None)
            self._set_verified()
        e = self.e
        if int(self.snaps[-1][1].item()) != e.n0 + e.w * e.rounds:
            raise RuntimeError("the expansion rounds did not grow the tree to its full size")

    def _set_verified(self):
        """The target's verified tokens: the root path of the grown tree's
        node at depth >= 2 with the largest subtree (lowest index on ties), so
        that the walk keeps that subtree.  Plain loops over the parent array."""
        nm = self.e.n_max
        g = self.meta_grown.cpu().numpy()
        par, tok, n = g[0:nm], g[nm:2 * nm], int(g[3 * nm])
        depth, size = [0] * n, [1] * n
        for i in range(n):
            depth[i] = 1 + (depth[par[i]] if par[i] >= 0 else 0)
        for i in range(n - 1, -1, -1):
            if par[i] >= 0:
                size[par[i]] += size[i]
        cand = [i for i in range(n) if 2 <= depth[i] <= self.M_VER]
        x = max(cand, key=lambda i: (size[i], -i))
        ver = []
        while x >= 0:
            ver.append(int(tok[x]))
            x = int(par[x])
        ver.reverse()
        self.verified.zero_()
        self.verified[0, :len(ver)] = self.torch.tensor(ver, dtype=self.torch.int32)
        self.vlen.fill_(len(ver))
        self.torch.cuda.synchronize()

    def cpu_baseline(self, budget):
        """The oracle for one step: per round, top-w selection (fp64) and the
        expansion attention of the new leaves."""
        import numpy as np

        import oracle
        e = self.e
        par = np.full(e.n_max, -1, dtype=np.int32)
        tok = np.zeros(e.n_max, dtype=np.int32)
        par[:e.n0], tok[:e.n0] = e.parent0, e.tok0
        rows = e.logits0.copy()
        n = e.n0
        t0 = time.perf_counter()
        for r in range(e.rounds):
            cum = oracle.cumulative_scores(par, tok, e.logits_root, rows, n)
            p, t, _ = oracle.select_top_w(par, tok, cum, e.logits_root, rows, n, e.w)
            par[n:n + e.w], tok[n:n + e.w] = p, t
            n += e.w
            oc = self.c_like()
            oc.parent, oc.n_nodes = par[None].copy(), np.array([n])
            oracle.expand(oc, e.q_new[r], e.w)
            rows = np.concatenate([rows, e.logits_new[r]])
        ver = self.verified[0, :int(self.vlen.item())].cpu().numpy()
        path, keep = oracle.token_walk(par, tok, n, ver)
        cum = oracle.cumulative_scores(par, tok, e.logits_root, rows[:n], n)
        pth = np.full((1, e.n_max), -1, dtype=np.int32)
        pth[0, :len(path)] = path
        _, _, par2, n2 = oracle.tree_cache_reroot([(e.k, e.v)], np.array([e.P]), par[None],
                                                  np.array([n]), pth, np.array([len(path)]),
                                                  np.array([keep]))
        tok2, cum2 = oracle.reroot_node_arrays(par, n, path, len(path), keep, tok,
                                               cum.astype(np.float32))
        oracle.select_subtree(par2[0], tok2, cum2, int(n2[0]), self.BS)
        dt = time.perf_counter() - t0
        return {"value": dt * 1e6, "unit": "us/step", "cores": _blas_threads(), "kind": "oracle",
                "sample": "all 4 rounds of one step (top-w selection + expansion attention) "
                          "and the walk, re-root and subtree selection",
                "host_cpus": len(os.sched_getaffinity(0))}

    def c_like(self):
        import numpy as np

        class _C:
            pass
        e, oc = self.e, _C()
        oc.B, oc.Hq, oc.d, oc.G, oc.scale, oc.dtype = 1, e.Hq, e.d, e.Hq // e.Hkv, e.scale, "bf16"
        oc.prefix_len = np.array([e.P])
        oc.k, oc.v, oc.block_table, oc.block_size = e.k, e.v, None, 0
        return oc


RUNNERS = {"chain_verify": ChainVerify, "paged_alternating": PagedAlternating,
           "tree_verify_l70b": TreeVerifyL70b, "draft_expand": DraftExpand}


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of known size (reference for PMC byte counters)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) / 1e3)
    return nbytes, sorted(t)[len(t) // 2]


def measure(ta, workload, a, dev):
    """Builds one workload, runs the warm-up, times a.steps steps and each
    phase; returns the JSON fields (no CPU baseline) and the workload."""
    import numpy as np
    import torch

    t0 = time.time()
    w = RUNNERS[workload](ta, _Up(dev))
    _log(f"generated {workload} inputs in {time.time() - t0:.1f} s")
    ws = ta.Workspace(dev)
    opts = {"kernel": a.kernel, "chunk_tokens": a.chunk}
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    nph = len(w.phases)
    for i in range(a.warmup):
        w.step(i, ws, None, opts)
    torch.cuda.synchronize()
    w.check()   # correctness guard for the timed configuration
    steps = range(a.warmup, a.warmup + a.steps)
    extra_ms = {}  # calls timed beside the step (graph mode only)

    if a.eager:
        # one Python call per entry point: host launch cost is inside the steps
        marks = [[ev() for _ in range(nph + 1)] for _ in range(a.steps)]
        start, stop = ev(), ev()
        torch.cuda.synchronize()
        start.record()
        for k, i in enumerate(steps):
            w.step(i, ws, marks[k], opts)
        stop.record()
        torch.cuda.synchronize()
        ms_per_step = start.elapsed_time(stop) / a.steps
        phase_ms = [[m[j].elapsed_time(m[j + 1]) for m in marks] for j in range(nph)]
        call_ms = phase_ms[0]
    else:
        # The K steps are captured once in a HIP graph (every size the kernels
        # need is in device memory) and replayed: the timed region is the
        # device's work, not the Python binding's.  Each phase is timed the
        # same way, as a graph of its K calls replayed PHASE_REPS times.
        def capture(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            return g

        def time_single_calls(fn_of_i, lead_graph, est_ms):
            """Durations (ms) of at least MIN_TIMED_CALLS single calls, each
            issued from Python between two events.  At least 10 ms of the same
            calls (replays of the phase's graph) are queued first, so the host
            has issued every timed call before the device reaches it: the
            intervals hold device time (plus the ~1 us of the events), not
            host launch latency, and the clocks are those of sustained work.
            (One-call graphs would add ~8 us of graph launch per call; a
            device-side spin as the lead lowers the clocks of the work after
            it.)"""
            n = max(MIN_TIMED_CALLS, len(steps))
            marks = [(ev(), ev()) for _ in range(n)]
            lead = max(1, int(np.ceil(10.0 / max(est_ms * len(steps), 1e-3))))
            torch.cuda.synchronize()
            for _ in range(lead):
                lead_graph.replay()
            for c, (e0, e1) in enumerate(marks):
                e0.record()
                fn_of_i(steps[c % len(steps)])
                e1.record()
            torch.cuda.synchronize()
            return [e0.elapsed_time(e1) for e0, e1 in marks]

        g_steps = capture(lambda: [w.step(i, ws, None, opts) for i in steps])
        g_steps.replay()
        torch.cuda.synchronize()
        w.check()
        start, stop = ev(), ev()
        torch.cuda.synchronize()
        start.record()
        g_steps.replay()
        stop.record()
        torch.cuda.synchronize()
        ms_per_step = start.elapsed_time(stop) / a.steps
        w.check()
        phase_ms = []
        for j in range(nph):
            g = capture(lambda: [w.phase(i, j, ws, opts) for i in steps])
            g.replay()
            per_call = []
            for _ in range(PHASE_REPS):
                e0, e1 = ev(), ev()
                torch.cuda.synchronize()
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                per_call.append(e0.elapsed_time(e1) / a.steps)
            phase_ms.append(per_call)
            if j == 0:
                call_ms = time_single_calls(lambda i: w.phase(i, 0, ws, opts), g,
                                            float(np.mean(per_call)))
            del g
        # Calls timed beside the step (not part of it), the same way, last:
        # they may rewrite the inputs.
        for name, fn in w.extras().items():
            g = capture(lambda: [fn(i, ws, opts) for i in steps])
            g.replay()
            per_call = []
            for _ in range(PHASE_REPS):
                e0, e1 = ev(), ev()
                torch.cuda.synchronize()
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                per_call.append(e0.elapsed_time(e1) / a.steps)
            extra_ms[name] = per_call
            del g
        del g_steps
    attn_ms = phase_ms[0]
    med = lambda x: float(np.median(x))  # noqa: E731
    pct = lambda x, p: float(np.percentile(x, p))  # noqa: E731

    steps_bytes = [w.attn_bytes(i) for i in steps]
    attn_s = float(np.mean(attn_ms)) / 1e3          # mean duration of one attention call
    achieved = float(np.mean([b["total"] for b in steps_bytes])) / attn_s / 1e9
    kv_gbps = float(np.mean([b["kv"] for b in steps_bytes])) / attn_s / 1e9
    call = "tree_attn_verify" if w.phases[0] == "verify" else "4 tree_attn_expand calls"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": read_traffic(workload),
                "kernel": f"{call} (attention kernel + split-combine kernel when split)",
                "algorithmic_bytes_per_launch": int(np.mean([b["total"] for b in steps_bytes])),
                "avg_launch_us": round(attn_s * 1e6, 2)}

    _, copy_s = copy_calibration(1 << 30, 3)
    res = {
        "metric": METRIC,
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": w.config,
        "launch": "eager (one Python call per entry point)" if a.eager else
                  "hip_graph (the K steps captured once, replayed)",
        "kv_read_GBps": round(kv_gbps, 1),
        "pct_hbm_peak": round(100 * kv_gbps / HBM_PEAK_GBPS, 2),
        f"{w.phases[0]}_us": {"median": round(med(call_ms) * 1e3, 2),
                              "p10": round(pct(call_ms, 10) * 1e3, 2),
                              "p90": round(pct(call_ms, 90) * 1e3, 2),
                              "calls": len(call_ms),
                              "mean_in_step_graph": round(float(np.mean(attn_ms)) * 1e3, 2)},
    }
    for j in range(1, nph):
        res[f"{w.phases[j]}_us"] = round(med(phase_ms[j]) * 1e3, 2)
    for name, ms in extra_ms.items():
        res[f"{name}_us"] = round(med(ms) * 1e3, 2)
    if extra_ms:
        res["beside_step"] = sorted(f"{name}_us" for name in extra_ms)
    res["device_copy_GBps"] = round(2 * (1 << 30) / copy_s / 1e9, 1)
    res["roofline"] = roofline
    return res, w


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=WORKLOADS, default=None,
                    help="the workload of the line (default chain_verify, with the other "
                         "workloads timed beside it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="without --workload: skip timing the other workloads beside chain_verify")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a 1 GiB device copy (for PMC byte-counter scaling)")
    ap.add_argument("--kernel", type=int, default=0,
                    help="0 auto, 1 generic, 2 MFMA (register prefetch), 3 MFMA (LDS-DMA ring)")
    ap.add_argument("--chunk", type=int, default=0, help="KV positions per split (0 = auto)")
    ap.add_argument("--eager", action="store_true",
                    help="issue every call from Python inside the timed region (no HIP graph)")
    a = ap.parse_args(argv)
    others_too = a.workload is None and not a.no_others
    if a.workload is None:
        a.workload = "chain_verify"

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the verify kernel shards by (sequence, KV head) with no exchange; "
              "run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_masked_verify_attn_amd as ta
    from tree_masked_verify_attn_amd import build as tb

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(tb.LIB):
        tb.build()
    ta.load_library()

    if a.copy_calib:
        nbytes, sec = copy_calibration()
        print(json.dumps({"copy_bytes": nbytes, "copy_s": sec,
                          "copy_GBps": 2 * nbytes / sec / 1e9}), flush=True)
        return

    dev = torch.device("cuda:0")
    res, w = measure(ta, a.workload, a, dev)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = w.cpu_baseline(a.cpu_budget)
        # the same oracle on one core (BLAS limited to one thread)
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:  # pragma: no cover
            threadpool_limits = None
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                one = w.cpu_baseline(a.cpu_budget)
            res["cpu_baseline_1core"] = one
    if others_too:
        # The other single-GPU workloads, timed the same way in this process
        # (not part of value): their step time, the attention call and its
        # HBM fraction.
        del w
        torch.cuda.empty_cache()
        others = {}
        for name in OTHER_WORKLOADS:
            r, w2 = measure(ta, name, a, dev)
            first = f"{r_phase0(r)}_us"
            others[name] = {"value": r["value"], "unit": r["unit"], first: r[first],
                            **{k: v for k, v in r.items() if k.endswith("_us") and k != first},
                            "roofline": {k: r["roofline"][k] for k in
                                         ("achieved", "frac", "traffic", "avg_launch_us")},
                            "config": r["config"]}
            del w2, r
            torch.cuda.empty_cache()
        res["other_workloads"] = others
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
