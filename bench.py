"""Benchmark of the tree-verify hot path on one MI355X.

One step = one pass of the whole path over one batch of the chain-verify
workload (batch 16, Hq=64, Hkv=8, d=128, bf16, prefix 32768 per sequence,
D = 15 chain drafts -> 128 query rows per KV head):

    tree_attn_verify -> accept_greedy_path -> tree_cache_reroot

followed by restoring the three tiny per-sequence arrays the re-root rewrote
(prefix_len, parent, n_nodes), so that every step sees the same input.  All
inputs are resident in HBM before timing starts.  The KV cache is 2.15 GB per
call, far beyond the 256 MB Infinity Cache, so every step reads it cold.

Prints one JSON line (metric, value = microseconds per step, roofline of the
verify kernel, CPU-oracle baseline on a bounded sample).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --copy-calib     # plain device copy of known size (PMC scaling)
"""
from __future__ import annotations

import argparse
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_attn_chain_verify_traffic.txt")


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the attention kernel sources (ties PMC traffic to a kernel version)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_masked_verify_attn_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.startswith("attn_") or f in ("ta_device.h", "ta_internal.h", "api.cpp"):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per verify launch from the committed PMC summary, if it still
    describes the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(c) -> dict:
    """Bytes the method must move per verify call: K and V once per (sequence,
    KV head) over P + n positions, Q in, O out, LSE out."""
    eb = 2 if c.dtype == "bf16" else 4
    kv = 0
    for b in range(c.B):
        T = int(c.prefix_len[b] + c.n_nodes[b])
        kv += 2 * T * c.Hkv * c.d * eb
    rows = int(c.n_nodes.sum())
    q = rows * c.Hq * c.d * eb
    return {"kv": kv, "q": q, "o": q, "lse": rows * c.Hq * 4,
            "total": kv + 2 * q + rows * c.Hq * 4}


def cpu_baseline(c, budget_s: float = 12.0) -> dict:
    """Time the oracle (as it stands) on a bounded sample of the same step and
    scale to microseconds per full step."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    pairs = [(b, hk) for b in range(c.B) for hk in range(c.Hkv)]
    rng = np.random.default_rng(0)
    order = rng.permutation(len(pairs))
    t_attn, done = 0.0, 0
    for j in order:
        b, hk = pairs[j]
        heads = list(range(hk * c.G, (hk + 1) * c.G))
        t0 = time.perf_counter()
        oracle.verify(c, batches=[b], heads=heads)
        t_attn += time.perf_counter() - t0
        done += 1
        if t_attn >= budget_s:
            break
    t0 = time.perf_counter()
    nb = min(4, c.B)
    pr, lr, br = oracle.accept_greedy_path(c.logits[:nb], c.parent[:nb], c.tok[:nb],
                                           c.n_nodes[:nb], c.root_tok[:nb])
    t_acc = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.tree_cache_reroot([], c.prefix_len[:nb], c.parent[:nb], c.n_nodes[:nb], pr, lr,
                             np.zeros(nb, dtype=bool))
    t_rr = time.perf_counter() - t0
    per_step = t_attn / done * len(pairs) + (t_acc + t_rr) / nb * c.B
    return {"value": per_step * 1e6, "unit": "us/step", "cores": int(blas), "kind": "oracle",
            "sample": f"{done} of {len(pairs)} (sequence, KV head) attention blocks "
                      f"({t_attn:.1f} s) + accept/re-root of {nb} of {c.B} sequences, "
                      f"scaled to one full step",
            "host_cpus": len(os.sched_getaffinity(0))}


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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a 1 GiB device copy (for PMC byte-counter scaling)")
    ap.add_argument("--kernel", type=int, default=0,
                    help="0 auto, 1 generic, 2 MFMA (register prefetch), 3 MFMA (LDS-DMA ring)")
    ap.add_argument("--chunk", type=int, default=0, help="KV positions per split (0 = auto)")
    a = ap.parse_args(argv)

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the verify kernel shards by (sequence, KV head) with no exchange; "
              "run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tree_masked_verify_attn_amd as ta
    from gen import config2_chain
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
    t0 = time.time()
    c = config2_chain()
    _log(f"generated chain-verify inputs in {time.time() - t0:.1f} s")

    def up(arr, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(arr.view(np.int16) if bf16 else arr)).to(dev)
        return t.view(torch.bfloat16) if bf16 else t

    q, k, v = up(c.q, True), up(c.k, True), up(c.v, True)
    P0, par0, n0 = up(c.prefix_len), up(c.parent), up(c.n_nodes)
    P, par, n = P0.clone(), par0.clone(), n0.clone()
    tok, root_tok, logits = up(c.tok), up(c.root_tok), up(c.logits)
    keep = torch.zeros(c.B, dtype=torch.uint8, device=dev)
    kv = ta.KVCache(k, v)
    out = torch.empty_like(q)
    lse = torch.empty((c.B, c.Hq, c.n_max), dtype=torch.float32, device=dev)
    path = torch.empty((c.B, c.n_max), dtype=torch.int32, device=dev)
    plen = torch.empty((c.B,), dtype=torch.int32, device=dev)
    bonus = torch.empty((c.B,), dtype=torch.int32, device=dev)
    ws = ta.Workspace(dev)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(marks=None):
        if marks is not None:
            marks[0].record()
        ta.tree_attn_verify(q, kv, P, par, n, c.scale, out=out, lse=lse, workspace=ws,
                            kernel=a.kernel, chunk_tokens=a.chunk)
        if marks is not None:
            marks[1].record()
        ta.accept_greedy_path(logits, par, tok, n, root_tok, path, plen, bonus)
        if marks is not None:
            marks[2].record()
        ta.tree_cache_reroot([kv], P, par, n, path, plen, keep)
        if marks is not None:
            marks[3].record()
        P.copy_(P0)
        par.copy_(par0)
        n.copy_(n0)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # correctness guard for the timed configuration: accepted lengths = planted
    if plen.cpu().tolist() != c.planted["path_len"]:
        raise RuntimeError("accepted lengths differ from the planted ones")

    marks = [[ev() for _ in range(4)] for _ in range(a.steps)]
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    start.record()
    for i in range(a.steps):
        step(marks[i])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / a.steps
    verify_ms = [m[0].elapsed_time(m[1]) for m in marks]
    accept_ms = [m[1].elapsed_time(m[2]) for m in marks]
    reroot_ms = [m[2].elapsed_time(m[3]) for m in marks]
    med = lambda x: float(np.median(x))  # noqa: E731
    pct = lambda x, p: float(np.percentile(x, p))  # noqa: E731

    alg = algorithmic_bytes(c)
    v_avg_s = float(np.mean(verify_ms)) / 1e3
    achieved = alg["total"] / v_avg_s / 1e9
    traffic = read_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic,
                "kernel": "tree_attn_verify call = attention kernel + split-combine kernel",
                "algorithmic_bytes_per_launch": alg["total"],
                "avg_launch_us": round(v_avg_s * 1e6, 2)}

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
        "config": {"workload": "chain_verify", "batch": c.B, "Hq": c.Hq, "Hkv": c.Hkv,
                   "head_dim": c.d, "prefix": int(c.prefix_len[0]), "D": c.n_max - 1,
                   "rows_per_kv_head": c.G * c.n_max, "vocab": c.vocab,
                   "step": "verify + accept + re-root (+ restore of 3 tiny arrays)"},
        "kv_read_GBps": round(alg["kv"] / v_avg_s / 1e9, 1),
        "pct_hbm_peak": round(100 * alg["kv"] / v_avg_s / 1e9 / HBM_PEAK_GBPS, 2),
        "verify_us": {"median": round(med(verify_ms) * 1e3, 2), "p10": round(pct(verify_ms, 10) * 1e3, 2),
                      "p90": round(pct(verify_ms, 90) * 1e3, 2)},
        "accept_us": round(med(accept_ms) * 1e3, 2),
        "reroot_us": round(med(reroot_ms) * 1e3, 2),
        "device_copy_GBps": round(2 * (1 << 30) / copy_s / 1e9, 1),
        "roofline": roofline,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(c, a.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
