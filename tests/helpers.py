"""Shared test helpers: upload seeded cases to the GPU, compare against the
oracle with the stated tolerances."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Float parity bars (against the float64 oracle):
#   fp32: |x - ref| <= 1e-5 * |ref| + 1e-5 * max|ref| over the (sequence, head) block
#   bf16: |x - ref| <= 1e-2 * |ref| + 2e-2
FP32_RTOL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def ensure_built():
    import tree_masked_verify_attn_amd as ta
    from tree_masked_verify_attn_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    return ta.load_library()


def dev_tensor(arr, dtype_name=None, device="cuda"):
    """numpy -> device tensor; uint16 arrays with dtype 'bf16' become bfloat16."""
    import torch
    if dtype_name == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def to_f64(t):
    import torch
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


class DevCase:
    """Device copies of a gen.Case's arrays plus a KVCache."""

    def __init__(self, case, device="cuda"):
        import tree_masked_verify_attn_amd as ta
        self.case = case
        dt = case.dtype
        self.q = dev_tensor(case.q, dt, device)
        self.k = dev_tensor(case.k, dt, device)
        self.v = dev_tensor(case.v, dt, device)
        self.prefix_len = dev_tensor(case.prefix_len.astype(np.int32), device=device)
        self.parent = dev_tensor(case.parent.astype(np.int32), device=device)
        self.n_nodes = dev_tensor(case.n_nodes.astype(np.int32), device=device)
        self.block_table = (dev_tensor(case.block_table.astype(np.int32), device=device)
                            if case.block_table is not None else None)
        self.kv = ta.KVCache(self.k, self.v, self.block_table,
                             T_cap=case.T_cap if case.block_table is not None else None)
        if case.tok is not None:
            self.tok = dev_tensor(case.tok.astype(np.int32), device=device)
            self.root_tok = dev_tensor(case.root_tok.astype(np.int32), device=device)
        if case.logits is not None:
            self.logits = dev_tensor(case.logits, device=device)


def assert_attn_close(O, L, O_ref, L_ref, dtype, rows_mask=None, what=""):
    """Elementwise bars; rows_mask [B][n_q] selects rows that are outputs."""
    O_ref = np.asarray(O_ref)
    L_ref = np.asarray(L_ref)
    B, n_q, Hq, d = O_ref.shape
    if rows_mask is None:
        rows_mask = ~np.isnan(O_ref[:, :, 0, 0])
    worst = 0.0
    for b in range(B):
        rows = np.nonzero(rows_mask[b])[0]
        if rows.size == 0:
            continue
        for h in range(Hq):
            o, r = O[b, rows, h], O_ref[b, rows, h]
            l, lr = L[b, h, rows], L_ref[b, h, rows]
            if dtype == "f32":
                atol_o = FP32_RTOL * np.abs(r).max()
                atol_l = FP32_RTOL * np.abs(lr).max()
                bound_o = atol_o + FP32_RTOL * np.abs(r)
                bound_l = atol_l + FP32_RTOL * np.abs(lr)
            else:
                bound_o = BF16_ATOL + BF16_RTOL * np.abs(r)
                bound_l = BF16_ATOL + BF16_RTOL * np.abs(lr)
            eo = np.abs(o - r)
            el = np.abs(l - lr)
            if not (np.all(eo <= bound_o) and np.all(el <= bound_l)):
                i = np.unravel_index(np.argmax(eo - bound_o), eo.shape)
                raise AssertionError(
                    f"{what} b={b} h={h}: max|dO|={eo.max():.3e} (bound at worst "
                    f"{bound_o[i]:.3e}), max|dLSE|={el.max():.3e}, any NaN="
                    f"{np.isnan(o).any() or np.isnan(l).any()}")
            worst = max(worst, float((eo / bound_o).max()), float((el / bound_l).max()))
    return worst


# ----------------------------------------------------------------------------
# Closed form of attention on the counting inputs (gen.structured): with zero
# queries every visible score is 0, so a row's LSE is ln(number of visible
# positions) = ln(P + depth(node)) and its output is the mean of the visible
# value rows (SwiftSpec summary, Section 3.1.3 Figure 3: prefix + ancestors +
# self; the zero-query closed form pinned in tests/test_oracle_attention.py).
# ----------------------------------------------------------------------------

def counting_expected(case, n_q, q_nodes_of):
    """Exact (float64) O [B][n_q][Hq][d] and LSE [B][Hq][n_q] of ``case`` built
    by ``gen.structured.counting_inputs`` (or a batch slice of one, with its
    ``planted["id_codes"]`` sliced alike); ``q_nodes_of(n)`` lists the node of
    each of the n_q query rows (verify: range(n_max); expand: n - w + r).
    Rows without a node are NaN."""
    import oracle
    from gen.structured import TILE, TREE_CODES, n_prefix_channels
    B, Hq, d = case.B, case.Hq, case.d
    G, Hkv = case.G, case.Hkv
    npc = n_prefix_channels(d)
    O = np.full((B, n_q, Hq, d), np.nan)
    L = np.full((B, Hq, n_q), np.nan)
    ids = np.repeat(np.asarray(case.planted["id_codes"], float), G, axis=1)   # [B][Hq]
    for b in range(B):
        P, n = int(case.prefix_len[b]), int(case.n_nodes[b])
        pref = np.bincount((np.arange(P) // TILE) % npc, minlength=npc).astype(float)
        for r, i in enumerate(q_nodes_of(n)):
            if not 0 <= i < n:
                continue
            vis = [int(x) for x in oracle.tree.visible_tree_columns(case.parent[b], i)]
            cnt = P + len(vis)
            tree = np.bincount(np.array(vis) % TREE_CODES, minlength=TREE_CODES).astype(float)
            row = np.r_[pref, tree, 0.0] / cnt
            O[b, r] = row[None, :]
            O[b, r, :, d - 1] = ids[b]
            L[b, :, r] = np.log(cnt)
    return O, L


def assert_counting_exact(O, L, O_x, L_x, what=""):
    """Bars for the counting inputs, from the arithmetic the kernels do on
    them: every probability is exactly 1 and every value an integer, so the
    fp32 sums are exact integers; LSE = (0 + log2 l) * ln 2 is within a few
    float32 ulp of ln l (hardware log2 ~1 ulp, the product 0.5 ulp); the
    output is count * (1/l) (two fp32 roundings) rounded once to bf16
    (half a bf16 ulp, at most 2^-8 relative).  A split row's partial sums
    are kept in fp16 for the combine (at most 2^-11 relative; the MFMA
    kernels), so the bar is 2^-8 + 2^-11 plus 2^-18 for the cross terms and
    the fp32 roundings.  Zero channels must be exactly zero and the identity
    channel exactly its integer code (within 2^-11 of an integer that bf16
    holds exactly, the output rounds to it)."""
    rows = ~np.isnan(O_x[..., 0, 0])
    Lr = np.transpose(L, (0, 2, 1))[rows]            # [rows][Hq]
    Lx = np.transpose(L_x, (0, 2, 1))[rows]
    ulp = np.spacing(np.abs(Lx).astype(np.float32)).astype(np.float64)
    errL = np.abs(Lr - Lx) / ulp
    if not np.all(errL <= 4.0):
        i = np.unravel_index(np.argmax(errL), errL.shape)
        raise AssertionError(f"{what}: LSE off by {errL[i]:.1f} fp32 ulp at row {i} "
                             f"(got {Lr[i]!r}, expected {Lx[i]!r})")
    Og, Ox = O[rows], O_x[rows]
    bound = (2.0 ** -8 + 2.0 ** -11 + 2.0 ** -18) * np.abs(Ox)
    bad = np.abs(Og - Ox) > bound
    if bad.any():
        i = np.unravel_index(np.argmax(np.abs(Og - Ox) - bound), Og.shape)
        raise AssertionError(f"{what}: output channel off at (row, head, channel) {i}: "
                             f"got {Og[i]!r}, expected {Ox[i]!r}; {int(bad.sum())} bad values")
    return float(errL.max())


def assert_lse_tight(L, L_ref, bound, what=""):
    """|LSE - LSE_ref| <= bound on every output row (NaN rows of the
    reference are skipped)."""
    ok = ~np.isnan(L_ref)
    err = np.abs(L[ok] - L_ref[ok])
    if not np.all(err <= bound):
        raise AssertionError(f"{what}: max |dLSE| = {np.nanmax(err):.3e} > {bound:.1e} "
                             f"({int((err > bound).sum())} rows)")
    return float(err.max()) if err.size else 0.0
