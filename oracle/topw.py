"""Top-w maximum-likelihood candidate selection (test infrastructure).

What is computed (SwiftSpec summary, Section 3.1.3, maximum-likelihood
expansion): every node's value is the log-softmax probability of its token
under its parent's distribution; a node's weight is the sum of values from the
root down to it; an expansion step takes the ``w`` best new leaves.

Readings: the candidate pool is every (expanded node, token) pair whose token
is not already a child of that node; the root (index -1) is expandable with
its own logits row; ties break by higher score, then lower parent index,
then lower token id.  The library's tree_expand_top_w is checked against
select_top_w; the draft-expansion workload's timing baseline calls both
functions here once per round.
"""
import numpy as np


def log_softmax(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return x - (m + np.log(np.exp(x - m).sum()))


def cumulative_scores(parent, tok, logits_root, logits_nodes, n: int) -> np.ndarray:
    """cum[i] = cum[parent[i]] + log_softmax(logits of parent)[tok[i]]; cum(root) = 0."""
    cum = np.zeros(n, dtype=np.float64)
    lsm_root = log_softmax(logits_root)
    cache = {}
    for i in range(n):
        p = int(parent[i])
        if p < 0:
            cum[i] = lsm_root[int(tok[i])]
        else:
            if p not in cache:
                cache[p] = log_softmax(logits_nodes[p])
            cum[i] = cum[p] + cache[p][int(tok[i])]
    return cum


def select_top_w(parent, tok, cum, logits_root, logits_nodes, n: int, w: int):
    """Pick ``w`` new leaves.  Returns (parents [w], tokens [w], scores [w])."""
    vocab = np.asarray(logits_root).shape[0]
    par_list, tok_list, score_list = [], [], []
    for p in range(-1, n):
        row = logits_root if p < 0 else logits_nodes[p]
        base = 0.0 if p < 0 else cum[p]
        score = base + log_softmax(row)
        taken = [int(tok[c]) for c in range(n) if int(parent[c]) == p]
        allowed = np.ones(vocab, dtype=bool)
        allowed[taken] = False
        t = np.nonzero(allowed)[0]
        par_list.append(np.full(t.size, p, dtype=np.int64))
        tok_list.append(t)
        score_list.append(score[t])
    P = np.concatenate(par_list)
    T = np.concatenate(tok_list)
    S = np.concatenate(score_list)
    order = np.lexsort((T, P, -S))[:w]
    return P[order].astype(np.int32), T[order].astype(np.int32), S[order]
