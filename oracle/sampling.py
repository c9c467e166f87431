"""Tree verification by speculative sampling, temperature > 0 (test
infrastructure).

What is computed (MineDraft notes, the PEARL walkthrough: a rejected draft
token is replaced by a sample from norm(max(0, p - q)); the same notes'
experimental setup samples at temperature 1.0; SwiftSpec summary, Section 3.1:
the draft is a tree whose edges continue a token sequence):

* At a node v the target's distribution is ``p_v = softmax(target[v] / T)``
  and the draft's ``q_v = softmax(draft[v] / T)`` (row v: after node v).
* The walk starts at the first node (lowest index) that hangs under the
  root (parent -1) and carries ``root_tok``, the token the target has already
  emitted there; none -> nothing accepted and ``bonus = root_tok``.
* At an accepted node v the children are tried in index order against a
  running target distribution r, first r = p_v.  Child c with token x is
  accepted when ``u[c] * q_v(x) < r(x)`` (probability min(1, r(x)/q_v(x))
  for u uniform on [0, 1)); the walk then moves to c.  A rejection replaces r
  by ``norm(max(0, r - q_v))`` (r is kept if that excess sums to 0) and the
  next child is tried.
* When no child of v is accepted (a leaf included), the bonus token is drawn
  from r by the inverse CDF: the smallest t whose running sum of r exceeds
  ``u_bonus * sum(r)`` (the last token with r > 0 if rounding leaves none).
* Outputs as for the greedy path: the accepted nodes from the top, their
  count, the bonus token.

Readings (the pages give only the residual rule): the acceptance
probability min(1, r/q) is the rule whose rejection branch is that residual;
siblings are independent draws from q at their parent, tried in index order
against the updated residual; the temperature divides both sides' logits;
the uniforms are inputs (one per node for its test, one per sequence for the
bonus).

With ``margins=True`` the function also returns, per sequence, how far each
decision lay from flipping: for the tests ``|r(x) - u q(x)| * Z / max(p(x),
q(x))`` (Z = product of the normalisers used so far at that node, which
scale rounding errors up), for the bonus the distance of ``u_bonus * sum(r)``
to the nearest boundary of the chosen token, over ``sum(r)``, times Z.
"""
import numpy as np


def softmax_t(row, temperature: float) -> np.ndarray:
    """softmax(row / T) in float64."""
    z = np.asarray(row, dtype=np.float64) / float(temperature)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def residual(r, q) -> tuple:
    """(norm(max(0, r - q)), excess sum); r itself when the excess is 0."""
    e = np.maximum(np.asarray(r, np.float64) - np.asarray(q, np.float64), 0.0)
    z = float(e.sum())
    if z > 0.0:
        return e / z, z
    return np.asarray(r, np.float64), 0.0


def sample_inverse_cdf(r, u: float) -> tuple:
    """(token, relative boundary distance): smallest t with cumsum(r)[t] > u*sum(r)."""
    r = np.asarray(r, dtype=np.float64)
    c = np.cumsum(r)
    total = c[-1]
    target = float(u) * total
    above = np.nonzero(c > target)[0]
    if above.size == 0:
        pos = np.nonzero(r > 0)[0]
        t = int(pos[-1]) if pos.size else r.shape[0] - 1
        return t, 0.0
    t = int(above[0])
    lo = c[t - 1] if t > 0 else 0.0
    gap = min(target - lo, c[t] - target) / total if total > 0 else 0.0
    return t, gap


def _children(parent_b, n):
    ch = [[] for _ in range(n)]
    for i in range(n):
        p = int(parent_b[i])
        if 0 <= p < i:
            ch[p].append(i)
    return ch


def accept_sampling_path(target_logits, draft_logits, parent, tok, n_nodes, root_tok,
                         u_accept, u_bonus, temperature, n_max=None, margins=False):
    """Returns ``path [B][n_max]`` (-1 padded), ``path_len [B]``, ``bonus [B]``
    (int32), and with ``margins`` also ``(test_margin [B], bonus_margin [B])``
    (inf where a sequence took no such decision)."""
    B = len(n_nodes)
    if n_max is None:
        n_max = parent.shape[1]
    path_out = np.full((B, n_max), -1, dtype=np.int32)
    path_len = np.zeros(B, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    tmarg = np.full(B, np.inf)
    bmarg = np.full(B, np.inf)
    for b in range(B):
        n = int(n_nodes[b])
        par = [int(parent[b, i]) if -1 <= int(parent[b, i]) < i else -1 for i in range(n)]
        top = [i for i in range(n) if par[i] < 0 and int(tok[b, i]) == int(root_tok[b])]
        if not top:
            bonus[b] = int(root_tok[b])
            continue
        ch = _children(par, n)
        v = top[0]
        path = [v]
        while True:
            p = softmax_t(target_logits[b][v], temperature)
            q = softmax_t(draft_logits[b][v], temperature)
            r, zprod = p, 1.0
            nxt = None
            for c in ch[v]:
                x = int(tok[b, c])
                u = float(u_accept[b, c])
                den = max(p[x], q[x])
                if den > 0:
                    tmarg[b] = min(tmarg[b], abs(r[x] - u * q[x]) * zprod / den)
                if u * q[x] < r[x]:
                    nxt = c
                    break
                r, z = residual(r, q)
                if z > 0:
                    zprod *= z
            if nxt is None:
                t, gap = sample_inverse_cdf(r, float(u_bonus[b]))
                bonus[b] = t
                bmarg[b] = gap * zprod
                break
            v = nxt
            path.append(v)
        path_out[b, : len(path)] = path
        path_len[b] = len(path)
    if margins:
        return path_out, path_len, bonus, (tmarg, bmarg)
    return path_out, path_len, bonus
