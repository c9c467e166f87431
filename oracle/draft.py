"""Draft-side steps of one draft-worker iteration (test infrastructure).

What is computed (SwiftSpec summary, Section 3.1.1 Algorithm 1 steps
Synchronize, Re-root and Select; Section 3.1.2 Figure 2; Section 3.2, the
update procedure):

* ``token_walk``: the target returns its verified tokens; the draft walks its
  tree from the root along them.  Every verified token found as a child of
  the current node moves the walk one node down.  If all of them are found,
  the last one is the new root and its subtree stays (Figure 2, iteration 1:
  verified t1, t3, t6 make t6 the root, and the nodes grown under it are the
  next input); if one is not in the tree, the walk stops there and a new tree
  starts (Figure 2, iteration 2: t16 is not in the tree).  The result is the
  (path, path length, keep flag) that the re-root of the tree cache takes.
* ``select_subtree``: the most promising subtree of bs nodes to send to the
  target.

Readings (the pages leave these open):

* A verified token matching several children of the current node (siblings
  with equal tokens) follows the lowest node index.
* "Most promising" = the largest expected number of accepted tokens under the
  draft's own distribution, the sum over the chosen nodes of the probability
  of their root path, exp(cum[i]).  cum never increases from a parent to its
  child (log-probabilities are <= 0), so the bs nodes of largest cum, ties
  broken by lower index, form a subtree (every chosen node's parent comes
  before it in that order) and maximise the sum; ``select_subtree`` returns
  them in node order with parents renumbered inside the selection.  For
  scores that rise along a path (outside that contract) a chosen node whose
  parent was left out gets parent -1.
"""
import numpy as np


def token_walk(parent, tok, n: int, verified):
    """(path, keep): the nodes matched by ``verified`` from the root, and
    whether every verified token was matched."""
    path = []
    cur = -1
    for v in verified:
        nxt = None
        for c in range(n):
            if int(parent[c]) == cur and int(tok[c]) == int(v):
                nxt = c
                break
        if nxt is None:
            return path, False
        path.append(nxt)
        cur = nxt
    return path, True


def select_subtree(parent, tok, cum, n: int, bs: int):
    """(nodes, new_parent, tokens) of the chosen subtree, nodes in increasing
    order, new_parent indexing into the selection (-1: child of the root)."""
    order = sorted(range(n), key=lambda i: (-float(cum[i]), i))
    chosen = sorted(order[:min(bs, n)])
    pos = {v: k for k, v in enumerate(chosen)}
    # a parent left out (only scores that rise along a path do that) reads -1
    new_parent = [pos.get(int(parent[v]), -1) if int(parent[v]) >= 0 else -1 for v in chosen]
    return (np.array(chosen, dtype=np.int32), np.array(new_parent, dtype=np.int32),
            np.array([int(tok[v]) for v in chosen], dtype=np.int32))
