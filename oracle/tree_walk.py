"""Second, independent formulation of the pyramid selection (test infrastructure).

TEST INFRASTRUCTURE ONLY: used by the CPU tests to pin ``oracle.reference``.

Where ``reference`` works with closed-form index arithmetic (ancestor index
diag // b**l, child ranges m*b .. m*b+b-1, pooled keys per level), this module
builds the pyramid as an explicit tree by grouping b consecutive nodes bottom-up,
carries each node's token range, decides "lies wholly before the query block"
from token ranges, computes every pooled key on demand from the tokens, and
scores with scipy's logsumexp.  It walks the tree top-down (PISA abstract:
selection starts at the coarsest level and continues level by level to the
finest), keeping an "open" frontier: the kept nodes plus the one node that
contains the query block.  Candidates of a level are the children of open
nodes that end at or before the query block's first token.

It implements the same readings of the pages as ``reference`` (listed there),
in particular: the node holding the query block is always expanded and is not
counted in K; equal scores prefer the lower position.
"""

from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


class Node:
    __slots__ = ("t0", "t1", "kids", "pos")

    def __init__(self, t0, t1, kids, pos):
        self.t0, self.t1, self.kids, self.pos = t0, t1, kids, pos


def build_tree(n_tokens: int, block: int, branching: int) -> list[list[Node]]:
    """Levels of Node objects, finest first, built by grouping b neighbours."""
    leaves = []
    for pos, t0 in enumerate(range(0, n_tokens, block)):
        leaves.append(Node(t0, min(t0 + block, n_tokens), [], pos))
    levels = [leaves]
    while len(levels[-1]) > 1:
        below = levels[-1]
        above = []
        for pos, start in enumerate(range(0, len(below), branching)):
            kids = below[start:start + branching]
            above.append(Node(kids[0].t0, kids[-1].t1, kids, pos))
        levels.append(above)
    return levels


def select_unit(rows: np.ndarray, keys: np.ndarray, q_start: int, block: int,
                branching: int, top_k: int, scale: float) -> list[int]:
    """Selected finest blocks (ascending) plus the query's own block.

    rows  [R, d] query rows; keys [Tk, d] of the KV head; q_start = position of
    the first query token of the unit (its block is the diagonal block).
    """
    tree = build_tree(keys.shape[0], block, branching)
    diag_t0 = (q_start // block) * block
    rows = np.asarray(rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)

    def score(node):
        mean = keys[node.t0:node.t1].mean(axis=0)
        return float(logsumexp(scale * (rows @ mean)))

    root = tree[-1][0]
    open_nodes = [root]
    kept = []
    for _level in range(len(tree) - 2, -1, -1):
        cand = [c for n in open_nodes for c in n.kids if c.t1 <= diag_t0]
        straddle = [c for n in open_nodes for c in n.kids if c.t0 <= diag_t0 < c.t1]
        if len(cand) > top_k:
            s = np.array([score(c) for c in cand])
            pos = np.array([c.pos for c in cand])
            order = np.lexsort((pos, -s))          # primary: score desc; then position asc
            cand = [cand[j] for j in order[:top_k]]
        kept = cand
        open_nodes = kept + straddle
    return sorted(n.pos for n in kept) + [q_start // block]
