"""Level-synchronous CPU oracle (float64 NumPy) for the pyramid selector and the
block-sparse causal attention that runs over its selection.

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the product path.

Notation (PISA abstract; PHBA §A.1.2):
  block     tokens per key block and per query block (64 throughout the path)
  nb        ceil(Tk / block), number of finest-level key blocks
  b         branching factor of the pyramid
  n_l       nodes at level l: n_0 = nb, n_{l+1} = ceil(n_l / b), down to one root
  K         nodes kept per level (the diagonal block is added on top of them)
  scale     1 / sqrt(d) unless given
  unit      (batch, KV head, query block); all query heads of the KV group share
            the unit's selection; query head h belongs to KV head h // (Hq / Hk)

Readings of the pages this oracle rests on (the pages leave these open):
  R1  Only nodes that lie entirely before the diagonal block are ever scored or
      kept.  The chain of ancestors of the diagonal block is always expanded and
      does not count against K; its fully-past children join the candidate set.
      PHBA routes only to strictly preceding blocks (§A.1.2); scoring a node
      that also covers future keys would let the future steer the selection.
  R2  The pyramid is built up to a single root.  Levels with at most K
      candidates keep all of them without scoring, so the start level does not
      change the result.
  R3  A pooled key is the mean of all key tokens the node covers (valid tokens
      only for a ragged last block), kept in full precision (fp64 here).
  R4  The LogSumExp of a unit runs over the union of the rows of all query heads
      of the KV group: G heads x (tokens of the query block).
  R5  Score of node n: log sum_r exp(scale * q_r . P_l[n]), natural log, no
      node-size term.
  R6  K counts kept fully-past nodes per level; the finest level therefore
      yields at most K historical blocks plus the diagonal block.
  R7  Equal scores: the lower node index wins.
  R8  Fewer than K candidates: keep them all; unused route slots hold -1
      (PHBA §A.1.2).
  R9  The route row lists the kept finest-level blocks in ascending order, then
      the diagonal block, then -1 padding up to K+1 slots.
  R10 Decode: the single query token sits at position Tk-1 and its own key is
      in the cache; its diagonal block is (Tk-1) // block.
  R11 Attention is token-causal: a query at position t sees key positions
      s <= t of its selected blocks only (this masks the diagonal block alone).
  R14 The backward treats the route table as fixed (a discrete choice with no
      gradient): q, k and v receive the gradient of the attention over the
      selected blocks only, and the pyramid and the scores receive none.  It
      recomputes the probabilities from the forward's log-sum-exp (PHBA §A.1.4).
  R15 Decode-time maintenance: after keys are appended, every node whose
      token range gains tokens holds the mean of all its tokens again (the
      pyramid equals a fresh build of the longer sequence); nodes that gain
      none are unchanged.  A pyramid laid out for a capacity C has the levels
      of ceil(C / block) blocks; levels above the root of the valid keys hold
      one node, the mean of all of them.
  R16 Packed sequences (PHBA §A.1.1-§A.1.2): a packed batch is a set of
      independent sequences, sequence s owning rows [cu[s], cu[s+1]) of every
      head.  Its blocks start at its own first row (boundaries from cu and the
      block size), its pooled keys average its own valid rows only, and its
      candidates, routes and attended keys never leave it; route slots of
      query blocks past its end hold -1.  So each sequence gets exactly the
      result of a batch-1 problem of its own length.
  R17 Budgets and fallback (PHAROS summary: per-head budgets from attention
      entropy, a wider budget when selection confidence is low; no formulas
      are given, these are ours): units of KV head h keep K_h nodes per level
      (K_h in [1, K]); at the finest level, if it was scored and the margin
      s(K_h-th best) - s(best rejected) is below a threshold tau, the unit
      keeps the best min(F, C) of the same candidates instead (F > K_h).
      Entropy budgets: K_h = clamp(round(total * H_h / sum H), k_min, k_max),
      rounding half up, an equal split when sum H = 0.
  R18 A route row is a set of blocks: the attention of a query reads each
      routed block once, however often the row lists it.  PHBA routes every
      query to top-K distinct strictly preceding blocks (§A.1.2) and its
      block-major metadata enumerates each (query, block) pair once (§A.1,
      §A.1.4); a row the selection writes never repeats a block, so this only
      fixes the meaning of rows written by hand.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


# ---------------------------------------------------------------------------
# Pyramid geometry (PISA abstract: O(log N) pooled levels)
# ---------------------------------------------------------------------------

def num_blocks(n_tokens: int, block: int) -> int:
    """Number of key blocks covering n_tokens tokens (the last may be ragged)."""
    return -(-n_tokens // block)


def level_sizes(n_blocks: int, branching: int) -> list[int]:
    """Node counts per level, finest first: n_0 = n_blocks, n_{l+1} = ceil(n_l/b),
    ending at the single root (reading R2)."""
    if n_blocks < 1:
        return []
    sizes = [n_blocks]
    while sizes[-1] > 1:
        sizes.append(-(-sizes[-1] // branching))
    return sizes


def node_block_range(level: int, m: int, n_blocks: int, branching: int) -> tuple[int, int]:
    """Finest-level blocks [lo, hi) covered by node m of a level."""
    span = branching ** level
    return m * span, min((m + 1) * span, n_blocks)


def children(level: int, m: int, sizes: list[int], branching: int) -> list[int]:
    """Children (at level-1) of node m of level `level`."""
    return [c for c in range(m * branching, (m + 1) * branching) if c < sizes[level - 1]]


# ---------------------------------------------------------------------------
# Pyramid build (reading R3)
# ---------------------------------------------------------------------------

def build_pyramid(k: np.ndarray, block: int, branching: int) -> list[np.ndarray]:
    """Mean-pooled key pyramid.

    k: [B, Hk, Tk, d] keys (any float dtype; upcast exactly to float64).
    Returns one float64 array [B, Hk, n_l, d] per level, finest first.  Every
    node is the plain mean of the key tokens it covers, taken straight from the
    tokens, not from the level below.
    """
    k = np.asarray(k, dtype=np.float64)
    B, Hk, Tk, d = k.shape
    nb = num_blocks(Tk, block)
    sizes = level_sizes(nb, branching)
    levels = []
    for lvl, n in enumerate(sizes):
        out = np.empty((B, Hk, n, d), dtype=np.float64)
        for m in range(n):
            lo, hi = node_block_range(lvl, m, nb, branching)
            t0, t1 = lo * block, min(hi * block, Tk)
            out[:, :, m, :] = k[:, :, t0:t1, :].mean(axis=2)
        levels.append(out)
    return levels


def append_pyramid(levels: list[np.ndarray], k: np.ndarray, old_len: int, block: int,
                   branching: int) -> list[np.ndarray]:
    """Pyramid of k[:, :, :new_len] from the pyramid `levels` of its first
    old_len tokens (new_len = k.shape[2]), by running sums (decode-time
    maintenance; reading R15): a node over tokens [t0, t1) had
    c_old = |[t0, t1) cut [0, old_len)| tokens; its new mean is
    (mean_old * c_old + sum of k over [max(t0, old_len), min(t1, new_len)))
    / c_new.  Nodes that gain no token keep their old value; new nodes (and
    new levels) start from c_old = 0.  Only the new tokens are read.
    """
    k = np.asarray(k, dtype=np.float64)
    B, Hk, new_len, d = k.shape
    if not 0 < old_len <= new_len:
        raise ValueError("need 0 < old_len <= new_len")
    nb_old, nb = num_blocks(old_len, block), num_blocks(new_len, block)
    sizes_old, sizes = level_sizes(nb_old, branching), level_sizes(nb, branching)
    out = []
    for lvl, n in enumerate(sizes):
        lv = np.zeros((B, Hk, n, d), dtype=np.float64)
        if lvl < len(sizes_old):
            lv[:, :, :sizes_old[lvl], :] = levels[lvl]
        elif sizes_old:
            lv[:, :, 0, :] = levels[-1][:, :, 0, :]  # the old root covers every old token
        for m in range(n):
            lo, hi = node_block_range(lvl, m, nb, branching)
            t0, t1 = lo * block, min(hi * block, new_len)
            c_old = max(0, min(t1, old_len) - t0)
            a = max(t0, old_len)
            if a >= t1:
                continue  # no new token under this node
            add_sum = k[:, :, a:t1, :].sum(axis=2)
            lv[:, :, m, :] = (lv[:, :, m, :] * c_old + add_sum) / (t1 - t0)
        out.append(lv)
    return out


def concat_levels(levels: list[np.ndarray]) -> np.ndarray:
    """Levels concatenated finest first along the node axis: [B, Hk, N_tot, d]."""
    return np.concatenate(levels, axis=2)


# ---------------------------------------------------------------------------
# Units
# ---------------------------------------------------------------------------

def _check_lengths(Tq: int, Tk: int) -> None:
    if not (Tq == Tk or Tq == 1):
        raise ValueError("oracle covers prefill (q_len == kv_len) and decode (q_len == 1) only")


def query_positions(Tq: int, Tk: int) -> np.ndarray:
    """Absolute position of every query token (prefill: t; decode: Tk-1, R10)."""
    _check_lengths(Tq, Tk)
    return np.arange(Tq) + (Tk - Tq)


def num_query_blocks(Tq: int, Tk: int, block: int) -> int:
    _check_lengths(Tq, Tk)
    return 1 if (Tq == 1 and Tk > 1) else num_blocks(Tq, block)


def unit_tokens(i: int, Tq: int, Tk: int, block: int) -> tuple[np.ndarray, int]:
    """Query-token indices of query block i and the unit's diagonal block."""
    pos = query_positions(Tq, Tk)
    if Tq == 1 and Tk > 1:
        toks = np.array([0])
    else:
        toks = np.arange(i * block, min((i + 1) * block, Tq))
    diag = int(pos[toks[0]]) // block
    return toks, diag


def unit_rows(q: np.ndarray, bi: int, hk: int, group: int, toks: np.ndarray) -> np.ndarray:
    """Rows of a unit (reading R4): every query head of the KV group, every token
    of the query block, stacked head-major into [G * len(toks), d] float64."""
    heads = range(hk * group, (hk + 1) * group)
    return np.concatenate([np.asarray(q[bi, h, toks, :], dtype=np.float64) for h in heads], axis=0)


# ---------------------------------------------------------------------------
# Selection (PISA abstract; readings R1, R4-R9)
# ---------------------------------------------------------------------------

def lse_scores(rows: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """s(n) = log sum_r exp(scale * rows[r] . keys[n]), max-subtracted, float64."""
    z = scale * (rows @ keys.T)            # [R, C]
    mx = z.max(axis=0)
    return mx + np.log(np.exp(z - mx).sum(axis=0))


def top_k_nodes(cand: list[int], s: np.ndarray, top_k: int) -> list[int]:
    """The top_k candidates by score, higher first; equal scores prefer the
    lower node index (reading R7)."""
    order = sorted(range(len(cand)), key=lambda j: (-s[j], cand[j]))
    return [cand[j] for j in order[:top_k]]


@dataclass
class UnitSelection:
    sel: list[int]                                   # kept finest blocks ascending, then diag
    kept: list[list[int]] = field(default_factory=list)       # per level (finest first), ascending
    cands: list[list[int]] = field(default_factory=list)      # per level, in construction order
    scores: list[np.ndarray | None] = field(default_factory=list)  # per level, None if unscored


def candidates(level: int, kept_above: list[int], diag: int, sizes: list[int],
               branching: int) -> list[int]:
    """Bounded candidate set of one level (reading R1).

    Top level: every node of that level lying wholly before the diagonal block's
    ancestor.  Below: the children of the nodes kept one level up, followed by
    the children of the diagonal's ancestor one level up that lie wholly before
    the diagonal's ancestor at this level.
    """
    anc = diag // branching ** level
    if level == len(sizes) - 1:
        return list(range(anc))
    anc_up = diag // branching ** (level + 1)
    out = []
    for p in kept_above:
        out.extend(children(level + 1, p, sizes, branching))
    out.extend(range(anc_up * branching, anc))
    return out


def select_unit(rows: np.ndarray, levels: list[np.ndarray], diag: int, branching: int,
                top_k: int, scale: float) -> UnitSelection:
    """Coarse-to-fine top-K for one unit.

    rows:   [R, d] query rows of the unit.
    levels: per level [n_l, d] pooled keys of the unit's (batch, KV head).
    """
    sizes = [lv.shape[0] for lv in levels]
    L = len(sizes)
    res = UnitSelection(sel=[], kept=[None] * L, cands=[None] * L, scores=[None] * L)
    kept: list[int] = []
    for level in range(L - 1, -1, -1):
        cand = candidates(level, kept, diag, sizes, branching)
        res.cands[level] = cand
        if len(cand) <= top_k:                      # R8: keep all, nothing to rank
            kept = sorted(cand)
        else:
            s = lse_scores(rows, levels[level][cand], scale)
            res.scores[level] = s
            kept = sorted(top_k_nodes(cand, s, top_k))
        res.kept[level] = kept
    res.sel = sorted(kept) + [diag]                  # R9
    return res


def finest_margin(s: np.ndarray, k: int) -> float:
    """The k-th best score minus the (k+1)-th best (the best rejected one)."""
    ordered = np.sort(np.asarray(s, dtype=np.float64))[::-1]
    return float(ordered[k - 1] - ordered[k])


def select_unit_budget(rows: np.ndarray, levels: list[np.ndarray], diag: int, branching: int,
                       k_h: int, scale: float, fallback_k: int = 0,
                       fallback_margin: float = 0.0) -> UnitSelection:
    """select_unit with a budget of k_h nodes per level and the finest-level
    confidence fallback of reading R17.  The result carries .fallback (bool)
    and .margin (the finest level's margin, None when it was not scored)."""
    res = select_unit(rows, levels, diag, branching, k_h, scale)
    res.fallback, res.margin = False, None
    s0 = res.scores[0]
    if s0 is not None:                               # the finest level was scored
        res.margin = finest_margin(s0, k_h)
        if fallback_k > k_h and res.margin < fallback_margin:
            cand = res.cands[0]
            kept = sorted(top_k_nodes(cand, s0, min(fallback_k, len(cand))))
            res.kept[0] = kept
            res.sel = kept + [diag]
            res.fallback = True
    return res


def budgets_from_entropy(entropy, total: int, k_min: int, k_max: int) -> list[int]:
    """Per-head budgets in proportion to attention entropy (reading R17)."""
    ent = [float(x) for x in entropy]
    tot = sum(ent)
    out = []
    for x in ent:
        share = total * x / tot if tot > 0 else total / len(ent)
        out.append(int(min(max(math.floor(share + 0.5), k_min), k_max)))
    return out


def select(q: np.ndarray, levels: list[np.ndarray], Tk: int, block: int, branching: int,
           top_k: int, scale: float | None = None, units=None):
    """Route table for every (or the listed) unit.

    q:      [B, Hq, Tq, d]; levels: output of build_pyramid for [B, Hk, Tk, d] keys.
    units:  optional iterable of (batch, kv_head, query_block); default all.
    Returns (sel, trace) with sel an int64 array [B, Hk, nqb, K+1] (-1 padded,
    rows not listed in `units` left at -2) and trace a dict keyed by unit
    holding the UnitSelection.
    """
    B, Hq, Tq, d = q.shape
    Hk = levels[0].shape[1]
    group = Hq // Hk
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nqb = num_query_blocks(Tq, Tk, block)
    sel = np.full((B, Hk, nqb, top_k + 1), -2, dtype=np.int64)
    trace = {}
    if units is None:
        units = [(bi, hk, i) for bi in range(B) for hk in range(Hk) for i in range(nqb)]
    for bi, hk, i in units:
        toks, diag = unit_tokens(i, Tq, Tk, block)
        rows = unit_rows(q, bi, hk, group, toks)
        lv = [x[bi, hk] for x in levels]
        us = select_unit(rows, lv, diag, branching, top_k, scale)
        sel[bi, hk, i, :] = -1
        sel[bi, hk, i, :len(us.sel)] = us.sel
        trace[(bi, hk, i)] = us
    return sel, trace


# ---------------------------------------------------------------------------
# Block-sparse causal attention (PHBA §3.1, §A.1.3; reading R11)
# ---------------------------------------------------------------------------

def attend_rows(rows: np.ndarray, row_pos: np.ndarray, k_bh: np.ndarray, v_bh: np.ndarray,
                blocks: list[int], block: int, scale: float):
    """Exact softmax attention of `rows` over the tokens of `blocks`.

    rows [R, d] at absolute positions row_pos [R]; k_bh, v_bh [Tk, d] of the KV
    head.  A row sees key position s only if s lies in a listed block and
    s <= its own position.  Returns (o [R, d], lse [R]) in float64.
    """
    Tk = k_bh.shape[0]
    blocks = list(dict.fromkeys(int(j) for j in blocks))      # R18: each block once
    key_pos = np.concatenate([np.arange(j * block, min((j + 1) * block, Tk)) for j in blocks])
    kk = np.asarray(k_bh[key_pos], dtype=np.float64)
    vv = np.asarray(v_bh[key_pos], dtype=np.float64)
    z = scale * (rows @ kk.T)                                  # [R, S]
    visible = key_pos[None, :] <= row_pos[:, None]
    z = np.where(visible, z, -np.inf)
    mx = z.max(axis=1, keepdims=True)
    p = np.exp(z - mx)
    denom = p.sum(axis=1, keepdims=True)
    o = (p @ vv) / denom
    lse = mx[:, 0] + np.log(denom[:, 0])
    return o, lse


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray, block: int,
              scale: float | None = None, units=None):
    """Block-sparse causal attention over a route table.

    q [B, Hq, Tq, d]; k, v [B, Hk, Tk, d]; sel [B, Hk, nqb, K+1] (-1 padded).
    Returns o [B, Hq, Tq, d] and lse [B, Hq, Tq] in float64 (NaN outside the
    listed units).
    """
    B, Hq, Tq, d = q.shape
    _, Hk, Tk, _ = k.shape
    group = Hq // Hk
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nqb = num_query_blocks(Tq, Tk, block)
    pos = query_positions(Tq, Tk)
    o = np.full((B, Hq, Tq, d), np.nan)
    lse = np.full((B, Hq, Tq), np.nan)
    if units is None:
        units = [(bi, hk, i) for bi in range(B) for hk in range(Hk) for i in range(nqb)]
    for bi, hk, i in units:
        toks, _ = unit_tokens(i, Tq, Tk, block)
        blocks = [int(x) for x in sel[bi, hk, i] if x >= 0]
        for h in range(hk * group, (hk + 1) * group):
            rows = np.asarray(q[bi, h, toks, :], dtype=np.float64)
            oo, ll = attend_rows(rows, pos[toks], k[bi, hk], v[bi, hk], blocks, block, scale)
            o[bi, h, toks, :] = oo
            lse[bi, h, toks] = ll
    return o, lse


# ---------------------------------------------------------------------------
# Backward of the block-sparse attention for a fixed route table (PHBA §A.1.4:
# probabilities recomputed from the forward's log-sum-exp; reading R14)
# ---------------------------------------------------------------------------

def attend_rows_backward(rows: np.ndarray, row_pos: np.ndarray, k_bh: np.ndarray,
                         v_bh: np.ndarray, blocks: list[int], block: int, scale: float,
                         d_out: np.ndarray, lse: np.ndarray, o: np.ndarray | None = None):
    """Gradients of o = softmax(scale * rows k^T) v over the visible keys of
    `blocks` (the same visibility as attend_rows), given d_out = dL/do and the
    forward's lse.  With P the probabilities, dP = d_out v^T,
    D = rowsum(d_out * o) = rowsum(P * dP) and dS = P * (dP - D):
      d_rows = scale * dS k,  dk = scale * dS^T rows,  dv = P^T d_out.
    Returns (d_rows [R, d], key_pos [S], dk [S, d], dv [S, d]) in float64; the
    key rows dk and dv belong to the key positions key_pos.

    o, when given, is the forward's output over the rows' whole route (the one
    lse belongs to) and D is taken from it; `blocks` may then be any subset of
    that route, and dk, dv are those keys' gradients exactly (d_rows is then
    only the part of the subset).  When o is None, D comes from P over
    `blocks`, which must be the whole route.
    """
    Tk = k_bh.shape[0]
    blocks = list(dict.fromkeys(int(j) for j in blocks))      # R18: each block once
    key_pos = np.concatenate([np.arange(j * block, min((j + 1) * block, Tk)) for j in blocks])
    kk = np.asarray(k_bh[key_pos], dtype=np.float64)
    vv = np.asarray(v_bh[key_pos], dtype=np.float64)
    z = scale * (rows @ kk.T)                                  # [R, S]
    visible = key_pos[None, :] <= row_pos[:, None]
    p = np.where(visible, np.exp(z - lse[:, None]), 0.0)       # P from the log-sum-exp
    if o is None:
        o = p @ vv
    dp = d_out @ vv.T
    dsum = (d_out * o).sum(axis=1, keepdims=True)              # D
    ds = p * (dp - dsum)
    d_rows = scale * (ds @ kk)
    dk = scale * (ds.T @ rows)
    dv = p.T @ d_out
    return d_rows, key_pos, dk, dv


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel: np.ndarray,
                       block: int, d_out: np.ndarray, scale: float | None = None,
                       lse: np.ndarray | None = None):
    """dq, dk, dv of block-sparse causal attention over a fixed route table.

    q, d_out [B, Hq, Tq, d]; k, v [B, Hk, Tk, d]; sel [B, Hk, nqb, K+1].  The
    gradients of the G query heads of a KV group add up in dk and dv.  lse is
    the forward's [B, Hq, Tq] log-sum-exp (recomputed when not given).  Returns
    float64 arrays shaped like q, k and v.  Prefill only (q_len == kv_len).
    """
    B, Hq, Tq, d = q.shape
    _, Hk, Tk, _ = k.shape
    if Tq != Tk:
        raise ValueError("the backward is defined for prefill (q_len == kv_len)")
    group = Hq // Hk
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if lse is None:
        _, lse = attention(q, k, v, sel, block, scale)
    nqb = num_query_blocks(Tq, Tk, block)
    pos = query_positions(Tq, Tk)
    dq = np.zeros((B, Hq, Tq, d))
    dk = np.zeros((B, Hk, Tk, d))
    dv = np.zeros((B, Hk, Tk, d))
    for bi in range(B):
        for hk in range(Hk):
            for i in range(nqb):
                toks, _ = unit_tokens(i, Tq, Tk, block)
                blocks = [int(x) for x in sel[bi, hk, i] if x >= 0]
                for h in range(hk * group, (hk + 1) * group):
                    rows = np.asarray(q[bi, h, toks, :], dtype=np.float64)
                    g = np.asarray(d_out[bi, h, toks, :], dtype=np.float64)
                    dr, kp, dkk, dvv = attend_rows_backward(
                        rows, pos[toks], k[bi, hk], v[bi, hk], blocks, block, scale, g,
                        np.asarray(lse[bi, h, toks], dtype=np.float64))
                    dq[bi, h, toks, :] = dr
                    np.add.at(dk[bi, hk], kp, dkk)
                    np.add.at(dv[bi, hk], kp, dvv)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Packed sequences (PHBA §A.1.1: packed inputs reset state at every sequence
# boundary; §A.1.2: block boundaries from cu and the block size, means over
# valid rows, routes inside the same sequence, -1 where nothing is
# available; reading R16)
# ---------------------------------------------------------------------------

def packed_spans(cu) -> list[tuple[int, int]]:
    """(first row, length) of every sequence: sequence s owns rows [cu[s], cu[s+1])."""
    cu = [int(x) for x in cu]
    return [(cu[s], cu[s + 1] - cu[s]) for s in range(len(cu) - 1)]


def packed_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu, max_len: int, block: int,
                   branching: int, top_k: int, scale: float | None = None):
    """The whole path on a packed batch, one sequence at a time.

    q [Hq, total, d]; k, v [Hk, total, d]; cu the batch+1 row offsets;
    max_len bounds every length and fixes the route table's query-block axis.
    Every sequence runs alone as a batch-1 problem of its own length
    (build_pyramid, select, attention).  Returns a dict with
      o [Hq, total, d], lse [Hq, total]   float64, NaN on rows of no sequence
      sel [S, Hk, ceil(max_len/block), K+1]   int64, -1 past each sequence
      levels   per sequence, the oracle pyramid levels ([1, Hk, n_l, d] each)
    """
    Hq, total, d = q.shape
    Hk = k.shape[0]
    spans = packed_spans(cu)
    nqb_max = -(-max_len // block)
    o = np.full((Hq, total, d), np.nan)
    lse = np.full((Hq, total), np.nan)
    sel = np.full((len(spans), Hk, nqb_max, top_k + 1), -1, dtype=np.int64)
    levels = []
    for s, (a, n) in enumerate(spans):
        if n > max_len:
            raise ValueError(f"sequence {s} has {n} rows, more than max_len {max_len}")
        if n == 0:
            levels.append([])
            continue
        qs = np.asarray(q[None, :, a:a + n, :], dtype=np.float64)
        ks = np.asarray(k[None, :, a:a + n, :], dtype=np.float64)
        vs = np.asarray(v[None, :, a:a + n, :], dtype=np.float64)
        lv = build_pyramid(ks, block, branching)
        ss, _ = select(qs, lv, n, block, branching, top_k, scale)
        oo, ll = attention(qs, ks, vs, ss, block, scale)
        o[:, a:a + n, :] = oo[0]
        lse[:, a:a + n] = ll[0]
        sel[s, :, :ss.shape[2], :] = ss[0]
        levels.append(lv)
    return dict(o=o, lse=lse, sel=sel, levels=levels)
