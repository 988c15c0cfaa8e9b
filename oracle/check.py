"""Tie-tolerant comparison of a device selection with the oracle (test infrastructure).

TEST INFRASTRUCTURE ONLY.

A device computes LogSumExp scores in fp32 with its own summation order, so two
candidates whose scores differ by less than that rounding can swap places.  One
swap at a coarse level changes every finer candidate set, so a mismatch is
judged level by level along the device's own per-level kept sets (its trace):

* at each level the candidate set is rebuilt from the device's kept set one
  level up (``reference.candidates``) and scored in float64;
* the device's kept set must be a subset of the candidates of size
  min(K, |candidates|), and its lowest float64 score may undercut the highest
  rejected score by at most ``tol`` (the near-tie gap, natural-log units);
* the device route row must be its finest kept set ascending, then the
  diagonal block, then -1.

A unit whose route row equals the oracle's is "exact"; one that differs but
passes the walk is a "near_tie" (with the largest amount by which a rejected
candidate outscored a kept one, at most ``tol``); anything else is a "fail".
"""

from __future__ import annotations

import numpy as np

from . import reference


def _padded(sel: list[int], width: int) -> list[int]:
    return list(sel) + [-1] * (width - len(sel))


def check_unit(rows, levels_bh, diag, branching, top_k, scale, dev_row, dev_kept_levels,
               tol=1e-4, k_finest=None, ref_row=None, row_width=None):
    """Judge one unit.

    rows            [R, d] query rows of the unit (float64)
    levels_bh       per level [n_l, d] float64 pooled keys of the unit's KV head
    dev_row         device route row (length K+1, -1 padded)
    dev_kept_levels per level (finest first) the device's kept node ids, -1 padded,
                    or None when the device gave no trace
    top_k           nodes kept per level; k_finest (default top_k) at the finest
                    level, where a budget fallback may keep more
    ref_row         the oracle's route row when the caller computed it (budget
                    and fallback selections); default select_unit's
    row_width       slots of a route row (default top_k + 1)
    Returns (status, info) with status in {"exact", "near_tie", "fail"}.
    """
    width = top_k + 1 if row_width is None else row_width
    k0 = top_k if k_finest is None else k_finest
    if ref_row is None:
        ref_row = reference.select_unit(rows, levels_bh, diag, branching, top_k, scale).sel
    ref = reference.UnitSelection(sel=list(ref_row))
    dev_row = [int(x) for x in dev_row]
    if dev_row == _padded(ref.sel, width):
        return "exact", {}
    if dev_kept_levels is None:
        return "fail", {"reason": "route row differs and no trace to judge it", "oracle": ref.sel,
                        "device": dev_row}
    sizes = [lv.shape[0] for lv in levels_bh]
    kept_above: list[int] = []
    worst = 0.0
    for level in range(len(sizes) - 1, -1, -1):
        cand = reference.candidates(level, kept_above, diag, sizes, branching)
        dev = sorted(int(x) for x in dev_kept_levels[level] if x >= 0)
        kl = k0 if level == 0 else top_k
        want = min(kl, len(cand))
        if len(dev) != want or not set(dev) <= set(cand) or len(set(dev)) != len(dev):
            return "fail", {"reason": "kept set is not a K-subset of the candidates", "level": level,
                            "cand": cand, "device": dev}
        if len(cand) > kl:
            s = reference.lse_scores(rows, levels_bh[level][cand], scale)
            by_id = dict(zip(cand, s))
            low_kept = min(by_id[c] for c in dev)
            high_rej = max(by_id[c] for c in cand if c not in set(dev))
            gap = high_rej - low_kept
            if gap > tol:
                return "fail", {"reason": "kept set is not a top-K within tolerance", "level": level,
                                "gap": float(gap)}
            worst = max(worst, float(gap))
        kept_above = dev
    if dev_row != _padded(sorted(kept_above) + [diag], width):
        return "fail", {"reason": "route row does not follow the finest kept set", "device": dev_row}
    return "near_tie", {"oracle": ref.sel, "device": dev_row, "gap": worst}
