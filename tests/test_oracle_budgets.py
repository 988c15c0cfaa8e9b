"""Pins of the oracle's per-head budgets and confidence fallback (reading R17;
PHAROS summary: budgets per head from attention entropy, a wider budget when
confidence is low).  The rules are this library's own, so the pins are
hand-worked values of those rules, the special cases that reduce to plain
selection, and a superset property; planted mistakes must fail them."""

import math

import numpy as np
import pytest

from oracle import reference

BLOCK = 64


def _flat_unit(x, d=4):
    """One query row (8, 0, ...) against six blocks whose pooled keys are
    (x_j, 0, ...), x_5 unused (the diagonal): with b >= 6 the pyramid is one
    level under the root, so the finest candidates are blocks 0..4 and their
    scores are scale * 8 * x_j = 4 x_j for d = 4."""
    rows = np.zeros((1, d))
    rows[0, 0] = 8.0
    lv0 = np.zeros((6, d))
    lv0[:, 0] = list(x) + [0.0]
    root = lv0.mean(axis=0, keepdims=True)
    return rows, [lv0, root], 1.0 / math.sqrt(d)


X = [0.10, 0.50, 0.48, 0.20, 0.90]   # scores 0.4, 2.0, 1.92, 0.8, 3.6


@pytest.mark.parametrize("k_h,fb_k,tau,want,fell", [
    (2, 0, 0.0, [1, 4, 5], False),        # plain top-2: blocks 4 (3.6) and 1 (2.0)
    (2, 3, 0.1, [1, 2, 4, 5], True),      # margin 2.0 - 1.92 = 0.08 < 0.1: keep 3
    (2, 3, 0.05, [1, 4, 5], False),       # 0.08 >= 0.05: no fallback
    (2, 2, 1.0, [1, 4, 5], False),        # F <= K_h: no effect
    (1, 4, 1.0, [4, 5], False),           # margin 3.6 - 2.0 = 1.6 >= 1.0
    (1, 4, 2.0, [1, 2, 3, 4, 5], True),   # 1.6 < 2.0: keep the best 4
    (3, 9, 1.5, [0, 1, 2, 3, 4, 5], True),  # margin 1.92 - 0.8 = 1.12; F past C keeps all
    (5, 6, 9.0, [0, 1, 2, 3, 4, 5], False),  # 5 candidates <= K_h: not scored
])
def test_hand_fallback(k_h, fb_k, tau, want, fell):
    rows, levels, scale = _flat_unit(X)
    us = reference.select_unit_budget(rows, levels, 5, 8, k_h, scale, fb_k, tau)
    assert us.sel == want and us.fallback == fell
    if k_h < 5:
        margins = {1: 1.6, 2: 0.08, 3: 1.12, 4: 0.4}
        assert us.margin == pytest.approx(margins[k_h], abs=1e-12)


def test_budget_equal_to_k_without_fallback_is_plain_selection():
    rng = np.random.default_rng(7)
    for trial in range(6):
        T = 64 * int(rng.integers(5, 40)) + int(rng.integers(0, 64))
        k = rng.standard_normal((1, 1, T, 16))
        q = rng.standard_normal((1, 2, T, 16))
        lv = reference.build_pyramid(k, BLOCK, 2)
        lvb = [x[0, 0] for x in lv]
        K = int(rng.integers(1, 6))
        for i in range(-(-T // BLOCK)):
            toks, diag = reference.unit_tokens(i, T, T, BLOCK)
            rows = reference.unit_rows(q, 0, 0, 2, toks)
            a = reference.select_unit(rows, lvb, diag, 2, K, 0.25)
            b = reference.select_unit_budget(rows, lvb, diag, 2, K, 0.25, 0, 0.0)
            assert a.sel == b.sel and not b.fallback


def test_fallback_keeps_a_superset_of_the_same_candidates():
    rng = np.random.default_rng(8)
    T = 64 * 37 + 9
    k = rng.standard_normal((1, 1, T, 16))
    q = rng.standard_normal((1, 4, T, 16))
    lvb = [x[0, 0] for x in reference.build_pyramid(k, BLOCK, 3)]
    fell = 0
    for i in range(-(-T // BLOCK)):
        toks, diag = reference.unit_tokens(i, T, T, BLOCK)
        rows = reference.unit_rows(q, 0, 0, 4, toks)
        base = reference.select_unit_budget(rows, lvb, diag, 3, 2, 0.25)
        wide = reference.select_unit_budget(rows, lvb, diag, 3, 2, 0.25, 5, 1e9)
        assert set(base.kept[0]) <= set(wide.kept[0]) <= set(base.cands[0])
        assert wide.kept[1:] == base.kept[1:]
        if base.scores[0] is not None:
            fell += 1
            assert wide.fallback and len(wide.kept[0]) == min(5, len(base.cands[0]))
            s = dict(zip(base.cands[0], base.scores[0]))
            rest = [s[c] for c in base.cands[0] if c not in wide.kept[0]]
            if rest:
                assert min(s[c] for c in wide.kept[0]) >= max(rest)
    assert fell > 10


@pytest.mark.parametrize("ent,total,kmin,kmax,want", [
    ([1.0, 2.0, 0.5, 0.0], 32, 2, 16, [9, 16, 5, 2]),   # 9.14, 18.29 -> 16, 4.57, 0 -> 2
    ([0.0, 0.0, 0.0], 9, 1, 8, [3, 3, 3]),              # equal split
    ([1.0, 1.0], 3, 1, 8, [2, 2]),                      # 1.5 rounds half up
    ([3.0], 7, 1, 64, [7]),
])
def test_budgets_from_entropy(ent, total, kmin, kmax, want):
    assert reference.budgets_from_entropy(ent, total, kmin, kmax) == want


_orig_margin = reference.finest_margin


def _margin_off_by_one(s, k):
    return _orig_margin(s, k + 1) if k + 1 < len(s) else _orig_margin(s, k)


def _margin_best_minus_kth(s, k):
    o = np.sort(np.asarray(s))[::-1]
    return float(o[0] - o[k - 1])


@pytest.mark.parametrize("mutant", [_margin_off_by_one, _margin_best_minus_kth])
def test_planted_margin_mistake_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(reference, "finest_margin", mutant)
    failed = 0
    for case in [(2, 3, 0.1, [1, 2, 4, 5], True), (2, 3, 0.05, [1, 4, 5], False),
                 (1, 4, 1.0, [4, 5], False), (1, 4, 2.0, [1, 2, 3, 4, 5], True)]:
        try:
            test_hand_fallback(*case)
        except AssertionError:
            failed += 1
    assert failed >= 1
