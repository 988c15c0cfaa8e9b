"""Pins for the CPU oracle: checks it against facts fixed outside itself.

* hand-worked examples (tests/golden/*.json, each with its derivation),
* closed forms of the pyramid means,
* reduction to textbook dense causal attention when K covers every past block
  (a brute-force loop and torch's scaled_dot_product_attention in float64),
* reduction to flat top-K over all earlier blocks for a one-level pyramid,
* invariants: the count of route entries, level-count invariance, all-equal
  scores picking the lowest indices,
* agreement with the independent tree-walk formulation on random ragged trees,
* the checker rejecting a selection that is wrong by more than the tolerance.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import check, reference, tree_walk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)["cases"]


# ---------------------------------------------------------------------------
# hand-worked selections
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("hand_selection.json"), ids=lambda c: c["name"])
def test_hand_selection(case):
    k = np.array(case["k"], dtype=np.float64)[None]            # [1, Hk, T, d]
    d = case["d"]
    rows = np.array(case["q_rows"], dtype=np.float64)
    levels = reference.build_pyramid(k, 1, case["branching"])
    lv = [x[0, 0] for x in levels]
    us = reference.select_unit(rows, lv, case["query_block"], case["branching"], case["top_k"],
                               1.0 / math.sqrt(d))
    assert us.sel == case["sel"]
    assert [list(x) for x in us.kept] == case["kept_per_level_finest_first"]
    if "scores_level0" in case:
        got = dict(zip(us.cands[0], us.scores[0]))
        for node, want in case["scores_level0"].items():
            assert got[int(node)] == pytest.approx(want, abs=1e-9)
    # the independent formulation agrees
    tw = tree_walk.select_unit(rows, k[0, 0], case["query_block"], 1, case["branching"],
                               case["top_k"], 1.0 / math.sqrt(d))
    assert tw == case["sel"]


def test_hand_selection_through_full_tensors():
    """Same case A through select() with [B, Hq, T, d] tensors and GQA head mapping."""
    case = _load("hand_selection.json")[0]
    k = np.array(case["k"], dtype=np.float64)[None]
    q = np.zeros((1, 1, 8, 1))
    q[0, 0, 7, 0] = 1.0
    levels = reference.build_pyramid(k, 1, 2)
    sel, _ = reference.select(q, levels, 8, 1, 2, 1, scale=1.0)
    assert list(sel[0, 0, 7]) == [5, 7]
    assert list(sel[0, 0, 0]) == [0, -1]


# ---------------------------------------------------------------------------
# hand-worked attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("hand_attention.json"), ids=lambda c: c["name"])
def test_hand_attention(case):
    T = len(case["q"])
    q = np.array(case["q"], dtype=np.float64).reshape(1, 1, T, 1)
    k = np.array(case["k"], dtype=np.float64).reshape(1, 1, T, 1)
    v = np.array(case["v"], dtype=np.float64).reshape(1, 1, T, 1)
    levels = reference.build_pyramid(k, 1, case["branching"])
    sel, _ = reference.select(q, levels, T, 1, case["branching"], case["top_k"], scale=1.0)
    if "sel_rows" in case:
        assert sel[0, 0].tolist() == case["sel_rows"]
    o, lse = reference.attention(q, k, v, sel, 1, scale=1.0)
    assert o[0, 0, :, 0] == pytest.approx(case["o"], abs=1e-12)
    assert lse[0, 0] == pytest.approx(case["lse"], abs=1e-12)


# ---------------------------------------------------------------------------
# pyramid closed forms
# ---------------------------------------------------------------------------

def test_level_sizes():
    assert reference.level_sizes(32, 2) == [32, 16, 8, 4, 2, 1]
    assert reference.level_sizes(2048, 4) == [2048, 512, 128, 32, 8, 2, 1]
    assert reference.level_sizes(16384, 4) == [16384, 4096, 1024, 256, 64, 16, 4, 1]
    assert reference.level_sizes(5, 2) == [5, 3, 2, 1]
    assert reference.level_sizes(1, 4) == [1]
    assert reference.level_sizes(0, 4) == []


def test_pyramid_constant_nodes():
    """Keys constant over every finest block: each node equals the token-weighted
    mean of the constants of the blocks it covers; a node inside one block's
    span is that constant exactly."""
    blk, b, nb, d = 4, 2, 8, 3
    vals = np.arange(nb, dtype=np.float64) * 1.5 - 2.0
    k = np.repeat(vals, blk)[None, None, :, None] * np.ones(d)
    levels = reference.build_pyramid(k, blk, b)
    assert np.array_equal(levels[0][0, 0, :, 0], vals)
    for lvl in range(1, len(levels)):
        span = b ** lvl
        for m in range(levels[lvl].shape[2]):
            want = vals[m * span:(m + 1) * span].mean()
            assert levels[lvl][0, 0, m, 0] == pytest.approx(want, abs=1e-12)


def test_pyramid_ragged_is_token_weighted():
    """nb=5 blocks, b=2, last block 1 token: the root is the global token mean,
    which differs from the mean of child means."""
    rng = np.random.default_rng(0)
    blk, b = 4, 2
    T = 4 * blk + 1
    k = rng.standard_normal((2, 3, T, 5))
    levels = reference.build_pyramid(k, blk, b)
    assert [x.shape[2] for x in levels] == [5, 3, 2, 1]
    np.testing.assert_allclose(levels[-1][:, :, 0], k.mean(axis=2), atol=1e-13)
    # level 1 node 2 covers block 4 only: the single last token
    np.testing.assert_allclose(levels[1][:, :, 2], k[:, :, 16], atol=0)
    # level 2 node 1 covers blocks 4 (1 token) .. : again the last token only
    np.testing.assert_allclose(levels[2][:, :, 1], k[:, :, 16], atol=0)
    # level 2 node 0 covers tokens 0..15
    np.testing.assert_allclose(levels[2][:, :, 0], k[:, :, :16].mean(axis=2), atol=1e-13)
    mean_of_means = levels[1][:, :, :].mean(axis=2)
    assert np.abs(mean_of_means - levels[-1][:, :, 0]).max() > 1e-3


# ---------------------------------------------------------------------------
# reductions to textbook routines
# ---------------------------------------------------------------------------

def _dense_causal_bruteforce(q, k, v, scale):
    B, Hq, T, d = q.shape
    G = Hq // k.shape[1]
    o = np.zeros_like(q)
    lse = np.zeros(q.shape[:3])
    for b in range(B):
        for h in range(Hq):
            for t in range(T):
                z = [scale * float(np.dot(q[b, h, t], k[b, h // G, s])) for s in range(t + 1)]
                m = max(z)
                w = [math.exp(x - m) for x in z]
                den = sum(w)
                o[b, h, t] = sum(w[s] * v[b, h // G, s] for s in range(t + 1)) / den
                lse[b, h, t] = m + math.log(den)
    return o, lse


@pytest.mark.parametrize("T,blk,b", [(37, 4, 2), (64, 8, 3), (50, 16, 4)])
def test_full_budget_equals_dense_causal(T, blk, b):
    """K >= number of past blocks: every block <= the query block is selected and
    the output is dense causal attention (brute force and torch SDPA, float64)."""
    rng = np.random.default_rng(T)
    B, Hq, Hk, d = 2, 4, 2, 8
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hk, T, d))
    v = rng.standard_normal((B, Hk, T, d))
    nb = reference.num_blocks(T, blk)
    K = nb - 1
    levels = reference.build_pyramid(k, blk, b)
    sel, _ = reference.select(q, levels, T, blk, b, K)
    for i in range(nb):
        assert list(sel[:, :, i][0, 0]) == list(range(i + 1)) + [-1] * (K - i)
    scale = 1 / math.sqrt(d)
    o, lse = reference.attention(q, k, v, sel, blk)
    o_bf, lse_bf = _dense_causal_bruteforce(q, k, v, scale)
    np.testing.assert_allclose(o, o_bf, atol=1e-12)
    np.testing.assert_allclose(lse, lse_bf, atol=1e-12)
    kk = torch.from_numpy(k).repeat_interleave(Hq // Hk, dim=1)
    vv = torch.from_numpy(v).repeat_interleave(Hq // Hk, dim=1)
    o_t = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kk, vv,
                                                           is_causal=True).numpy()
    np.testing.assert_allclose(o, o_t, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_one_level_equals_flat_topk(seed):
    """b >= nb: the pyramid is the blocks plus a root, and the selection is flat
    top-K of the LSE score over all earlier blocks (argsort + scipy logsumexp)."""
    rng = np.random.default_rng(seed)
    blk, d, G = 4, 6, 2
    nb = int(rng.integers(3, 20))
    T = nb * blk - int(rng.integers(0, blk))
    K = int(rng.integers(1, 6))
    q = rng.standard_normal((1, G, T, d))
    k = rng.standard_normal((1, 1, T, d))
    levels = reference.build_pyramid(k, blk, nb)            # b = nb
    assert len(levels) == 2
    sel, _ = reference.select(q, levels, T, blk, nb, K)
    scale = 1 / math.sqrt(d)
    for i in range(reference.num_blocks(T, blk)):
        rows = q[0, :, i * blk:(i + 1) * blk, :].reshape(-1, d)
        means = np.stack([k[0, 0, j * blk:(j + 1) * blk].mean(axis=0) for j in range(i)]) if i else None
        if i == 0:
            flat = []
        else:
            s = logsumexp(scale * rows @ means.T, axis=0)
            order = np.argsort(-s, kind="stable")             # stable: ties keep lower index
            flat = sorted(order[:K].tolist())
        want = flat + [i]
        assert list(sel[0, 0, i][:len(want)]) == want
        assert all(x == -1 for x in sel[0, 0, i][len(want):])


def test_one_token_blocks_reduce_to_per_query_centroid_routing():
    """With one-token query rows the LSE score is the scaled dot product with the
    block centroid, so one-level selection is top-K of q . centroid (the flat
    per-query routing by block means of PHBA §3.1)."""
    rng = np.random.default_rng(7)
    blk, d, T, K = 8, 5, 80, 3
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, T, d))
    levels = reference.build_pyramid(k, blk, 16)
    sel, _ = reference.select(q, levels, T, blk, 16, K)
    cent = k[0, 0].reshape(10, blk, d).mean(axis=1)
    dots = cent[:9] @ q[0, 0, 0]
    want = sorted(np.argsort(-dots)[:K].tolist()) + [9]
    assert list(sel[0, 0, 0]) == want


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def _random_problem(rng, b=None):
    blk = int(rng.choice([1, 2, 4]))
    b = b or int(rng.integers(2, 5))
    nb = int(rng.integers(1, 41))
    T = nb * blk - (int(rng.integers(0, blk)) if blk > 1 else 0)
    d = int(rng.integers(1, 6))
    G = int(rng.integers(1, 3))
    K = int(rng.integers(1, 7))
    q = rng.standard_normal((1, G, T, d))
    k = rng.standard_normal((1, 1, T, d)) + rng.standard_normal(d)
    return blk, b, T, d, G, K, q, k


@pytest.mark.parametrize("seed", range(40))
def test_invariants_random(seed):
    rng = np.random.default_rng(100 + seed)
    blk, b, T, d, G, K, q, k = _random_problem(rng)
    levels = reference.build_pyramid(k, blk, b)
    sel, trace = reference.select(q, levels, T, blk, b, K)
    scale = 1 / math.sqrt(d)
    for i in range(sel.shape[2]):
        row = sel[0, 0, i]
        valid = [int(x) for x in row if x >= 0]
        # count: min(K, i) + 1, ascending, diagonal last, -1 padding only at the end
        assert len(valid) == min(K, i) + 1
        assert valid[-1] == i and valid == sorted(valid)
        assert all(x == -1 for x in row[len(valid):])
        # the independent tree-walk formulation agrees
        toks = np.arange(i * blk, min((i + 1) * blk, T))
        rows = np.concatenate([q[0, h, toks, :] for h in range(G)], axis=0)
        assert tree_walk.select_unit(rows, k[0, 0], i * blk, blk, b, K, scale) == valid
        # level-count invariance: dropping levels above one with <= K+1 nodes
        sizes = [x.shape[2] for x in levels]
        top = min(j for j, n in enumerate(sizes) if n <= K + 1)
        lv = [x[0, 0] for x in levels[:top + 1]]
        assert reference.select_unit(rows, lv, i, b, K, scale).sel == valid


def test_zero_queries_pick_lowest_blocks():
    """q = 0 makes every score log(R): all ties, so the lowest indices win."""
    rng = np.random.default_rng(3)
    blk, b, T, d, K = 4, 3, 4 * 30, 4, 5
    q = np.zeros((1, 2, T, d))
    k = rng.standard_normal((1, 1, T, d))
    levels = reference.build_pyramid(k, blk, b)
    sel, _ = reference.select(q, levels, T, blk, b, K)
    for i in range(30):
        want = list(range(min(K, i))) + [i]
        assert list(sel[0, 0, i][:len(want)]) == want


def test_decode_unit_uses_last_position():
    """Decode: the query at Tk-1 selects like the last row of a prefill whose
    query block holds that row alone, and sees every token of its selection."""
    rng = np.random.default_rng(11)
    blk, b, T, d, K, G = 4, 2, 4 * 13 + 2, 4, 3, 2
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    qd = rng.standard_normal((1, G, 1, d))
    levels = reference.build_pyramid(k, blk, b)
    sel, _ = reference.select(qd, levels, T, blk, b, K)
    assert sel.shape == (1, 1, 1, K + 1)
    diag = (T - 1) // blk
    rows = qd[0, :, 0, :]
    want = reference.select_unit(rows, [x[0, 0] for x in levels], diag, b, K, 1 / math.sqrt(d)).sel
    assert list(sel[0, 0, 0]) == want
    assert tree_walk.select_unit(rows, k[0, 0], T - 1, blk, b, K, 1 / math.sqrt(d)) == want
    o, lse = reference.attention(qd, k, v, sel, blk)
    toks = np.concatenate([np.arange(j * blk, min((j + 1) * blk, T)) for j in want])
    for h in range(G):
        z = (k[0, 0, toks] @ qd[0, h, 0]) / math.sqrt(d)
        w = np.exp(z - z.max())
        np.testing.assert_allclose(o[0, h, 0], w @ v[0, 0, toks] / w.sum(), atol=1e-12)
        assert lse[0, h, 0] == pytest.approx(z.max() + math.log(w.sum()), abs=1e-12)


def test_attention_equals_masked_dense():
    """Gathered attention equals dense attention with every unselected key and
    every future key masked out."""
    rng = np.random.default_rng(5)
    blk, b, T, d, K, Hq, Hk = 4, 2, 4 * 12, 6, 2, 4, 2
    q = rng.standard_normal((1, Hq, T, d))
    k = rng.standard_normal((1, Hk, T, d))
    v = rng.standard_normal((1, Hk, T, d))
    levels = reference.build_pyramid(k, blk, b)
    sel, _ = reference.select(q, levels, T, blk, b, K)
    o, lse = reference.attention(q, k, v, sel, blk)
    for h in range(Hq):
        hk = h // (Hq // Hk)
        z = q[0, h] @ k[0, hk].T / math.sqrt(d)
        allowed = np.zeros((T, T), dtype=bool)
        for t in range(T):
            for j in sel[0, hk, t // blk]:
                if j >= 0:
                    allowed[t, j * blk:(j + 1) * blk] = True
        allowed &= np.tril(np.ones((T, T), dtype=bool))
        z = np.where(allowed, z, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p = p / p.sum(1, keepdims=True)
        np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)
        np.testing.assert_allclose(o[0, h], p @ v[0, hk], atol=1e-12)
        np.testing.assert_allclose(lse[0, h], logsumexp(z, axis=1), atol=1e-12)


# ---------------------------------------------------------------------------
# the checker
# ---------------------------------------------------------------------------

def _unit_fixture():
    rng = np.random.default_rng(21)
    blk, b, T, d, K = 4, 2, 4 * 16, 8, 2
    q = rng.standard_normal((1, 1, T, d))
    k = rng.standard_normal((1, 1, T, d))
    levels = reference.build_pyramid(k, blk, b)
    lv = [x[0, 0] for x in levels]
    i = 15
    rows = q[0, 0, i * blk:(i + 1) * blk]
    ref = reference.select_unit(rows, lv, i, b, K, 1 / math.sqrt(d))
    return rows, lv, i, b, K, 1 / math.sqrt(d), ref


def test_checker_accepts_oracle_and_rejects_planted_mistake():
    rows, lv, i, b, K, scale, ref = _unit_fixture()
    row = ref.sel + [-1] * (K + 1 - len(ref.sel))
    kept = [x + [-1] * (K - len(x)) for x in ref.kept]
    assert check.check_unit(rows, lv, i, b, K, scale, row, kept)[0] == "exact"
    # plant a mistake: swap the worst kept finest block for the worst-scored candidate
    s = dict(zip(ref.cands[0], ref.scores[0]))
    worst_rej = min((c for c in ref.cands[0] if c not in ref.kept[0]), key=lambda c: s[c])
    bad0 = sorted([worst_rej] + ref.kept[0][1:])
    bad_kept = [bad0 + [-1] * (K - len(bad0))] + kept[1:]
    bad_row = bad0 + [i]
    status, info = check.check_unit(rows, lv, i, b, K, scale, bad_row, bad_kept)
    assert status == "fail" and info["level"] == 0
    # a route row inconsistent with its own trace fails too
    status, _ = check.check_unit(rows, lv, i, b, K, scale, bad_row, kept)
    assert status == "fail"


def test_checker_accepts_near_tie_swap():
    """Two candidates within the tolerance may swap; the walk follows the swap."""
    rows, lv, i, b, K, scale, ref = _unit_fixture()
    lv = [x.copy() for x in lv]
    # make the best rejected finest candidate tie with the lowest kept one up to 1e-7
    s = dict(zip(ref.cands[0], ref.scores[0]))
    low_kept = min(ref.kept[0], key=lambda c: s[c])
    best_rej = max((c for c in ref.cands[0] if c not in ref.kept[0]), key=lambda c: s[c])
    lv[0][best_rej] = lv[0][low_kept] * (1 + 1e-9)
    ref2 = reference.select_unit(rows, lv, i, b, K, scale)
    swapped = sorted([c for c in ref2.kept[0] if c != best_rej and c != low_kept] +
                     [low_kept if best_rej in ref2.kept[0] else best_rej])
    row = swapped + [i]
    kept = [swapped] + [x + [-1] * (K - len(x)) for x in ref2.kept[1:]]
    status, info = check.check_unit(rows, lv, i, b, K, scale, row, kept)
    assert status == "near_tie" and info["gap"] < 1e-4
