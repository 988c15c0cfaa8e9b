"""Pins of the oracle's packed-sequence path (reading R16; PHBA §A.1.1-§A.1.2):
block boundaries come from cu and the block size, pooled keys average a
sequence's own valid rows, routes and attended keys never leave the sequence,
and route slots past a sequence's end hold -1.  Each pin checks the oracle
against something other than itself: direct means of row slices, the textbook
dense causal softmax, isolation under perturbation, and the dense batch layout."""

import math

import numpy as np
import pytest

from oracle import reference

BLOCK = 64


def _inputs(lengths, Hq=4, Hk=2, d=16, spare=0, seed=0):
    rng = np.random.default_rng(seed)
    total = sum(lengths) + spare
    q = rng.standard_normal((Hq, total, d))
    k = rng.standard_normal((Hk, total, d))
    v = rng.standard_normal((Hk, total, d))
    if spare:
        for x in (q, k, v):
            x[:, total - spare:] = np.nan
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q, k, v, cu


def _spans(lengths):
    """(first row, length) of each sequence, from the lengths themselves."""
    return [(sum(lengths[:s]), n) for s, n in enumerate(lengths)]


def test_block_boundaries_follow_cu():
    """Level-0 node j of sequence s is the mean of rows [cu[s] + 64j,
    min(cu[s] + 64(j+1), cu[s+1])); the root is the mean of all its rows.
    Rows no sequence owns (NaN here) are never read."""
    lengths = [70, 0, 130, 133, 1]
    q, k, v, cu = _inputs(lengths, spare=7)
    out = reference.packed_forward(q, k, v, cu, 192, BLOCK, 2, 2)
    for s, (a, n) in enumerate(_spans(lengths)):
        lv = out["levels"][s]
        if n == 0:
            assert lv == []
            continue
        nb = -(-n // BLOCK)
        assert lv[0].shape[2] == nb
        for j in range(nb):
            rows = k[:, a + BLOCK * j:a + min(BLOCK * (j + 1), n)]
            np.testing.assert_allclose(lv[0][0, :, j], rows.mean(axis=1), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lv[-1][0, :, 0], k[:, a:a + n].mean(axis=1), rtol=0, atol=1e-12)
    total = q.shape[1]
    assert np.isfinite(out["o"][:, :sum(lengths)]).all()
    assert np.isnan(out["o"][:, sum(lengths):total]).all()


def test_routes_stay_inside_the_sequence():
    """Query block i of a sequence routes to blocks j <= i of the same
    sequence: j < i kept once, i (the diagonal) present; rows of query blocks
    past the sequence's end hold -1 only."""
    lengths = [700, 64, 65, 1000]
    q, k, v, cu = _inputs(lengths, seed=1)
    K = 3
    out = reference.packed_forward(q, k, v, cu, 1024, BLOCK, 2, K)
    sel = out["sel"]
    assert sel.shape == (4, 2, 16, K + 1)
    for s, (a, n) in enumerate(_spans(lengths)):
        nqb = -(-n // BLOCK)
        for hk in range(2):
            for i in range(16):
                row = [int(x) for x in sel[s, hk, i]]
                if i >= nqb:
                    assert row == [-1] * (K + 1)
                    continue
                ids = [x for x in row if x >= 0]
                assert ids[-1] == i and len(set(ids)) == len(ids)
                assert all(0 <= x < i for x in ids[:-1])
                assert ids[:-1] == sorted(ids[:-1])
                assert len(ids) == min(K, i) + 1


def _dense_causal(qs, ks, vs, scale):
    """Textbook causal softmax attention of one head: [T, d] each."""
    T = qs.shape[0]
    z = scale * qs @ ks.T
    z[np.triu_indices(T, 1)] = -np.inf
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    return (p @ vs) / p.sum(axis=1, keepdims=True), m[:, 0] + np.log(p.sum(axis=1))


def test_full_budget_is_dense_causal_attention():
    """With K at least every sequence's block count, every earlier block is
    kept, so each sequence gets plain causal attention over its own rows."""
    lengths = [130, 1, 257, 64]
    q, k, v, cu = _inputs(lengths, spare=5, seed=2)
    out = reference.packed_forward(q, k, v, cu, 320, BLOCK, 2, 5)
    scale = 1.0 / math.sqrt(q.shape[2])
    for a, n in _spans(lengths):
        for h in range(4):
            o, lse = _dense_causal(q[h, a:a + n], k[h // 2, a:a + n], v[h // 2, a:a + n], scale)
            np.testing.assert_allclose(out["o"][h, a:a + n], o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(out["lse"][h, a:a + n], lse, rtol=0, atol=1e-12)


def test_sequences_are_isolated():
    """Changing every row of the other sequences leaves a sequence's pooled
    keys, routes, outputs and log-sum-exp bit for bit unchanged."""
    lengths = [300, 200, 450]
    q, k, v, cu = _inputs(lengths, seed=3)
    base = reference.packed_forward(q, k, v, cu, 512, BLOCK, 2, 2)
    a, n = _spans(lengths)[1]
    rng = np.random.default_rng(9)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        mask = np.ones(x.shape[1], bool)
        mask[a:a + n] = False
        x[:, mask] = rng.standard_normal(x[:, mask].shape) * 5
    alt = reference.packed_forward(q2, k2, v2, cu, 512, BLOCK, 2, 2)
    assert np.array_equal(base["sel"][1], alt["sel"][1])
    assert np.array_equal(base["o"][:, a:a + n], alt["o"][:, a:a + n])
    assert np.array_equal(base["lse"][:, a:a + n], alt["lse"][:, a:a + n])
    for x, y in zip(base["levels"][1], alt["levels"][1]):
        assert np.array_equal(x, y)
    assert not np.array_equal(base["sel"][0], alt["sel"][0]) or \
        not np.array_equal(base["o"][:, :a], alt["o"][:, :a])


@pytest.mark.parametrize("n", [256, 200])
def test_equal_lengths_match_the_dense_batch(n):
    """S sequences of one length packed back to back give the dense batch
    [S, H, n, d] results: the layouts are the same data."""
    S = 3
    q, k, v, cu = _inputs([n] * S, seed=4)
    out = reference.packed_forward(q, k, v, cu, n, BLOCK, 2, 2)
    qd = q.reshape(4, S, n, -1).transpose(1, 0, 2, 3)
    kd = k.reshape(2, S, n, -1).transpose(1, 0, 2, 3)
    vd = v.reshape(2, S, n, -1).transpose(1, 0, 2, 3)
    lv = reference.build_pyramid(kd, BLOCK, 2)
    sel, _ = reference.select(qd, lv, n, BLOCK, 2, 2)
    o, lse = reference.attention(qd, kd, vd, sel, BLOCK)
    assert np.array_equal(out["sel"], sel)
    np.testing.assert_allclose(out["o"], o.transpose(1, 0, 2, 3).reshape(4, S * n, -1), rtol=0,
                               atol=1e-12)
    np.testing.assert_allclose(out["lse"], lse.transpose(1, 0, 2).reshape(4, S * n), rtol=0,
                               atol=1e-12)


_orig_spans = reference.packed_spans


def _spans_shifted_start(cu):
    return [(a + 1, max(n - 1, 0)) for a, n in _orig_spans(cu)]


def _spans_leak_previous(cu):
    out = []
    for a, n in _orig_spans(cu):   # each sequence also sees the one before it
        b = out[-1][0] if out else a
        out.append((b, a + n - b))
    return out


@pytest.mark.parametrize("mutant", [_spans_shifted_start, _spans_leak_previous])
def test_planted_packing_mistake_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(reference, "packed_spans", mutant)
    failed = 0
    for pin in (test_block_boundaries_follow_cu, test_full_budget_is_dense_causal_attention,
                test_routes_stay_inside_the_sequence):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1
