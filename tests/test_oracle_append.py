"""Pins of the oracle's decode-time pyramid maintenance (oracle/reference.py,
append_pyramid; reading R15), on the CPU: the running-sum update must equal a
fresh build of the longer sequence (build_pyramid takes every node's mean
straight from its tokens, a different formulation), for single-token and
multi-token appends, across block boundaries and level-count changes, and when
chained token by token; a planted mistake in the update fails."""

import numpy as np
import pytest

import oracle.reference as ref


def _keys(seed, T, B=1, Hk=2, d=4):
    return np.random.default_rng(seed).standard_normal((B, Hk, T, d))


def _close(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert x.shape == y.shape
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


@pytest.mark.parametrize("old,new,b", [
    (1, 2, 2), (63, 64, 2), (64, 65, 4), (100, 101, 3), (64 * 16, 64 * 16 + 1, 4),
    (64 * 4 + 5, 64 * 9 + 30, 2), (70, 70, 4), (5, 64 * 20, 4), (64 * 8, 64 * 8 + 64, 16),
])
def test_append_equals_fresh_build(old, new, b):
    k = _keys(old * 7 + new, new)
    block = 64
    got = ref.append_pyramid(ref.build_pyramid(k[:, :, :old], block, b), k, old, block, b)
    _close(got, ref.build_pyramid(k, block, b))


def test_chained_single_token_appends():
    k = _keys(3, 64 * 3 + 10, d=3)
    block, b = 64, 2
    lv = ref.build_pyramid(k[:, :, :100], block, b)
    for t in range(101, k.shape[2] + 1):
        lv = ref.append_pyramid(lv, k[:, :, :t], t - 1, block, b)
    _close(lv, ref.build_pyramid(k, block, b))


def test_untouched_nodes_keep_their_values():
    k = _keys(4, 64 * 10 + 3)
    block, b = 64, 2
    old = ref.build_pyramid(k[:, :, :64 * 10], block, b)
    new = ref.append_pyramid(old, k, 64 * 10, block, b)
    # level 0: blocks 0..9 are untouched, block 10 is new
    assert np.array_equal(new[0][:, :, :10], old[0])
    # level 1: nodes 0..4 cover blocks 0..9 only
    assert np.array_equal(new[1][:, :, :5], old[1][:, :, :5])


def test_planted_mistake_is_caught():
    """Updating a node with the plain mean of its new tokens (dropping the old
    tokens' weight) must not match the fresh build."""
    k = _keys(5, 64 * 2 + 9)
    block, b = 64, 2
    old_len = 64 * 2 + 3
    lv = ref.build_pyramid(k[:, :, :old_len], block, b)
    got = ref.append_pyramid(lv, k, old_len, block, b)
    bad = [x.copy() for x in got]
    bad[0][:, :, 2] = k[:, :, old_len:].mean(axis=2)
    fresh = ref.build_pyramid(k, block, b)
    _close(got, fresh)
    assert not np.allclose(bad[0], fresh[0])
