"""The oracle's pins are strong enough: each plausible mistake planted in the
oracle (on the CPU, by monkeypatching one of its functions) makes at least one
pin of tests/test_oracle.py fail."""

import math

import numpy as np
import pytest

import oracle.reference as ref
from tests import test_oracle as pins

_orig_lse = ref.lse_scores
_orig_cand = ref.candidates
_orig_topk = ref.top_k_nodes
_orig_attend = ref.attend_rows
_orig_build = ref.build_pyramid


def _lse_no_scale(rows, keys, scale):
    return _orig_lse(rows, keys, 1.0)


def _lse_best_row(rows, keys, scale):
    return (scale * (rows @ keys.T)).max(axis=0)


def _lse_mean_query(rows, keys, scale):
    return scale * (rows.mean(axis=0) @ keys.T)


def _topk_high_index_on_ties(cand, s, top_k):
    order = sorted(range(len(cand)), key=lambda j: (-s[j], -cand[j]))
    return [cand[j] for j in order[:top_k]]


def _cand_with_straddling_ancestor(level, kept_above, diag, sizes, branching):
    out = _orig_cand(level, kept_above, diag, sizes, branching)
    anc = diag // branching ** level
    return out + ([anc] if anc != diag or level > 0 else [])


def _cand_without_ancestor_siblings(level, kept_above, diag, sizes, branching):
    if level == len(sizes) - 1:
        return _orig_cand(level, kept_above, diag, sizes, branching)
    out = []
    for p in kept_above:
        out.extend(ref.children(level + 1, p, sizes, branching))
    return out


def _cand_off_by_one(level, kept_above, diag, sizes, branching):
    out = _orig_cand(level, kept_above, diag, sizes, branching)
    anc = diag // branching ** level
    return [c for c in out if c != anc - 1]


def _attend_no_causal_mask(rows, row_pos, k_bh, v_bh, blocks, block, scale):
    return _orig_attend(rows, np.full_like(row_pos, 10 ** 9), k_bh, v_bh, blocks, block, scale)


def _attend_sqrt_scale(rows, row_pos, k_bh, v_bh, blocks, block, scale):
    return _orig_attend(rows, row_pos, k_bh, v_bh, blocks, block, math.sqrt(scale))


def _build_mean_of_child_means(k, block, branching):
    levels = _orig_build(k, block, branching)
    for lvl in range(1, len(levels)):
        below = levels[lvl - 1]
        for m in range(levels[lvl].shape[2]):
            kids = [c for c in range(m * branching, (m + 1) * branching) if c < below.shape[2]]
            levels[lvl][:, :, m] = below[:, :, kids].mean(axis=2)
    return levels


SEL_CASES = pins._load("hand_selection.json")
ATT_CASES = pins._load("hand_attention.json")


def _run_selection_pins():
    for c in SEL_CASES:
        pins.test_hand_selection(c)
    pins.test_full_budget_equals_dense_causal(37, 4, 2)
    for seed in range(3):
        pins.test_one_level_equals_flat_topk(seed)
    pins.test_zero_queries_pick_lowest_blocks()
    for seed in range(10):
        pins.test_invariants_random(seed)


def _run_attention_pins():
    for c in ATT_CASES:
        pins.test_hand_attention(c)
    pins.test_full_budget_equals_dense_causal(37, 4, 2)
    pins.test_attention_equals_masked_dense()


def _run_pyramid_pins():
    pins.test_pyramid_constant_nodes()
    pins.test_pyramid_ragged_is_token_weighted()


MUTATIONS = [
    ("lse_scores", _lse_no_scale, _run_selection_pins),
    ("lse_scores", _lse_best_row, _run_selection_pins),
    ("lse_scores", _lse_mean_query, _run_selection_pins),
    ("top_k_nodes", _topk_high_index_on_ties, _run_selection_pins),
    ("candidates", _cand_with_straddling_ancestor, _run_selection_pins),
    ("candidates", _cand_without_ancestor_siblings, _run_selection_pins),
    ("candidates", _cand_off_by_one, _run_selection_pins),
    ("attend_rows", _attend_no_causal_mask, _run_attention_pins),
    ("attend_rows", _attend_sqrt_scale, _run_attention_pins),
    ("build_pyramid", _build_mean_of_child_means, _run_pyramid_pins),
]


@pytest.mark.parametrize("name,mutant,pinset", MUTATIONS, ids=lambda x: getattr(x, "__name__", x))
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pinset):
    monkeypatch.setattr(ref, name, mutant)
    with pytest.raises(AssertionError):
        pinset()


def test_unmutated_pins_pass():
    _run_selection_pins()
    _run_attention_pins()
    _run_pyramid_pins()
