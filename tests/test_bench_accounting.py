"""The benchmark's work accounting (algorithmic flops and bytes behind its
roofline figures) against counts taken from the oracle's own selection on
small problems: scored candidates per unit, pyramid geometry and the visible
(query row, key) pairs of the attention.  CPU only."""

import math

import numpy as np
import pytest
import torch

import bench
from hierarchical_block_sparse_amd import workloads as W
from oracle import reference


@pytest.mark.parametrize("n,b", [(1, 2), (5, 2), (32, 2), (33, 4), (512, 4), (2048, 4), (16384, 4),
                                 (100, 3), (4096, 8)])
def test_level_sizes_match_oracle(n, b):
    assert bench._level_sizes(n, b) == reference.level_sizes(n, b)
    assert bench._num_blocks(n * 64 - 3) == reference.num_blocks(n * 64 - 3, 64)


@pytest.mark.parametrize("T,b,K,decode", [(64 * 40, 2, 4, False), (64 * 37, 4, 6, False),
                                          (64 * 100, 3, 5, False), (64 * 90 + 7, 4, 8, True)])
def test_scored_candidates_match_oracle(T, b, K, decode):
    cfg = W.Config("acct", 1, 2, 1, 1 if decode else T, T, 16, torch.float32, b, K, 0, seed=3)
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 1, T, 16))
    q = rng.standard_normal((1, 2, cfg.q_len, 16))
    levels = [x[0, 0] for x in reference.build_pyramid(k, 64, b)]
    scored = 0
    nqb = reference.num_query_blocks(cfg.q_len, T, 64)
    for i in range(nqb):
        toks, diag = reference.unit_tokens(i, cfg.q_len, T, 64)
        rows = reference.unit_rows(q, 0, 0, 2, toks)
        us = reference.select_unit(rows, levels, diag, b, K, 0.25)
        scored += sum(len(c) for c, s in zip(us.cands, us.scores) if s is not None)
    assert bench.scored_candidates(cfg) == scored


@pytest.mark.parametrize("nqb,K", [(20, 4), (33, 8), (7, 16)])
def test_attention_flops_count_visible_pairs(nqb, K):
    T, d, G = 64 * nqb, 32, 2
    cfg = W.Config("acct", 1, G, 1, T, T, d, torch.bfloat16, 4, K, 0, seed=3)
    pos = reference.query_positions(T, T)
    pairs = 0
    for i in range(nqb):
        blocks = list(range(max(0, i - K), i + 1))   # min(K, i) earlier blocks and the diagonal
        for t in range(i * 64, i * 64 + 64):
            pairs += sum(1 for j in blocks for s in range(j * 64, j * 64 + 64) if s <= pos[t])
    flops, byts = bench.attn_work(cfg)
    assert flops == pairs * G * 4 * d
    tiles = sum(min(K, i) + 1 for i in range(nqb))
    assert byts == 2 * G * T * d * 2 + tiles * 2 * 64 * d * 2
    assert math.isclose(bench.attn_work(cfg.with_(batch=3))[0], 3 * flops)


def test_planted_recall_bounds():
    """Every block listed (K >= query blocks) gives recall 1, no block gives 0,
    and listing exactly the planted blocks of each unit gives 1 as well."""
    cfg = W.Config("acct", 2, 4, 2, 64 * 12, 64 * 12, 16, torch.float32, 2, 12, 3, seed=9)
    nqb = 12
    full = torch.tensor(np.broadcast_to(np.arange(13) - 1, (2, 2, nqb, 13)).copy(), dtype=torch.int32)
    assert bench.planted_recall(cfg, full) == 1.0
    assert bench.planted_recall(cfg, torch.full((2, 2, nqb, 13), -1, dtype=torch.int32)) == 0.0
    exact = torch.full((2, 2, nqb, 13), -1, dtype=torch.int32)
    for (bi, hk, i), blocks in W.planted_blocks(cfg).items():
        exact[bi, hk, i, :len(blocks)] = torch.tensor(sorted(blocks), dtype=torch.int32)
    assert bench.planted_recall(cfg, exact) == 1.0
    assert bench.planted_recall(cfg.with_(n_planted=0), full) is None
