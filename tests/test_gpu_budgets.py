"""GPU parity of selection with per-head budgets and the confidence fallback
(reading R17; PHAROS summary), through the C ABI.

  * Budgets equal to K without fallback give the bits of pyr_select_topk.
  * Per-KV-head budgets, with and without the fallback, on the MFMA scorer
    (bf16, G = 4) and the vector scorer (fp32, G = 2): every unit's route row
    equals the oracle's (select_unit_budget) or passes the tie-tolerant walk
    with K_h kept per level and, at the finest level, the count the device's
    fallback decision implies; that decision must agree with the oracle's
    margin (computed in float64 on the device's own candidate set) unless the
    margin lies within 1e-3 of the threshold, where either decision is right.
    The threshold is the median oracle margin, so about half of the scored
    units fall back.
  * Attention over the budget routes matches the oracle (the attention bars).
"""

import math

import numpy as np
import pytest
import torch

import hierarchical_block_sparse_amd as H
from hierarchical_block_sparse_amd import workloads as W
from oracle import check, reference
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu
C = W.Config
AMBIGUOUS = 1e-3


def test_full_budgets_equal_plain_selection():
    cfg = C("budget_plain", 1, 8, 2, 64 * 33 + 5, 64 * 33 + 5, 128, torch.bfloat16, 4, 8, 4,
            seed=71)
    q, k, v = W.make_inputs(cfg, "cuda")
    p = GH.problem(cfg)
    pyr = H.alloc_pyramid(p)
    H.pyr_build_pyramid(p, k, pyr)
    a, b = H.alloc_sel(p), H.alloc_sel(p)
    H.pyr_select_topk(p, q, pyr, a)
    kh = torch.full((cfg.n_kv_heads,), cfg.top_k, dtype=torch.int32, device="cuda")
    H.pyr_select_topk_budgets(p, q, pyr, b, kh, 0, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    H.pyr_select_topk_budgets(p, q, pyr, b, None, cfg.top_k, 1e30)   # F = K: no effect
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _device_kept(tids, bi, hk, i):
    return [list(tids[bi, hk, i, lvl]) for lvl in range(tids.shape[3])]


@pytest.mark.parametrize("name,dtype,d,Hq,Hk,b,K,budgets,fb_k", [
    ("bf16_g4", torch.bfloat16, 128, 8, 2, 4, 8, [3, 6], 7),
    ("bf16_g4_nofb", torch.bfloat16, 128, 8, 2, 4, 8, [2, 8], 0),
    ("f32_g2", torch.float32, 64, 4, 2, 2, 6, [1, 4], 5),
])
def test_budgets_and_fallback(name, dtype, d, Hq, Hk, b, K, budgets, fb_k):
    T = 64 * 40 + 17
    cfg = C(name, 1, Hq, Hk, T, T, d, dtype, b, K, 4, seed=72)
    q, k, v = W.make_inputs(cfg, "cuda")
    p = GH.problem(cfg)
    pyr = H.alloc_pyramid(p)
    H.pyr_build_pyramid(p, k, pyr)
    torch.cuda.synchronize()
    q64, k64, v64 = GH.f64(q), GH.f64(k), GH.f64(v)
    lv = reference.build_pyramid(k64, 64, b)
    scale = 1.0 / math.sqrt(d)
    units = GH.all_units(cfg)
    rows_of = {}
    margins = []
    for (bi, hk, i) in units:
        toks, diag = reference.unit_tokens(i, T, T, 64)
        rows_of[(bi, hk, i)] = reference.unit_rows(q64, bi, hk, cfg.group, toks)
        us = reference.select_unit_budget(rows_of[(bi, hk, i)], [x[bi, hk] for x in lv], diag, b,
                                          budgets[hk], scale)
        if us.margin is not None:
            margins.append(us.margin)
    tau = float(np.median(margins)) if fb_k else 0.0
    kh = torch.tensor(budgets, dtype=torch.int32, device="cuda")
    sel = H.alloc_sel(p)
    tids, tsc = H.alloc_trace(p)
    H.pyr_select_topk_budgets(p, q, pyr, sel, kh, fb_k, tau, tids, tsc)
    torch.cuda.synchronize()
    GH.log(f"case {name}: budgets {budgets}, fallback {fb_k} below margin {tau:.4f}")
    if not fb_k:
        # no fallback: without the score trace the bf16 pass with bounded
        # re-scoring runs, and must keep the same nodes bit for bit
        sel_f = H.alloc_sel(p)
        tids_f = torch.full_like(tids, -7)
        H.pyr_select_topk_budgets(p, q, pyr, sel_f, kh, 0, 0.0, tids_f, None)
        torch.cuda.synchronize()
        assert torch.equal(sel_f, sel) and torch.equal(tids_f, tids)
    sel_h, tids_h = sel.cpu().numpy(), tids.cpu().numpy()
    counts = {"exact": 0, "near_tie": 0, "fail": 0}
    fell = ambiguous = 0
    for (bi, hk, i) in units:
        toks, diag = reference.unit_tokens(i, T, T, 64)
        rows = rows_of[(bi, hk, i)]
        lvb = [x[bi, hk] for x in lv]
        kh_u = budgets[hk]
        dev_kept = _device_kept(tids_h, bi, hk, i)
        n0 = sum(1 for x in dev_kept[0] if x >= 0)
        # the margin on the device's own finest candidate set, in float64
        cand0 = reference.candidates(0, sorted(x for x in dev_kept[1] if x >= 0) if len(lvb) > 1
                                     else [], diag, [x.shape[0] for x in lvb], b)
        dev_fell = False
        if fb_k > kh_u and len(cand0) > kh_u:
            s0 = reference.lse_scores(rows, lvb[0][cand0], scale)
            m = reference.finest_margin(s0, kh_u)
            dev_fell = n0 == min(fb_k, len(cand0)) and n0 != kh_u
            if abs(m - tau) < AMBIGUOUS:
                ambiguous += 1
            else:
                assert dev_fell == (m < tau), f"unit {(bi, hk, i)}: margin {m} vs {tau}"
        fell += dev_fell
        ref = reference.select_unit_budget(rows, lvb, diag, b, kh_u, scale, fb_k, tau)
        status, info = check.check_unit(rows, lvb, diag, b, kh_u, scale, sel_h[bi, hk, i],
                                        dev_kept, tol=GH.SEL_TOL,
                                        k_finest=min(fb_k, len(cand0)) if dev_fell else kh_u,
                                        ref_row=ref.sel if dev_fell == ref.fallback else None,
                                        row_width=K + 1)
        counts[status] += 1
        assert status != "fail", f"unit {(bi, hk, i)}: {info}"
    GH.log(f"  selection {counts}; {fell} units fell back, {ambiguous} near the threshold")
    if fb_k:
        assert fell > 0
    e_o, e_l = GH.judge_attention(q64, k64, v64, cfg, sel_h, *_attend(p, q, k, v, sel), units)
    GH.log(f"  attention over the budget routes: O err {e_o:.2e}, LSE err {e_l:.2e}")
    tol_o, tol_l = GH.TOL[dtype]
    assert e_o <= tol_o and e_l <= tol_l


def _attend(p, q, k, v, sel):
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    H.pyr_block_sparse_attn(p, q, k, v, sel, o, lse, H.alloc_workspace(p))
    torch.cuda.synchronize()
    return o, lse
