"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
judge it with the oracle (float64, CPU).  The oracle only ever sees the
generated inputs (copied back from the device byte for byte); the device
results are only ever judged."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import hierarchical_block_sparse_amd as H
from hierarchical_block_sparse_amd import workloads as W
from oracle import check, reference

TOL = {  # (O max-abs, LSE max-abs) per input dtype
    torch.bfloat16: (2e-2, 1e-3),
    torch.float32: (1e-4, 1e-5),
}
SEL_TOL = 1e-4  # near-tie gap on the natural-log LSE score


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def problem(cfg: W.Config) -> H.Problem:
    return H.Problem(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.q_len,
                     cfg.kv_len, cfg.branching, cfg.top_k, cfg.dtype)


def run_device(cfg: W.Config, q, k, v, trace=True, sel_in=None, fused=False):
    """Build, select (with trace) and attend on the device.  With sel_in the
    attention runs over those route rows instead of the device selection;
    with fused, selection and attention run in one pyr_select_attn call."""
    p = problem(cfg)
    pyr = H.alloc_pyramid(p)
    H.pyr_build_pyramid(p, k, pyr)
    sel = H.alloc_sel(p)
    tids, tsc = H.alloc_trace(p) if trace else (None, None)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if fused:
        assert sel_in is None
        H.pyr_select_attn(p, q, k, v, pyr, sel, o, lse, H.alloc_workspace(p), tids, tsc)
    else:
        H.pyr_select_topk(p, q, pyr, sel, tids, tsc)
        route = sel if sel_in is None else sel_in.to(torch.int32).to(q.device).contiguous()
        H.pyr_block_sparse_attn(p, q, k, v, route, o, lse, H.alloc_workspace(p))
    torch.cuda.synchronize()
    if trace:
        check_fast_selection(p, q, k, v, pyr, sel, tids, o if fused else None,
                             lse if fused else None)
    return dict(pyr=pyr, sel=sel, tids=tids, tsc=tsc, o=o, lse=lse)


def check_fast_selection(p, q, k, v, pyr, sel, tids, o=None, lse=None):
    """Without a score trace (and without a fallback) the selection ranks
    each level by counting on all its waves instead of recording scores and
    the margin on one: its route rows and trace ids must be those of the
    traced selection, bit for bit -- with the id trace and without any trace.
    With o and lse (a fused call) the fused launch without traces must also
    give the same outputs."""
    sel_f, sel_n = H.alloc_sel(p), H.alloc_sel(p)
    tids_f = torch.full_like(tids, -7)
    if o is None:
        H.pyr_select_topk(p, q, pyr, sel_f, tids_f, None)
        H.pyr_select_topk(p, q, pyr, sel_n)
    else:
        o_n, lse_n = torch.empty_like(o), torch.empty_like(lse)
        H.pyr_select_attn(p, q, k, v, pyr, sel_f, torch.empty_like(o), None,
                          H.alloc_workspace(p), tids_f, None)
        H.pyr_select_attn(p, q, k, v, pyr, sel_n, o_n, lse_n, H.alloc_workspace(p))
    torch.cuda.synchronize()
    assert torch.equal(sel_f, sel), "route rows with the id trace only differ from the traced ones"
    assert torch.equal(sel_n, sel), "route rows without traces differ from the traced ones"
    assert torch.equal(tids_f, tids), "trace ids without the score trace differ"
    if o is not None:
        assert torch.equal(o_n.view(torch.int16), o.view(torch.int16))
        assert torch.equal(lse_n, lse)


def oracle_levels(k64, cfg, bh=None):
    """Oracle pyramid levels, optionally for a subset of (batch, kv_head) pairs."""
    if bh is None:
        return reference.build_pyramid(k64, cfg.block, cfg.branching)
    out = {}
    for (bi, hk) in bh:
        lv = reference.build_pyramid(k64[bi:bi + 1, hk:hk + 1], cfg.block, cfg.branching)
        out[(bi, hk)] = [x[0, 0] for x in lv]
    return out


def check_split_plane(dev_pyr):
    """Plane 1 of a two-plane (bf16 problem) pyramid must hold, bit for bit,
    hi = bf16(x) and lo = bf16(x - hi) of plane 0's fp32 means x (round to
    nearest even, as torch converts)."""
    if dev_pyr.shape[2] < 2:
        return
    x = dev_pyr[:, :, 0]
    split = dev_pyr[:, :, 1].contiguous().view(torch.bfloat16)      # [..., 2d]
    d = x.shape[-1]
    hi_ref = x.to(torch.bfloat16)
    lo_ref = (x - hi_ref.float()).to(torch.bfloat16)
    assert torch.equal(split[..., :d].view(torch.int16), hi_ref.view(torch.int16))
    assert torch.equal(split[..., d:].view(torch.int16), lo_ref.view(torch.int16))


def check_pyramid(dev_pyr, levels, k_absmax):
    """dev_pyr: [B, Hk, planes, nodes, d] from the device; levels: the
    oracle's per-level means.  Returns (max abs error of plane 0, tolerance)
    after checking the split plane."""
    check_split_plane(dev_pyr)
    dev = dev_pyr[:, :, 0].detach().cpu().numpy().astype(np.float64)
    ref = reference.concat_levels(levels)
    err = np.abs(dev - ref).max() if ref.size else 0.0
    return err, 1e-5 * max(k_absmax, 1.0)


def judge_selection(q64, levels_of, cfg, sel, tids, units):
    """Tie-tolerant check of the device route rows for the listed units.
    levels_of(bi, hk) -> per-level [n_l, d] float64 pooled keys."""
    scale = 1.0 / math.sqrt(cfg.head_dim)
    sel = sel.cpu().numpy()
    tids = tids.cpu().numpy() if tids is not None else None
    counts = {"exact": 0, "near_tie": 0, "fail": 0}
    worst, fails = 0.0, []
    for (bi, hk, i) in units:
        toks, diag = reference.unit_tokens(i, cfg.q_len, cfg.kv_len, cfg.block)
        rows = reference.unit_rows(q64, bi, hk, cfg.group, toks)
        kept = None if tids is None else [list(tids[bi, hk, i, lvl]) for lvl in range(tids.shape[3])]
        status, info = check.check_unit(rows, levels_of(bi, hk), diag, cfg.branching, cfg.top_k,
                                        scale, sel[bi, hk, i], kept, tol=SEL_TOL)
        counts[status] += 1
        if status == "near_tie":
            worst = max(worst, info["gap"])
        if status == "fail" and len(fails) < 5:
            fails.append(((bi, hk, i), info))
    return counts, worst, fails


def oracle_sel_rows(q64, levels_of, cfg, units):
    """Oracle route rows for the listed units: dict unit -> list (K+1, -1 padded)."""
    scale = 1.0 / math.sqrt(cfg.head_dim)
    out = {}
    for (bi, hk, i) in units:
        toks, diag = reference.unit_tokens(i, cfg.q_len, cfg.kv_len, cfg.block)
        rows = reference.unit_rows(q64, bi, hk, cfg.group, toks)
        us = reference.select_unit(rows, levels_of(bi, hk), diag, cfg.branching, cfg.top_k, scale)
        out[(bi, hk, i)] = us.sel + [-1] * (cfg.top_k + 1 - len(us.sel))
    return out


def judge_attention(q64, k64, v64, cfg, route, o_dev, lse_dev, units, kv_index=None):
    """Max abs error of device O and LSE against the oracle over `route` rows
    (numpy [B, Hk, nqb, K+1]) for the listed units.  kv_index maps a unit's
    (bi, hk) to the index of its K/V slab in k64/v64 when those hold a subset."""
    scale = 1.0 / math.sqrt(cfg.head_dim)
    o_dev = o_dev.detach().float().cpu().numpy()
    lse_dev = lse_dev.detach().cpu().numpy()
    pos = reference.query_positions(cfg.q_len, cfg.kv_len)
    e_o = e_l = 0.0
    for (bi, hk, i) in units:
        toks, _ = reference.unit_tokens(i, cfg.q_len, cfg.kv_len, cfg.block)
        blocks = [int(x) for x in route[bi, hk, i] if x >= 0]
        kb, kh = kv_index(bi, hk) if kv_index else (bi, hk)
        for h in range(hk * cfg.group, (hk + 1) * cfg.group):
            rows = q64[bi, h, toks, :]
            oo, ll = reference.attend_rows(rows, pos[toks], k64[kb, kh], v64[kb, kh], blocks,
                                           cfg.block, scale)
            e_o = max(e_o, float(np.abs(o_dev[bi, h, toks, :] - oo).max()))
            e_l = max(e_l, float(np.abs(lse_dev[bi, h, toks] - ll).max()))
    return e_o, e_l


def all_units(cfg):
    nqb = reference.num_query_blocks(cfg.q_len, cfg.kv_len, cfg.block)
    return [(bi, hk, i) for bi in range(cfg.batch) for hk in range(cfg.n_kv_heads)
            for i in range(nqb)]
