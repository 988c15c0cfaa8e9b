"""GPU parity of pyr_select_attn, selection and attention in one call (PISA
abstract: the kernels fuse routing with LogSumExp scoring; PHBA §A.1.3: the
forward works straight from the query-centric routes), through the C ABI.

Where the library runs one fused launch (bfloat16 prefill, four query heads
per KV head, branching * (top_k + 1) <= 192):
  * the route rows pass the oracle's tie-tolerant walk along the device trace
    with no failure; rows that differ from pyr_select_topk's (score rounding
    in another order) pass it as well;
  * the trace's kept scores match pyr_select_topk's within 1e-4 wherever the
    kept ids agree;
  * o and lse equal, bit for bit, what pyr_block_sparse_attn computes over the
    route rows the call wrote, and match the oracle's attention over them
    (bf16: 2e-2 / 1e-3).
Everywhere else (two query heads per KV head, float32, a wider candidate set,
decode) the call runs the two kernels in turn and every output equals the
separate calls' bit for bit.  A packed batch through the fused launch leaves
rows no sequence owns untouched and blanks route rows past each sequence.
"""

import numpy as np
import pytest
import torch

import hierarchical_block_sparse_amd as H
from hierarchical_block_sparse_amd import workloads as W
from oracle import reference
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu
C = W.Config

CASES = [
    # name, dtype, d, Hq, Hk, Tq, Tk, b, K, planted, one launch
    ("fused_d128", torch.bfloat16, 128, 8, 2, 64 * 37 + 19, 64 * 37 + 19, 4, 8, 4, True),
    ("fused_d64_b2", torch.bfloat16, 64, 8, 2, 64 * 29 + 1, 64 * 29 + 1, 2, 6, 2, True),
    ("fused_b2_k95", torch.bfloat16, 64, 4, 1, 64 * 130 + 7, 64 * 130 + 7, 2, 95, 4, True),
    ("two_launch_b4_k48", torch.bfloat16, 128, 4, 1, 64 * 70 + 3, 64 * 70 + 3, 4, 48, 4, False),
    ("two_launch_g2", torch.bfloat16, 128, 4, 2, 64 * 21 + 40, 64 * 21 + 40, 4, 8, 4, False),
    ("two_launch_f32", torch.float32, 64, 8, 2, 64 * 20 + 5, 64 * 20 + 5, 2, 4, 0, False),
    ("two_launch_decode", torch.bfloat16, 128, 8, 2, 1, 64 * 40 + 9, 4, 8, 4, False),
]


def _outputs(p, q):
    sel = H.alloc_sel(p)
    tids, tsc = H.alloc_trace(p)
    o = torch.empty_like(q)
    lse = torch.empty(p.lse_shape, dtype=torch.float32, device=q.device)
    return sel, tids, tsc, o, lse


def _separate(p, q, k, v, pyr):
    sel, tids, tsc, o, lse = _outputs(p, q)
    H.pyr_select_topk(p, q, pyr, sel, tids, tsc)
    H.pyr_block_sparse_attn(p, q, k, v, sel, o, lse, H.alloc_workspace(p))
    return sel, tids, tsc, o, lse


def _fused(p, q, k, v, pyr):
    sel, tids, tsc, o, lse = _outputs(p, q)
    H.pyr_select_attn(p, q, k, v, pyr, sel, o, lse, H.alloc_workspace(p), tids, tsc)
    return sel, tids, tsc, o, lse


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _attend_over(p, q, k, v, sel):
    o = torch.empty_like(q)
    lse = torch.empty(p.lse_shape, dtype=torch.float32, device=q.device)
    H.pyr_block_sparse_attn(p, q, k, v, sel, o, lse, H.alloc_workspace(p))
    return o, lse


def _trace_scores_agree(tids_a, tsc_a, tids_b, tsc_b):
    """Max |score difference| over the trace rows whose kept ids agree."""
    ia, ib = tids_a.cpu().numpy(), tids_b.cpu().numpy()
    sa, sb = tsc_a.cpu().numpy(), tsc_b.cpu().numpy()
    same = (ia == ib).all(axis=-1)            # [..., L]
    xa, xb = sa[same][:, :-1], sb[same][:, :-1]   # kept scores (the last slot: best rejected)
    both = np.isfinite(xa) & np.isfinite(xb)
    assert np.array_equal(np.isnan(xa), np.isnan(xb))
    return float(np.abs(xa[both] - xb[both]).max()) if both.any() else 0.0, int(same.sum())


@pytest.mark.parametrize("name,dtype,d,Hq,Hk,Tq,Tk,b,K,planted,fused", CASES,
                         ids=[c[0] for c in CASES])
def test_select_attn(name, dtype, d, Hq, Hk, Tq, Tk, b, K, planted, fused):
    cfg = C(name, 1 if Tq > 1 else 2, Hq, Hk, Tq, Tk, d, dtype, b, K, planted, seed=81)
    q, k, v = W.make_inputs(cfg, "cuda")
    p = GH.problem(cfg)
    GH.log(f"case {name}: B={cfg.batch} Hq={Hq} Hk={Hk} Tq={Tq} Tk={Tk} d={d} b={b} K={K}, "
           f"{'one launch' if fused else 'two launches'}")
    pyr = H.alloc_pyramid(p)
    H.pyr_build_pyramid(p, k, pyr)
    sel_s, tids_s, tsc_s, o_s, lse_s = _separate(p, q, k, v, pyr)
    sel_f, tids_f, tsc_f, o_f, lse_f = _fused(p, q, k, v, pyr)
    torch.cuda.synchronize()

    if not fused:
        assert torch.equal(sel_f, sel_s) and torch.equal(tids_f, tids_s)
        assert torch.equal(_bits(tsc_f), _bits(tsc_s))
        assert torch.equal(_bits(o_f), _bits(o_s)) and torch.equal(lse_f, lse_s)
        GH.log("  every output equals the separate calls' bit for bit")
        return

    # the attention half: bit for bit the separate kernel's over the same routes
    o2, lse2 = _attend_over(p, q, k, v, sel_f)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o_f), _bits(o2)) and torch.equal(lse_f, lse2)

    # the selection half against the oracle
    q64, k64, v64 = GH.f64(q), GH.f64(k), GH.f64(v)
    lv = reference.build_pyramid(k64, 64, b)
    levels_of = lambda bi, hk: [x[bi, hk] for x in lv]  # noqa: E731
    units = GH.all_units(cfg)
    counts, worst, fails = GH.judge_selection(q64, levels_of, cfg, sel_f, tids_f, units)
    assert not fails, fails
    differ = [u for u in units if not torch.equal(sel_f[u], sel_s[u])]
    if differ:   # the separate route of those units must pass the walk as well
        c2, _, f2 = GH.judge_selection(q64, levels_of, cfg, sel_s, tids_s, differ)
        assert not f2, f2
    e_sc, n_rows = _trace_scores_agree(tids_f, tsc_f, tids_s, tsc_s)
    assert e_sc <= GH.SEL_TOL
    e_o, e_l = GH.judge_attention(q64, k64, v64, cfg, sel_f.cpu().numpy(), o_f, lse_f, units)
    GH.log(f"  selection {counts} (worst near-tie gap {worst:.1e}); {len(differ)} of "
           f"{len(units)} route rows differ from the separate call; kept scores within "
           f"{e_sc:.1e} on {n_rows} trace rows; O err {e_o:.2e}, LSE err {e_l:.2e}")
    tol_o, tol_l = GH.TOL[dtype]
    assert e_o <= tol_o and e_l <= tol_l


LENGTHS = [1, 63, 64, 65, 0, 700, 2000, 130, 1500, 129]
MAX_LEN = 2048
SPARE = 37
SENTINEL = 7.0


def test_select_attn_packed():
    cfg = C("fused_packed", 1, 8, 2, MAX_LEN, MAX_LEN, 128, torch.bfloat16, 4, 8, 4, seed=82)
    q, k, v, cu = W.make_packed_inputs(cfg, LENGTHS, "cuda", spare_rows=SPARE)
    p = H.problem_for_packed(q, k, cu, MAX_LEN, cfg.branching, cfg.top_k)
    GH.log(f"packed: {len(LENGTHS)} sequences, {p.total_len} rows, one launch")
    pyr = torch.zeros(H.pyramid_shape(p), dtype=torch.float32, device="cuda")
    H.pyr_build_pyramid(p, k, pyr)
    sel_s, tids_s, _, _, _ = _separate(p, q, k, v, pyr)
    sel_f, tids_f, _, o_f, lse_f = _outputs(p, q)
    o_f.fill_(SENTINEL)
    lse_f.fill_(SENTINEL)
    H.pyr_select_attn(p, q, k, v, pyr, sel_f, o_f, lse_f, H.alloc_workspace(p), tids_f, None)
    o2, lse2 = _attend_over(p, q, k, v, sel_f)
    torch.cuda.synchronize()
    used = sum(LENGTHS)
    assert bool((o_f[:, used:] == SENTINEL).all()) and bool((lse_f[:, used:] == SENTINEL).all())
    assert torch.equal(_bits(o_f[:, :used]), _bits(o2[:, :used]))
    assert torch.equal(lse_f[:, :used], lse2[:, :used])
    q64, k64, v64 = GH.f64(q), GH.f64(k), GH.f64(v)
    counts = {"exact": 0, "near_tie": 0, "fail": 0}
    err_o = err_l = 0.0
    a = 0
    for s, n in enumerate(LENGTHS):
        nqb = -(-n // 64)
        assert bool((sel_f[s, :, nqb:] == -1).all()), f"sequence {s}: rows past its end"
        if n == 0:
            continue
        cs = cfg.with_(batch=1, q_len=n, kv_len=n)
        lv = reference.build_pyramid(k64[None, :, a:a + n], 64, cfg.branching)
        lv_bh = {hk: [x[0, hk] for x in lv] for hk in range(cfg.n_kv_heads)}
        units = [(0, hk, i) for hk in range(cfg.n_kv_heads) for i in range(nqb)]
        qs = q64[None, :, a:a + n]
        c, _, fails = GH.judge_selection(qs, lambda bi, hk: lv_bh[hk], cs,
                                         sel_f[s:s + 1, :, :nqb], tids_f[s:s + 1, :, :nqb], units)
        assert not fails, f"sequence {s}: {fails}"
        for key in counts:
            counts[key] += c[key]
        eo, el = GH.judge_attention(qs, k64[None, :, a:a + n], v64[None, :, a:a + n], cs,
                                    sel_f[s:s + 1].cpu().numpy(), o_f[:, a:a + n].unsqueeze(0),
                                    lse_f[:, a:a + n].unsqueeze(0), units)
        err_o, err_l = max(err_o, eo), max(err_l, el)
        a += n
    n_diff = int((sel_f != sel_s).any(dim=-1).sum())
    GH.log(f"  selection {counts}; {n_diff} route rows differ from the separate call; "
           f"O err {err_o:.2e} LSE err {err_l:.2e}")
    tol_o, tol_l = GH.TOL[torch.bfloat16]
    assert err_o <= tol_o and err_l <= tol_l
