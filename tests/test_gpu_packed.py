"""GPU parity of packed batches (reading R16; PHBA §A.1.1-§A.1.2), through the
C ABI.

A packed batch of mixed lengths (empty, single-token, ragged and
block-aligned sequences, followed by rows of NaN that no sequence owns) runs
through build, select and attend.  For every sequence:
  * the pyramid's valid nodes, the route rows, the output and the log-sum-exp
    equal, bit for bit, those of the dense path on that sequence alone
    (batch 1, its own length);
  * the valid pyramid nodes match the float64 oracle (max abs error
    <= 1e-5 max|k|), the route rows pass the oracle's tie-tolerant walk, and
    the output and log-sum-exp match the oracle's attention over the device
    routes (bf16: 2e-2 / 1e-3, fp32: 1e-4 / 1e-5);
  * route rows past the sequence's end hold -1 only, and rows of o and lse
    that no sequence owns keep what they held before the call.
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

LENGTHS = [1, 63, 64, 65, 0, 700, 2000, 130, 1500, 129]
MAX_LEN = 2048
SPARE = 37
SENTINEL = 7.0

CASES = [
    # name, dtype, d, Hq, Hk, b, K, planted
    ("bf16_d128_g4", torch.bfloat16, 128, 8, 2, 4, 8, 4),
    ("bf16_d64_g2", torch.bfloat16, 64, 4, 2, 2, 6, 2),
    ("bf16_d128_g1", torch.bfloat16, 128, 2, 2, 4, 8, 4),
    ("f32_d64_g2", torch.float32, 64, 4, 2, 2, 4, 2),
]


def _dense_problem(cfg, n):
    return H.Problem(1, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, n, n, cfg.branching,
                     cfg.top_k, cfg.dtype)


def _valid_sizes(n, b):
    return reference.level_sizes(-(-n // 64), b)


@pytest.mark.parametrize("name,dtype,d,Hq,Hk,b,K,planted", CASES, ids=[c[0] for c in CASES])
def test_packed_batch(name, dtype, d, Hq, Hk, b, K, planted):
    cfg = C(name, 1, Hq, Hk, MAX_LEN, MAX_LEN, d, dtype, b, K, planted, seed=61)
    q, k, v, cu = W.make_packed_inputs(cfg, LENGTHS, "cuda", spare_rows=SPARE)
    p = H.problem_for_packed(q, k, cu, MAX_LEN, b, K)
    GH.log(f"case {name}: {len(LENGTHS)} sequences, total {p.total_len} rows, "
           f"levels {H.pyr_num_levels(p)}")
    pyr = torch.zeros(H.pyramid_shape(p), dtype=torch.float32, device="cuda")
    H.pyr_build_pyramid(p, k, pyr)
    sel = H.alloc_sel(p)
    tids, tsc = H.alloc_trace(p)
    H.pyr_select_topk(p, q, pyr, sel, tids, tsc)
    o = torch.full_like(q, SENTINEL)
    lse = torch.full(p.lse_shape, SENTINEL, dtype=torch.float32, device="cuda")
    H.pyr_block_sparse_attn(p, q, k, v, sel, o, lse, H.alloc_workspace(p))
    torch.cuda.synchronize()

    used = sum(LENGTHS)
    assert bool((o[:, used:] == SENTINEL).all()) and bool((lse[:, used:] == SENTINEL).all())
    nqb_max = H.pyr_num_query_blocks(p)
    L = H.pyr_num_levels(p)
    q64, k64, v64 = GH.f64(q), GH.f64(k), GH.f64(v)
    err_p = err_o = err_l = 0.0
    counts = {"exact": 0, "near_tie": 0, "fail": 0}
    a = 0
    for s, n in enumerate(LENGTHS):
        nqb = -(-n // 64)
        assert bool((sel[s, :, nqb:] == -1).all()), f"sequence {s}: rows past its end"
        if n == 0:
            a += n
            continue
        # the dense path on the sequence alone gives the same bits
        pd = _dense_problem(cfg, n)
        qs, ks, vs = (x[:, a:a + n].unsqueeze(0).contiguous() for x in (q, k, v))
        dpyr = H.alloc_pyramid(pd)
        H.pyr_build_pyramid(pd, ks, dpyr)
        dsel = H.alloc_sel(pd)
        H.pyr_select_topk(pd, qs, dpyr, dsel)
        do = torch.empty_like(qs)
        dl = torch.empty(qs.shape[:3], dtype=torch.float32, device="cuda")
        H.pyr_block_sparse_attn(pd, qs, ks, vs, dsel, do, dl, H.alloc_workspace(pd))
        torch.cuda.synchronize()
        assert torch.equal(sel[s, :, :nqb], dsel[0]), f"sequence {s}: routes differ from dense"
        assert torch.equal(o[:, a:a + n].contiguous().view(torch.int16 if dtype == torch.bfloat16
                                                            else torch.int32),
                           do[0].view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
        assert torch.equal(lse[:, a:a + n], dl[0])
        sizes = _valid_sizes(n, b)
        for lvl, m in enumerate(sizes):
            op, od = H.pyr_level_offset(p, lvl), H.pyr_level_offset(pd, lvl)
            assert torch.equal(pyr[s, :, :, op:op + m], dpyr[0, :, :, od:od + m]), \
                f"sequence {s} level {lvl}"
        # and the oracle agrees; levels above the sequence's root repeat the root
        cs = cfg.with_(batch=1, q_len=n, kv_len=n)
        lv = reference.build_pyramid(k64[None, :, a:a + n], 64, b)
        for lvl in range(L):
            ref = lv[min(lvl, len(lv) - 1)][0]
            off = H.pyr_level_offset(p, lvl)
            dev = GH.f64(pyr[s, :, 0, off:off + ref.shape[1]])
            err_p = max(err_p, float(np.abs(dev - ref).max()))
        units = [(0, hk, i) for hk in range(Hk) for i in range(nqb)]
        lv_bh = {hk: [x[0, hk] for x in lv] for hk in range(Hk)}
        c, worst, fails = GH.judge_selection(q64[None, :, a:a + n], lambda bi, hk: lv_bh[hk], cs,
                                             sel[s:s + 1, :, :nqb], tids[s:s + 1, :, :nqb], units)
        assert not fails, f"sequence {s}: {fails}"
        for key in counts:
            counts[key] += c[key]
        eo, el = GH.judge_attention(q64[None, :, a:a + n], k64[None, :, a:a + n],
                                    v64[None, :, a:a + n], cs, sel[s:s + 1].cpu().numpy(),
                                    o[:, a:a + n].unsqueeze(0), lse[:, a:a + n].unsqueeze(0),
                                    units)
        err_o, err_l = max(err_o, eo), max(err_l, el)
        a += n
    tol_o, tol_l = GH.TOL[dtype]
    tol_p = 1e-5 * max(float(np.abs(k64[:, :used]).max()), 1.0)
    GH.log(f"  pyramid err {err_p:.2e} (tol {tol_p:.0e}); selection {counts}; "
           f"O err {err_o:.2e} LSE err {err_l:.2e}")
    assert err_p <= tol_p
    assert counts["fail"] == 0
    assert err_o <= tol_o and err_l <= tol_l
    GH.check_split_plane(pyr)


def test_packed_single_sequence_equals_dense_batch():
    """One packed sequence of the full length is the dense batch-1 problem."""
    cfg = C("packed_one", 1, 8, 2, 64 * 24 + 5, 64 * 24 + 5, 128, torch.bfloat16, 4, 8, 4,
            seed=62)
    n = cfg.q_len
    q, k, v, cu = W.make_packed_inputs(cfg, [n], "cuda")
    o, lse, sel, _ = H.forward_packed(q, k, v, cu, n, cfg.branching, cfg.top_k)
    od, ld, seld, _ = H.forward(q[None], k[None], v[None], cfg.branching, cfg.top_k)
    torch.cuda.synchronize()
    assert torch.equal(sel, seld)
    assert torch.equal(o.view(torch.int16), od[0].view(torch.int16))
    assert torch.equal(lse, ld[0])
