"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle.

Every case runs build -> select (with per-level trace) -> attention on the
device and judges:
  * pyramid: max abs error <= 1e-5 * max|k|;
  * selection: every unit either equals the oracle's route row ("exact") or
    differs only through near-ties whose float64 score gap is < 1e-4, checked
    level by level along the device trace; no failures;
  * attention, isolated: the device attention run over the ORACLE's route rows
    against the oracle attention (O max-abs 2e-2 bf16 / 1e-4 fp32, LSE 1e-3 /
    1e-5);
  * end to end: device outputs of the whole path against the oracle for every
    unit whose route row is exact (near-tie units: against the oracle
    attention over the device's route row, which the selection check has just
    shown to be a valid top-K within tolerance).
"""

import math

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
    # tiny fp32 at its full size: B=1 H=2 T=2048 d=64, b=2, K=4 + diagonal
    W.CONFIGS["tiny_fp32"],
    # MHA bf16 with a ragged tail and planted retrieval
    C("mha_ragged", 1, 2, 2, 64 * 40 + 17, 64 * 40 + 17, 128, torch.bfloat16, 4, 8, 4, seed=11),
    # GQA G=4 bf16 (the 128K workload's shape, shortened)
    C("gqa4_8k", 1, 8, 2, 8192, 8192, 128, torch.bfloat16, 4, 16, 8, seed=12),
    # GQA G=8, one KV head (the 1M workload's shape, shortened)
    C("gqa8_4k", 1, 8, 1, 4096, 4096, 128, torch.bfloat16, 4, 16, 16, seed=13),
    # G=8 with (K+1) * G/4 = 82 workgroup visits per key block: the attention
    # reads v through its block-transposed copy in the workspace; d = 64,
    # two KV heads, ragged tail
    C("gqa8_k40_vt", 1, 16, 2, 64 * 72 + 29, 64 * 72 + 29, 64, torch.bfloat16, 4, 40, 8, seed=30),
    # d=64 bf16, G=2, b=3, two batch entries
    C("d64_g2_b3", 2, 4, 2, 64 * 50, 64 * 50, 64, torch.bfloat16, 3, 6, 4, seed=14),
    # odd group size G=3 (generic selection path, one head per workgroup attention)
    C("g3_bf16", 1, 6, 2, 64 * 33 + 5, 64 * 33 + 5, 128, torch.bfloat16, 2, 5, 3, seed=15),
    # fp32 with d=128 and G=2
    C("fp32_d128_g2", 1, 4, 2, 64 * 24, 64 * 24, 128, torch.float32, 4, 3, 0, seed=16),
    # fp32 attention workgroup shapes: four heads of d=64 (8 waves), four heads of
    # d=128 (two workgroups of two heads), three heads (one head per workgroup);
    # ragged tails
    C("fp32_d64_g4", 1, 8, 2, 64 * 21 + 9, 64 * 21 + 9, 64, torch.float32, 2, 6, 0, seed=24),
    C("fp32_d128_g4", 1, 8, 2, 64 * 18 + 40, 64 * 18 + 40, 128, torch.float32, 4, 5, 0, seed=25),
    C("fp32_d128_g3", 1, 6, 2, 64 * 15 + 1, 64 * 15 + 1, 128, torch.float32, 3, 4, 0, seed=26),
    # fp32, eight heads per KV head at d = 128 (four two-head workgroups per
    # unit), K beyond the history: route rows padded with -1
    C("fp32_g8_k_exceeds", 1, 16, 2, 64 * 9 + 33, 64 * 9 + 33, 128, torch.float32, 2, 12, 0, seed=29),
    # decode: 4 sequences, 1 token each at kv_len-1 (ragged last block)
    C("decode_small", 4, 8, 2, 1, 64 * 300 + 5, 128, torch.bfloat16, 4, 16, 8, seed=17),
    C("decode_fp32_g1", 3, 2, 2, 1, 64 * 70, 64, torch.float32, 2, 7, 0, seed=18),
    # decode selection with many more candidates than threads (b*K + b - 1 = 803
    # against 256: the ranking's extra candidates spread by key batch), sixteen
    # query heads per KV head (the whole 16-row tile real), d = 64
    C("decode_g16_d64_k200", 2, 32, 2, 1, 64 * 700 + 3, 64, torch.bfloat16, 4, 200, 8, seed=27),
    # decode, eight heads per KV head, 403 candidates per scored level
    C("decode_g8_k100", 2, 16, 2, 1, 64 * 500 + 40, 128, torch.bfloat16, 4, 100, 8, seed=28),
    # K larger than the number of past blocks everywhere
    C("k_exceeds", 1, 4, 2, 64 * 9, 64 * 9, 128, torch.bfloat16, 2, 12, 0, seed=19),
    # one pyramid level below the root (b >= nb)
    C("one_level", 1, 4, 4, 64 * 12, 64 * 12, 64, torch.bfloat16, 16, 3, 2, seed=20),
]


def _run_case(cfg):
    GH.log(f"case {cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hk={cfg.n_kv_heads} "
           f"Tq={cfg.q_len} Tk={cfg.kv_len} d={cfg.head_dim} {cfg.dtype} b={cfg.branching} K={cfg.top_k}")
    q, k, v = W.make_inputs(cfg, "cuda")
    dev = GH.run_device(cfg, q, k, v)
    q64, k64, v64 = GH.f64(q), GH.f64(k), GH.f64(v)
    levels = GH.oracle_levels(k64, cfg)
    return q, k, v, dev, q64, k64, v64, levels


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_parity(cfg):
    q, k, v, dev, q64, k64, v64, levels = _run_case(cfg)
    # pyramid
    err, tol = GH.check_pyramid(dev["pyr"], levels, float(np.abs(k64).max()))
    GH.log(f"  pyramid max abs err {err:.3e} (tol {tol:.1e})")
    assert err <= tol
    # selection
    units = GH.all_units(cfg)
    lv_of = lambda bi, hk: [x[bi, hk] for x in levels]  # noqa: E731
    counts, worst, fails = GH.judge_selection(q64, lv_of, cfg, dev["sel"], dev["tids"], units)
    GH.log(f"  selection {counts} worst near-tie gap {worst:.2e}")
    assert counts["fail"] == 0, fails
    assert counts["near_tie"] <= max(2, len(units) // 50)
    # attention over the oracle's route rows
    osel = GH.oracle_sel_rows(q64, lv_of, cfg, units)
    route = np.full(tuple(dev["sel"].shape), -1, dtype=np.int64)
    for u, row in osel.items():
        route[u] = row
    iso = GH.run_device(cfg, q, k, v, trace=False, sel_in=torch.from_numpy(route))
    e_o, e_l = GH.judge_attention(q64, k64, v64, cfg, route, iso["o"], iso["lse"], units)
    tol_o, tol_l = GH.TOL[cfg.dtype]
    GH.log(f"  attention (oracle routes) O err {e_o:.3e} LSE err {e_l:.3e}")
    assert e_o <= tol_o and e_l <= tol_l
    # end to end
    dsel = dev["sel"].cpu().numpy()
    e_o, e_l = GH.judge_attention(q64, k64, v64, cfg, dsel, dev["o"], dev["lse"], units)
    GH.log(f"  end to end O err {e_o:.3e} LSE err {e_l:.3e}")
    assert e_o <= tol_o and e_l <= tol_l


def test_full_budget_is_dense_causal():
    """K >= nb - 1: every block <= i is selected and the output is dense causal
    attention (torch SDPA in float64 on the CPU)."""
    cfg = W.CONFIGS["tiny_fp32"].with_(top_k=31, name="tiny_fp32_K31")
    q, k, v = W.make_inputs(cfg, "cuda")
    dev = GH.run_device(cfg, q, k, v)
    sel = dev["sel"].cpu().numpy()
    for i in range(32):
        assert list(sel[0, 0, i]) == list(range(i + 1)) + [-1] * (31 - i)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.cpu().double(), k.cpu().double(), v.cpu().double(), is_causal=True)
    err = (dev["o"].cpu().double() - ref).abs().max().item()
    GH.log(f"  dense causal max err {err:.3e}")
    assert err <= 1e-4


def test_full_budget_bf16_gqa_is_dense_causal():
    cfg = C("dense_bf16", 1, 8, 2, 64 * 10, 64 * 10, 128, torch.bfloat16, 4, 9, 0, seed=21)
    q, k, v = W.make_inputs(cfg, "cuda")
    dev = GH.run_device(cfg, q, k, v)
    kk = k.cpu().double().repeat_interleave(4, dim=1)
    vv = v.cpu().double().repeat_interleave(4, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q.cpu().double(), kk, vv, is_causal=True)
    err = (dev["o"].cpu().double() - ref).abs().max().item()
    GH.log(f"  dense causal bf16 max err {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("K,kvals,want", [
    (1, [5, -5, 1, 1, 2, 3, 0, 9], [5, 7]),
    (2, [5, -5, 1, 1, 2, 3, 0, 9], [4, 5, 7]),
    (3, [5, -5, 1, 1, 2, 3, 0, 9], [0, 4, 5, 7]),
    (1, [5, -5, 1, 1, 2, 2, 0, 9], [4, 7]),        # exact tie -> lower index
])
def test_hand_examples_lifted(K, kvals, want):
    """The hand-worked selections of tests/golden/hand_selection.json lifted to
    64-token blocks: every key of block j is (k_j, 0, ...), the query block's rows
    are (8, 0, ...) (d=64, b=2).  All rows and tokens are equal, so every score
    is the 1-token score shifted by log 64 and exact ties stay exact: the device
    must reproduce the hand results exactly."""
    d, T = 64, 8 * 64
    k = torch.zeros((1, 1, T, d), dtype=torch.bfloat16)
    for j, x in enumerate(kvals):
        k[0, 0, j * 64:(j + 1) * 64, 0] = x
    q = torch.zeros((1, 1, T, d), dtype=torch.bfloat16)
    q[0, 0, 7 * 64:, 0] = 8.0        # scale 1/8: q.k / 8 = k_j as in the hand example
    v = torch.randn((1, 1, T, d)).to(torch.bfloat16)
    cfg = C("lifted", 1, 1, 1, T, T, d, torch.bfloat16, 2, K, 0)
    dev = GH.run_device(cfg, q.cuda(), k.cuda(), v.cuda())
    row = dev["sel"][0, 0, 7].cpu().tolist()
    assert row == want + [-1] * (K + 1 - len(want))


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 129])
def test_short_sequences(T):
    for dtype in (torch.bfloat16, torch.float32):
        cfg = C(f"short{T}", 1, 4, 2, T, T, 128, dtype, 4, 2, 0, seed=30 + T)
        q, k, v = W.make_inputs(cfg, "cuda")
        dev = GH.run_device(cfg, q, k, v)
        q64, k64, v64 = GH.f64(q), GH.f64(k), GH.f64(v)
        levels = GH.oracle_levels(k64, cfg)
        sel, _ = reference.select(q64, levels, T, 64, 4, 2)
        assert np.array_equal(dev["sel"].cpu().numpy(), sel)
        o, lse = reference.attention(q64, k64, v64, sel, 64)
        tol_o, tol_l = GH.TOL[dtype]
        assert np.abs(dev["o"].float().cpu().numpy() - o).max() <= tol_o
        assert np.abs(dev["lse"].cpu().numpy() - lse).max() <= tol_l


def test_empty_inputs_are_noops():
    p = H.Problem(0, 4, 2, 128, 128, 128, 4, 4, torch.bfloat16)
    e = torch.empty((0, 4, 128, 128), dtype=torch.bfloat16, device="cuda")
    ek = torch.empty((0, 2, 128, 128), dtype=torch.bfloat16, device="cuda")
    H.pyr_build_pyramid(p, ek, torch.empty(H.pyramid_shape(p), device="cuda"))
    p0 = H.Problem(1, 4, 2, 128, 0, 0, 4, 4, torch.bfloat16)
    assert H.pyr_pyramid_nodes(p0) == 0
    torch.cuda.synchronize()
    assert e.numel() == 0


def test_deterministic_and_in_bounds():
    """Two runs give bitwise-identical outputs, and nothing is written past the
    end of any output buffer (sentinel tails stay intact)."""
    cfg = C("det", 1, 8, 2, 64 * 30 + 7, 64 * 30 + 7, 128, torch.bfloat16, 4, 6, 4, seed=40)
    q, k, v = W.make_inputs(cfg, "cuda")
    p = GH.problem(cfg)
    pad = 4096
    outs = []
    for _ in range(2):
        shape = H.pyramid_shape(p)
        pyr_buf = torch.full((math.prod(shape) + pad,), 7.0, device="cuda")
        pyr = pyr_buf[:-pad].view(shape)
        H.pyr_build_pyramid(p, k, pyr)
        nqb = H.pyr_num_query_blocks(p)
        sel_buf = torch.full((2 * nqb * 7 + pad,), -77, dtype=torch.int32, device="cuda")
        sel = sel_buf[:-pad].view(1, 2, nqb, 7)
        H.pyr_select_topk(p, q, pyr, sel)
        o_buf = torch.full((q.numel() + pad,), 3.0, dtype=torch.bfloat16, device="cuda")
        o = o_buf[:-pad].view(q.shape)
        lse_buf = torch.full((8 * cfg.q_len + pad,), 5.0, device="cuda")
        lse = lse_buf[:-pad].view(1, 8, cfg.q_len)
        H.pyr_block_sparse_attn(p, q, k, v, sel, o, lse)
        torch.cuda.synchronize()
        assert bool((pyr_buf[-pad:] == 7.0).all())
        assert bool((sel_buf[-pad:] == -77).all())
        assert bool((o_buf[-pad:] == 3.0).all())
        assert bool((lse_buf[-pad:] == 5.0).all())
        outs.append((pyr.clone(), sel.clone(), o.clone(), lse.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
