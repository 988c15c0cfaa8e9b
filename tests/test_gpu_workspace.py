"""GPU checks of the attention's optional prefill workspace: dense bfloat16
prefill with G = q_heads/kv_heads a multiple of 4 and (top_k + 1) * G/4 >= 16
reads v through a block-transposed copy written into the workspace when the
caller passes one of pyr_attn_workspace_bytes(p) bytes.  The copy only moves
v's elements (keys past the sequence end become zeros, which the causal mask
weights by 0), so o and lse must be the same bits as with no workspace, with
a workspace one byte short (v read directly), and through pyr_select_attn's
two-launch path.  Parity of the workspace path with the oracle is covered by
the bfloat16 prefill cases of test_gpu_parity.py and test_gpu_routes.py that
clear the threshold, which pass the workspace.
"""

import pytest
import torch

import hierarchical_block_sparse_amd as H
from hierarchical_block_sparse_amd import workloads as W
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

C = W.Config
BF = torch.bfloat16
CASES = [
    # G = 4, d = 128, two sequences, ragged last block, K + 1 = 64
    C("ws_g4_d128", 2, 8, 2, 64 * 70 + 7, 64 * 70 + 7, 128, BF, 4, 63, 0, seed=71),
    # G = 8 (two workgroups per unit), d = 64
    C("ws_g8_d64", 1, 16, 2, 64 * 40 + 33, 64 * 40 + 33, 64, BF, 4, 31, 0, seed=72),
    # G = 16, one partial block; K beyond the history
    C("ws_g16_single_block", 1, 16, 1, 37, 37, 128, BF, 2, 15, 0, seed=73),
    # route rows of 71 entries (two 64-entry chunks)
    C("ws_g4_k70", 1, 8, 2, 64 * 80 + 9, 64 * 80 + 9, 64, BF, 4, 70, 0, seed=74),
]


def _attn(p, q, k, v, sel, ws):
    o = torch.empty_like(q)
    lse = torch.empty(p.lse_shape, dtype=torch.float32, device=q.device)
    H.pyr_block_sparse_attn(p, q, k, v, sel, o, lse, ws)
    torch.cuda.synchronize()
    return o, lse


def _same(a, b):
    return (torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
            and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32)))


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_transposed_v_same_bits(cfg):
    GH.log(f"case {cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hk={cfg.n_kv_heads} "
           f"T={cfg.kv_len} d={cfg.head_dim} K={cfg.top_k}")
    p = GH.problem(cfg)
    need = H.pyr_attn_workspace_bytes(p)
    nb = -(-cfg.kv_len // 64)
    assert need == cfg.batch * cfg.n_kv_heads * nb * 64 * cfg.head_dim * 2
    q, k, v = W.make_inputs(cfg, "cuda")
    sel = W.make_route(cfg, with_invalid=True, repeats=True).cuda()
    direct = _attn(p, q, k, v, sel, None)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN-patterned
    via_vt = _attn(p, q, k, v, sel, ws)
    assert _same(direct, via_vt)
    short = _attn(p, q, k, v, sel, ws[:need - 1])
    assert _same(direct, short)
    assert torch.isfinite(direct[0].float()).all() and torch.isfinite(direct[1]).all()


def test_transposed_v_with_spare_capacity():
    """k and v hold kv_capacity > kv_len rows; rows past kv_len are NaN and
    must be read by neither path."""
    T, cap = 64 * 9 + 21, 64 * 12 + 5
    cfg = C("ws_capacity", 2, 16, 2, T, T, 128, BF, 4, 31, 0, seed=75)
    q, k0, v0 = W.make_inputs(cfg, "cuda")
    p = H.Problem(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, T, T,
                  cfg.branching, cfg.top_k, cfg.dtype, kv_capacity=cap)
    k = torch.full((2, 2, cap, 128), float("nan"), dtype=BF, device="cuda")
    v = torch.full_like(k, float("nan"))
    k[:, :, :T] = k0
    v[:, :, :T] = v0
    sel = W.make_route(cfg, with_invalid=True, repeats=False).cuda()
    need = H.pyr_attn_workspace_bytes(p)
    assert need == 2 * 2 * (-(-T // 64)) * 64 * 128 * 2
    direct = _attn(p, q, k, v, sel, None)
    via_vt = _attn(p, q, k, v, sel, H.alloc_workspace(p))
    assert torch.isfinite(direct[0].float()).all()
    assert _same(direct, via_vt)
    # and the same bits as the problem without spare capacity
    p0 = GH.problem(cfg)
    assert _same(direct, _attn(p0, q, k0, v0, sel, H.alloc_workspace(p0)))


def test_select_attn_two_launch_path_uses_workspace():
    """G = 8 takes pyr_select_attn's two-launch path, whose attention gets the
    workspace: same bits as selection then attention without a workspace."""
    cfg = C("ws_select_attn_g8", 1, 16, 2, 64 * 40 + 3, 64 * 40 + 3, 128, BF, 4, 31, 0, seed=76)
    p = GH.problem(cfg)
    assert H.pyr_attn_workspace_bytes(p) > 0
    q, k, v = W.make_inputs(cfg, "cuda")
    pyr = H.alloc_pyramid(p)
    H.pyr_build_pyramid(p, k, pyr)
    sel_a, sel_b = H.alloc_sel(p), H.alloc_sel(p)
    o = torch.empty_like(q)
    lse = torch.empty(p.lse_shape, dtype=torch.float32, device="cuda")
    H.pyr_select_attn(p, q, k, v, pyr, sel_a, o, lse, H.alloc_workspace(p))
    H.pyr_select_topk(p, q, pyr, sel_b)
    ref = _attn(p, q, k, v, sel_b, None)
    assert torch.equal(sel_a, sel_b)
    assert _same((o, lse), ref)
