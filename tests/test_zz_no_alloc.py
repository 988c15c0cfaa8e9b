"""The allocation-free attention entry point (pyr_block_sparse_attn_noalloc):
through the C ABI it must give, bit for bit, what pyr_block_sparse_attn gives
with a caller's workspace, over the same route rows, on two calls in a row
(the second one smaller, so the shared scratch array holds the first call's
partials when the second starts), for the decode kernels that use the
scratch (bf16 on the matrix cores, fp32 on the vector units) and for a
prefill problem (no scratch).  Outputs of both are also checked against the
float64 oracle."""

import numpy as np
import pytest
import torch

import hierarchical_block_sparse_amd as H
from hierarchical_block_sparse_amd import workloads as W
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

C = W.Config
BF, F32 = torch.bfloat16, torch.float32


def _both(cfg, check_oracle):
    GH.log(f"case {cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hk={cfg.n_kv_heads} "
           f"Tq={cfg.q_len} Tk={cfg.kv_len} d={cfg.head_dim} {cfg.dtype} K={cfg.top_k}")
    q, k, v = W.make_inputs(cfg, "cuda")
    p = GH.problem(cfg)
    dev = GH.run_device(cfg, q, k, v, trace=False)   # selection + attention with a workspace
    o2 = torch.full_like(q, float("nan"))
    lse2 = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    H.pyr_block_sparse_attn_noalloc(p, q, k, v, dev["sel"], o2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(dev["o"].view(torch.int8), o2.view(torch.int8)), cfg.name
    assert torch.equal(dev["lse"], lse2), cfg.name
    if check_oracle:
        e_o, e_l = GH.judge_attention(GH.f64(q), GH.f64(k), GH.f64(v), cfg,
                                      dev["sel"].cpu().numpy(), o2, lse2, GH.all_units(cfg))
        tol_o, tol_l = GH.TOL[cfg.dtype]
        GH.log(f"  O err {e_o:.3e}, LSE err {e_l:.3e}")
        assert e_o <= tol_o and e_l <= tol_l


@pytest.mark.parametrize("dtype", [BF, F32], ids=["bf16", "fp32"])
def test_noalloc_decode_twice(dtype):
    d = 128 if dtype == BF else 64
    big = C("na_decode_big", 16, 16, 4, 1, 64 * 200 + 9, d, dtype, 4, 24, 4, seed=61)
    small = C("na_decode_small", 3, 8, 2, 1, 64 * 50 + 1, d, dtype, 4, 9, 2, seed=62)
    p = GH.problem(big)
    assert 0 < H.pyr_attn_workspace_bytes(p) <= 16 << 20
    _both(big, check_oracle=False)
    _both(small, check_oracle=True)


def test_noalloc_prefill():
    _both(C("na_prefill", 1, 8, 2, 64 * 20 + 5, 64 * 20 + 5, 128, BF, 4, 6, 2, seed=63),
          check_oracle=True)


def test_noalloc_rejects_oversized_decode():
    """A decode problem whose partial states exceed the 16 MiB array is
    refused before anything runs (the caller-workspace entry point takes it)."""
    cfg = C("na_too_big", 512, 32, 8, 1, 65, 128, BF, 4, 64, 0, seed=64)
    p = GH.problem(cfg)
    assert H.pyr_attn_workspace_bytes(p) > 16 << 20
    q, k, v = W.make_inputs(cfg, "cuda")
    sel = H.alloc_sel(p)
    sel.fill_(0)
    o = torch.empty_like(q)
    with pytest.raises(H.PyrError) as e:
        H.pyr_block_sparse_attn_noalloc(p, q, k, v, sel, o)
    assert e.value.status == 5 and "allocation-free" in e.value.detail
