"""The hot path under HIP graph capture: the library's calls launch kernels
only (no allocation, no memset, no synchronisation), so a whole step --
decode: append the newest key to the pyramid, select, attend; prefill: build,
select, attend, with the transposed-V workspace and with the fused entry
point -- can be captured once and replayed.  Each test captures a step on
static buffers, then replays it three times; before each replay the program
rewrites the queries in place (eager work) and synchronises, and after it
every output (pyramid, route rows, o, lse) must equal bit for bit an eager run
of the same step on the same inputs.  The decode step is also captured with
the allocation-free attention entry point, whose callers include code under
graph capture.
"""

import pytest
import torch

import hierarchical_block_sparse_amd as H
from hierarchical_block_sparse_amd import workloads as W
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

C = W.Config
BF = torch.bfloat16


def _capture(step):
    """Warm the step up on a side stream, then capture it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.int8), b.contiguous().view(torch.int8))


def _replays(g, q, outs, eager, seed):
    """Three replays, each after rewriting q in place; `eager()` returns the
    eager step's outputs on the current inputs, in the order of outs."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    for r in range(3):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert _same(a, b), f"replay {r}: output {i} differs from the eager step"
        GH.log(f"  replay {r}: {len(outs)} outputs equal the eager step")


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_decode_step_graph(noalloc):
    cfg = C("graph_decode", 4, 8, 2, 1, 64 * 300 + 5, 128, BF, 4, 16, 4, seed=81)
    GH.log(f"case {cfg.name} noalloc={noalloc}: B={cfg.batch} Tk={cfg.kv_len} K={cfg.top_k}")
    q, k, v = W.make_inputs(cfg, "cuda")
    T = cfg.kv_len
    mk = lambda n: H.Problem(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, 1, n,
                             cfg.branching, cfg.top_k, cfg.dtype, kv_capacity=T)
    p_prev, p = mk(T - 1), mk(T)
    pyr0 = torch.zeros(H.pyramid_shape(p), dtype=torch.float32, device="cuda")
    H.pyr_build_pyramid(p_prev, k, pyr0)          # the cache's pyramid before the newest key

    def run(pyr, sel, o, lse, ws):
        H.pyr_append_pyramid(p, k, T - 1, pyr)
        H.pyr_select_topk(p, q, pyr, sel)
        if noalloc:
            H.pyr_block_sparse_attn_noalloc(p, q, k, v, sel, o, lse)
        else:
            H.pyr_block_sparse_attn(p, q, k, v, sel, o, lse, ws)

    pyr, sel = pyr0.clone(), H.alloc_sel(p)
    o, lse = torch.empty_like(q), torch.empty(p.lse_shape, dtype=torch.float32, device="cuda")
    ws = None if noalloc else H.alloc_workspace(p)
    if noalloc:   # the first call on a device looks its scratch array up: not under capture
        run(pyr.clone(), H.alloc_sel(p), torch.empty_like(o), torch.empty_like(lse), None)
    g = _capture(lambda: run(pyr, sel, o, lse, ws))

    def eager():
        pyr2, sel2 = pyr0.clone(), H.alloc_sel(p)
        o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
        run(pyr2, sel2, o2, lse2, None if noalloc else H.alloc_workspace(p))
        return pyr2, sel2, o2, lse2

    _replays(g, q, (pyr, sel, o, lse), eager, seed=810)


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_prefill_step_graph(fused):
    # G = 8 with (K+1) * G/4 = 64 workgroup visits per key block: the attention
    # reads V through its transposed copy in the workspace; the fused case takes
    # G = 4 with b * (K+1) <= 192, one launch for selection and attention
    if fused:
        cfg = C("graph_prefill_fused", 1, 8, 2, 64 * 40 + 3, 64 * 40 + 3, 128, BF, 4, 15, 4,
                seed=82)
    else:
        cfg = C("graph_prefill_vt", 1, 16, 2, 64 * 40 + 3, 64 * 40 + 3, 128, BF, 4, 31, 4,
                seed=83)
    GH.log(f"case {cfg.name}: Hq={cfg.n_q_heads} Hk={cfg.n_kv_heads} T={cfg.kv_len} K={cfg.top_k}")
    q, k, v = W.make_inputs(cfg, "cuda")
    p = GH.problem(cfg)
    if not fused:
        assert H.pyr_attn_workspace_bytes(p) > 0

    def run(pyr, sel, o, lse, ws):
        H.pyr_build_pyramid(p, k, pyr)
        if fused:
            H.pyr_select_attn(p, q, k, v, pyr, sel, o, lse, ws)
        else:
            H.pyr_select_topk(p, q, pyr, sel)
            H.pyr_block_sparse_attn(p, q, k, v, sel, o, lse, ws)

    def bufs():
        return (H.alloc_pyramid(p), H.alloc_sel(p), torch.empty_like(q),
                torch.empty(p.lse_shape, dtype=torch.float32, device="cuda"))

    pyr, sel, o, lse = bufs()
    ws = H.alloc_workspace(p)
    g = _capture(lambda: run(pyr, sel, o, lse, ws))

    def eager():
        out = bufs()
        run(*out, H.alloc_workspace(p))
        return out

    _replays(g, q, (pyr, sel, o, lse), eager, seed=820 + int(fused))
