"""GPU parity of the attention backward for a fixed route table (PHBA §A.1.4:
probabilities recomputed from the forward's log-sum-exp, block-major key
gradients) against the float64 oracle, through the C ABI.

Each case runs the device forward (over the device selection, or over a
synthetic route table with unsorted, future, out-of-range and padded entries)
and then the device backward, and compares dq, dk and dv with
oracle.reference.attention_backward over the same route rows, q, k, v and
dout (the oracle recomputes its own float64 forward).

Tolerance, from the arithmetic: the kernels round P and dS = P (dP - D) to
bfloat16 (relative 2^-9) before the three products, accumulate in fp32 and
round each output once to bfloat16 (relative 2^-9); D is formed from the
bfloat16 forward output o.  Against outputs of size ~1 these give errors of a
few 1e-3, so the test asks for a max-abs error <= 2e-2 * max|ref| and a
relative Frobenius error <= 1e-2 per gradient; a dropped term, a wrong scale,
a lost head or a transposed operand gives errors of order 1.
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
BF = torch.bfloat16
CASES = [
    # GQA G=4 (the 128K workload's shape, shortened) with a ragged tail
    C("bwd_g4_ragged", 1, 8, 2, 64 * 20 + 17, 64 * 20 + 17, 128, BF, 4, 8, 4, seed=31),
    # MHA, d=64, two batch entries
    C("bwd_mha_d64_b2", 2, 2, 2, 64 * 12, 64 * 12, 64, BF, 2, 5, 0, seed=32),
    # G=2, d=128, ragged
    C("bwd_g2_d128", 1, 4, 2, 64 * 16 + 40, 64 * 16 + 40, 128, BF, 4, 6, 2, seed=33),
    # G=8, one KV head (the 1M workload's shape, shortened)
    C("bwd_g8_d128", 1, 8, 1, 64 * 24, 64 * 24, 128, BF, 4, 8, 4, seed=34),
    # odd G=3, d=64, one token past a block boundary
    C("bwd_g3_d64", 1, 6, 2, 64 * 10 + 1, 64 * 10 + 1, 64, BF, 2, 4, 0, seed=35),
    # a single partial block
    C("bwd_tiny", 1, 4, 2, 5, 5, 64, BF, 2, 1, 0, seed=36),
    # more than 32 query blocks (two bitmap words per key block), G=4, d=64
    C("bwd_two_words", 1, 4, 1, 64 * 70 + 9, 64 * 70 + 9, 64, BF, 4, 6, 2, seed=37),
    # 400 query blocks: key block rows split into work items of 3 query blocks
    # (multi-word rows, chunks across word boundaries, light and split rows)
    C("bwd_chunked", 1, 8, 2, 64 * 400, 64 * 400, 64, BF, 4, 15, 4, seed=39),
]
REL_MAX, REL_FRO = 2e-2, 1e-2


def _forward(cfg, q, k, v, route=None):
    """Device forward; returns (route rows used, o, lse)."""
    dev = GH.run_device(cfg, q, k, v, trace=False, sel_in=route)
    sel = dev["sel"] if route is None else route.to(torch.int32).to(q.device).contiguous()
    return sel, dev["o"], dev["lse"]


def _backward(cfg, q, k, v, sel, o, lse, dout):
    p = GH.problem(cfg)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = H.alloc_bwd_workspace(p)
    ws.fill_(0xA5)    # the workspace's contents on entry must not matter
    H.pyr_block_sparse_attn_bwd(p, q, k, v, sel, o, lse, dout, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return dq, dk, dv


def _judge(name, dev, ref):
    d = GH.f64(dev)
    assert np.isfinite(d).all(), f"{name}: non-finite values"
    scale = max(float(np.abs(ref).max()), 1e-30)
    e_max = float(np.abs(d - ref).max()) / scale
    e_fro = float(np.linalg.norm(d - ref) / max(np.linalg.norm(ref), 1e-30))
    GH.log(f"  {name}: max err {e_max:.2e} of max|ref| {scale:.3e}, rel fro {e_fro:.2e}")
    assert e_max <= REL_MAX and e_fro <= REL_FRO, name


def _check(cfg, route=None):
    GH.log(f"case {cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hk={cfg.n_kv_heads} "
           f"T={cfg.q_len} d={cfg.head_dim} K={cfg.top_k} route={'synthetic' if route is not None else 'selected'}")
    q, k, v = W.make_inputs(cfg, "cuda")
    dout = W.make_grad_out(cfg, "cuda")
    sel, o, lse = _forward(cfg, q, k, v, route)
    dq, dk, dv = _backward(cfg, q, k, v, sel, o, lse, dout)
    rq, rk, rv = reference.attention_backward(GH.f64(q), GH.f64(k), GH.f64(v),
                                              sel.cpu().numpy().astype(np.int64), cfg.block,
                                              GH.f64(dout))
    _judge("dq", dq, rq)
    _judge("dk", dk, rk)
    _judge("dv", dv, rv)
    return q, k, v, sel, o, lse, dout, (dq, dk, dv)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_backward_selected_routes(cfg):
    _check(cfg)


@pytest.mark.parametrize("cfg", CASES[:5], ids=lambda c: c.name)
def test_backward_synthetic_routes(cfg):
    _check(cfg, W.make_route(cfg))


def test_backward_is_deterministic():
    cfg = CASES[0]
    q, k, v, sel, o, lse, dout, first = _check(cfg)
    again = _backward(cfg, q, k, v, sel, o, lse, dout)
    for a, b in zip(first, again):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("G,d", [(4, 128), (1, 64)])
def test_backward_full_budget_is_dense_causal(G, d):
    """K >= nb - 1: every row sees every earlier key, so the gradients are
    those of dense causal attention (torch autograd of SDPA in float64 on the
    CPU, KV heads repeated over their group)."""
    T = 64 * 9 + 30
    cfg = C(f"bwd_dense_g{G}", 1, 2 * G, 2, T, T, d, BF, 4, 9, 0, seed=38 + G)
    q, k, v = W.make_inputs(cfg, "cuda")
    dout = W.make_grad_out(cfg, "cuda")
    sel, o, lse = _forward(cfg, q, k, v)
    dq, dk, dv = _backward(cfg, q, k, v, sel, o, lse, dout)
    qd = q.cpu().double().requires_grad_()
    kd = k.cpu().double().requires_grad_()
    vd = v.cpu().double().requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(
        qd, kd.repeat_interleave(G, dim=1), vd.repeat_interleave(G, dim=1), is_causal=True)
    out.backward(dout.cpu().double())
    _judge("dq", dq, qd.grad.numpy())
    _judge("dk", dk, kd.grad.numpy())
    _judge("dv", dv, vd.grad.numpy())


def test_backward_unlisted_blocks_and_blind_rows():
    """Key blocks that no route row lists get exactly zero dk and dv, and rows
    that see no key at all (their route lists only a later block; the forward
    gives lse = -inf) get exactly zero dq and add nothing, whatever the
    workspace held."""
    cfg = C("bwd_blind_rows", 1, 4, 2, 64 * 8, 64 * 8, 128, BF, 4, 2, 0, seed=40)
    q, k, v = W.make_inputs(cfg, "cuda")
    dout = W.make_grad_out(cfg, "cuda")
    route = torch.full((1, 2, 8, 3), -1, dtype=torch.int32)
    for i in range(8):
        route[0, :, i, 0] = i                  # the diagonal blocks ...
    route[0, 0, 7, 1] = 2                      # ... block 2 for one unit of KV head 0
    route[0, 1, 5, 0] = 0                      # KV head 1: unit 5 sees block 0 only,
    route[0, 1, 3, 0] = 6                      # unit 3 lists only a later block
    sel, o, lse = _forward(cfg, q, k, v, route)
    assert torch.isneginf(lse[0, 2:4, 192:256]).all()
    dq, dk, dv = _backward(cfg, q, k, v, sel, o, lse, dout)
    assert not dq[0, 2:4, 192:256].any()
    for j in (3, 5):
        assert not dk[0, 1, 64 * j:64 * j + 64].any() and not dv[0, 1, 64 * j:64 * j + 64].any()
    q64, k64, v64 = GH.f64(q), GH.f64(k), GH.f64(v)
    r64 = route.numpy().astype(np.int64)
    with np.errstate(invalid="ignore"):
        _, olse = reference.attention(q64, k64, v64, r64, 64)
    olse[~np.isfinite(olse)] = -np.inf     # rows with no visible key
    rq, rk, rv = reference.attention_backward(q64, k64, v64, r64, 64, GH.f64(dout), lse=olse)
    _judge("dq", dq, rq)
    _judge("dk", dk, rk)
    _judge("dv", dv, rv)
