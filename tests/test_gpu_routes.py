"""GPU parity for route rows the selection does not write: rows that list a
block more than once (reading R18: a route row is a set, so the block is
attended once), with out-of-range ids and -1 padding mixed in, through every
attention kernel and the backward.

Each case runs pyr_block_sparse_attn over W.make_route(..., repeats=True) and
checks o and lse against oracle.reference.attention over the same rows (which
reads each listed block once), and that the device gives the same bits over
the rows with their repeats removed (first occurrences kept, in order).  The
backward case compares dq, dk, dv with oracle.reference.attention_backward.
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
BF, F32 = torch.bfloat16, torch.float32
CASES = [
    # four query heads per KV head: attn_prefill_pp
    C("rep_g4_d128", 1, 8, 2, 64 * 12 + 7, 64 * 12 + 7, 128, BF, 4, 6, 0, seed=51),
    # two heads per KV head, d = 64: attn_prefill_mfma<64, 4, 1>
    C("rep_g2_d64", 1, 4, 2, 64 * 10, 64 * 10, 64, BF, 2, 5, 0, seed=52),
    # MHA, d = 128: attn_prefill_mfma<128, 2, 1>
    C("rep_mha_d128", 2, 2, 2, 64 * 9 + 30, 64 * 9 + 30, 128, BF, 4, 4, 0, seed=53),
    # fp32: attn_prefill_f32<64, 4>
    C("rep_fp32", 1, 4, 2, 64 * 8 + 3, 64 * 8 + 3, 64, F32, 2, 4, 0, seed=54),
    # decode, bf16 (attn_decode_mfma) and fp32 (attn_decode_split); K + 1 > 8
    # so a row spans several splits and a repeat can sit in a later split
    C("rep_decode_bf16", 3, 8, 2, 1, 64 * 40 + 5, 128, BF, 4, 12, 0, seed=55),
    C("rep_decode_fp32", 2, 4, 2, 1, 64 * 30, 64, F32, 2, 10, 0, seed=56),
    # K + 1 = 71 entries: rows span two 64-entry chunks of the route-set check
    # and some repeats sit in the second chunk, their first occurrence in the first
    C("rep_g4_k70", 1, 8, 2, 64 * 80 + 9, 64 * 80 + 9, 128, BF, 4, 70, 0, seed=60),
]


def _cross_chunk_repeats(route):
    """Rows in which an entry at position >= 64 repeats a block first listed
    before position 64."""
    r = route.numpy()
    n = 0
    for idx in np.ndindex(r.shape[:-1]):
        row = [int(x) for x in r[idx]]
        first = {}
        for pos, j in enumerate(row):
            if j < 0:
                continue
            if j in first and first[j] < 64 <= pos:
                n += 1
                break
            first.setdefault(j, pos)
    return n


def _dedup(route):
    """The route rows with every repeat removed (first occurrences kept, in
    row order) and -1 padding at the end."""
    r = route.numpy()
    out = np.full_like(r, -1)
    for idx in np.ndindex(r.shape[:-1]):
        row = list(dict.fromkeys(int(x) for x in r[idx]))
        out[idx][:len(row)] = row
    return torch.from_numpy(out)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_repeated_route_entries(cfg):
    GH.log(f"case {cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hk={cfg.n_kv_heads} "
           f"Tq={cfg.q_len} Tk={cfg.kv_len} d={cfg.head_dim} {cfg.dtype} K={cfg.top_k}")
    route = W.make_route(cfg, with_invalid=True, repeats=True)
    r = route.numpy()
    reps = sum(len([x for x in r[idx] if x >= 0]) > len(set(int(x) for x in r[idx] if x >= 0))
               for idx in np.ndindex(r.shape[:-1]))
    assert reps > 0, "the generator planted no repeat"
    if cfg.top_k + 1 > 64:
        assert _cross_chunk_repeats(route) > 0, "no repeat crosses the 64-entry chunk boundary"
    q, k, v = W.make_inputs(cfg, "cuda")
    dev = GH.run_device(cfg, q, k, v, trace=False, sel_in=route)
    dev2 = GH.run_device(cfg, q, k, v, trace=False, sel_in=_dedup(route))
    assert torch.equal(dev["o"].view(torch.int8), dev2["o"].view(torch.int8))
    assert torch.equal(dev["lse"], dev2["lse"])
    q64, k64, v64 = GH.f64(q), GH.f64(k), GH.f64(v)
    units = GH.all_units(cfg)
    # the oracle over the rows as they are: entries outside [0, nb) dropped,
    # repeats attended once (reading R18)
    nb = -(-cfg.kv_len // 64)
    rr = np.where((r >= 0) & (r < nb), r, -1)
    e_o, e_l = GH.judge_attention(q64, k64, v64, cfg, rr, dev["o"], dev["lse"], units)
    tol_o, tol_l = GH.TOL[cfg.dtype]
    GH.log(f"  {reps} rows with repeats; O err {e_o:.3e}, LSE err {e_l:.3e}")
    assert e_o <= tol_o and e_l <= tol_l


@pytest.mark.parametrize("K,T", [(7, 64 * 14 + 9), (70, 64 * 76 + 9)], ids=["k7", "k70"])
def test_backward_repeated_route_entries(K, T):
    cfg = C(f"rep_bwd_g4_k{K}", 1, 8, 2, T, T, 128, BF, 4, K, 0, seed=57)
    GH.log(f"case {cfg.name}: backward over route rows with repeats")
    route = W.make_route(cfg, with_invalid=True, repeats=True)
    if K + 1 > 64:
        assert _cross_chunk_repeats(route) > 0, "no repeat crosses the 64-entry chunk boundary"
    q, k, v = W.make_inputs(cfg, "cuda")
    dout = W.make_grad_out(cfg, "cuda")
    dev = GH.run_device(cfg, q, k, v, trace=False, sel_in=route)
    p = GH.problem(cfg)
    sel = route.to(torch.int32).cuda().contiguous()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = H.alloc_bwd_workspace(p)
    H.pyr_block_sparse_attn_bwd(p, q, k, v, sel, dev["o"], dev["lse"], dout, dq, dk, dv, ws)
    torch.cuda.synchronize()
    nb = -(-cfg.kv_len // 64)
    r = route.numpy().astype(np.int64)
    r = np.where((r >= 0) & (r < nb), r, -1)
    rq, rk, rv = reference.attention_backward(GH.f64(q), GH.f64(k), GH.f64(v), r, 64,
                                              GH.f64(dout))
    for name, d, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        dd = GH.f64(d)
        scale = max(float(np.abs(ref).max()), 1e-30)
        e_max = float(np.abs(dd - ref).max()) / scale
        e_fro = float(np.linalg.norm(dd - ref) / max(np.linalg.norm(ref), 1e-30))
        GH.log(f"  {name}: max err {e_max:.2e} of max|ref| {scale:.3e}, rel fro {e_fro:.2e}")
        assert e_max <= 2e-2 and e_fro <= 1e-2, name


@pytest.mark.parametrize("d", [128, 64])
def test_scores_far_above_the_first_block(d):
    """Rows whose scores on a later block exceed those on their first block by
    far more than the 2^64 headroom of a fixed softmax reference: the output
    must still be exact softmax attention (the kernel recomputes such rows
    with exact maxima).  Query rows are (32, 0, ...); keys of block 0 are
    zero, keys of block 3 are (64, 0, ...), so block 3 scores 2048 * scale
    (about 261 in log2 units at d = 128) and block 0 scores 0."""
    T = 64 * 8 + 5
    cfg = C(f"far_scores_d{d}", 1, 8, 2, T, T, d, BF, 4, 8, 0, seed=58)
    q, k, v = W.make_inputs(cfg, "cuda")
    q[:, :, 64 * 4:] = 0
    q[:, :, 64 * 4:, 0] = 32.0
    k[:, :, 0:64] = 0
    k[:, :, 3 * 64:4 * 64] = 0
    k[:, :, 3 * 64:4 * 64, 0] = 64.0
    nqb = -(-T // 64)
    route = torch.full((1, 2, nqb, 9), -1, dtype=torch.int32)
    for i in range(nqb):
        route[0, :, i, :i + 1] = torch.arange(i + 1)
    dev = GH.run_device(cfg, q, k, v, trace=False, sel_in=route)
    e_o, e_l = GH.judge_attention(GH.f64(q), GH.f64(k), GH.f64(v), cfg, route.numpy(), dev["o"],
                                  dev["lse"], GH.all_units(cfg))
    tol_o, tol_l = GH.TOL[cfg.dtype]
    GH.log(f"  {cfg.name}: O err {e_o:.3e}, LSE err {e_l:.3e}")
    assert e_o <= tol_o and e_l <= tol_l
