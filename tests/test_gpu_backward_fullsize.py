"""GPU parity of the attention backward at the full workload sizes, in the
launch configuration the benchmark's training pass times (whole tensors on the
device, the device selection as the route, one backward call: the key
gradients of busy key blocks split into work items whose fp32 partial sums
are added afterwards).

The float64 oracle (PHBA §A.1.4; oracle.reference) checks samples:
  * dk and dv of sampled key blocks of one KV head: the busiest blocks (block
    0 and the most visited ones, split over many work items), a block split
    over a few items, a light block (one item) and the last block (only its
    own query block visits it).  For every query block whose route lists the
    block, the oracle runs that unit's forward over its whole route (o and
    lse of all G heads' rows) and then the backward of the block's keys alone
    (attend_rows_backward over [j] given that o and lse), and sums them;
  * dq of every row of sampled units.
The route rows are the device selection's (the backward's input, which the
selection tests judge); everything else the oracle recomputes from q, k, v
and dout.  Bars as in the small backward tests: max-abs error <= 2e-2 of the
largest reference value and relative Frobenius error <= 1e-2 per gradient.

At 1M tokens (one KV head, K = 64) block 0 is visited by every query block
(16,384 units, about 18 TFLOP of float64 oracle work), so the sample there
takes blocks of up to a few hundred visitors, which run through the same
split items, partial slots and ordered reduction.
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
REL_MAX, REL_FRO = 2e-2, 1e-2


def _visitors(route_slab, nb):
    """visitors[j] = sorted query blocks whose route row lists key block j."""
    out = [[] for _ in range(nb)]
    for i, row in enumerate(route_slab):
        for j in set(int(x) for x in row if 0 <= x < nb):
            out[j].append(i)
    return out


def _pick_blocks(vis, budget, rng):
    """Key blocks to check: the busiest ones that fit the oracle budget (block
    0 first), one with a few hundred visitors or fewer, a light one and the
    last block.  Returns [(block, reason)]."""
    nb = len(vis)
    cnt = np.array([len(x) for x in vis])
    picks = []
    for j in [0] + list(np.argsort(-cnt, kind="stable")[:3]):
        if cnt[j] <= budget and all(j != p for p, _ in picks):
            picks.append((int(j), "busy"))
            break
    mid = [j for j in range(nb) if 100 <= cnt[j] <= 300]
    if mid:
        picks.append((int(rng.choice(mid)), "split over a few items"))
    light = [j for j in range(nb) if 2 <= cnt[j] <= 16]
    if light:
        picks.append((int(rng.choice(light)), "light"))
    picks.append((nb - 1, "last"))
    return picks


@pytest.mark.parametrize("name,budget", [("gqa_128k", 2100), ("prefill_1m", 300)],
                         ids=["gqa_128k", "prefill_1m"])
def test_backward_fullsize_sampled(name, budget):
    cfg = W.CONFIGS[name]
    G, d = cfg.group, cfg.head_dim
    GH.log(f"full-size backward {name}: Hq={cfg.n_q_heads} Hk={cfg.n_kv_heads} T={cfg.q_len} "
           f"K={cfg.top_k}")
    q, k, v = W.make_inputs(cfg, "cuda")
    dout = W.make_grad_out(cfg, "cuda")
    dev = GH.run_device(cfg, q, k, v, trace=False)
    sel, o, lse = dev["sel"], dev["o"], dev["lse"]
    del dev["pyr"]
    p = GH.problem(cfg)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = H.alloc_bwd_workspace(p)
    GH.log(f"  backward workspace {ws.numel() / 2**30:.2f} GiB")
    H.pyr_block_sparse_attn_bwd(p, q, k, v, sel, o, lse, dout, dq, dk, dv, ws)
    torch.cuda.synchronize()
    del ws, o, lse
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all()

    rng = np.random.default_rng(91)
    hk = int(rng.integers(cfg.n_kv_heads))
    nb = -(-cfg.kv_len // 64)
    nqb = -(-cfg.q_len // 64)
    route = sel[0, hk].cpu().numpy()
    vis = _visitors(route, nb)
    picks = _pick_blocks(vis, budget, rng)
    GH.log(f"  KV head {hk}: key blocks " + ", ".join(
        f"{j} ({len(vis[j])} visitors, {why})" for j, why in picks))
    heads = slice(hk * G, (hk + 1) * G)
    q_h = q[0, heads].cpu()           # bf16 on the host; slices go to float64 per unit
    g_h = dout[0, heads].cpu()
    k64 = GH.f64(k[0, hk])
    v64 = GH.f64(v[0, hk])
    pos_all = reference.query_positions(cfg.q_len, cfg.kv_len)
    scale = 1.0 / math.sqrt(d)

    def unit_rows(i):
        toks, _ = reference.unit_tokens(i, cfg.q_len, cfg.kv_len, 64)
        rows = q_h[:, toks].reshape(-1, d).double().numpy()
        grad = g_h[:, toks].reshape(-1, d).double().numpy()
        return toks, rows, grad, np.tile(pos_all[toks], G)

    ref_dk = {j: np.zeros((min(64, cfg.kv_len - 64 * j), d)) for j, _ in picks}
    ref_dv = {j: np.zeros_like(ref_dk[j]) for j, _ in picks}
    wanted = sorted(set(i for j, _ in picks for i in vis[j]))
    GH.log(f"  oracle: forward of {len(wanted)} visiting units")
    for i in wanted:
        _, rows, grad, pos = unit_rows(i)
        blocks = [int(x) for x in route[i] if 0 <= x < nb]
        o_u, lse_u = reference.attend_rows(rows, pos, k64, v64, blocks, 64, scale)
        for j, _ in picks:
            if i in vis[j]:
                _, _, dkj, dvj = reference.attend_rows_backward(rows, pos, k64, v64, [j], 64, scale,
                                                                grad, lse_u, o=o_u)
                ref_dk[j] += dkj
                ref_dv[j] += dvj

    def judge(name, dev_t, ref_t):
        dd = GH.f64(dev_t)
        sc = max(float(np.abs(ref_t).max()), 1e-30)
        e_max = float(np.abs(dd - ref_t).max()) / sc
        e_fro = float(np.linalg.norm(dd - ref_t) / max(np.linalg.norm(ref_t), 1e-30))
        GH.log(f"  {name}: max err {e_max:.2e} of max|ref| {sc:.3e}, rel fro {e_fro:.2e}")
        assert e_max <= REL_MAX and e_fro <= REL_FRO, name

    for j, why in picks:
        rows = slice(64 * j, 64 * j + ref_dk[j].shape[0])
        judge(f"dk block {j} ({why})", dk[0, hk, rows], ref_dk[j])
        judge(f"dv block {j} ({why})", dv[0, hk, rows], ref_dv[j])

    # dq of every row of sampled units (the heaviest last one included)
    for i in sorted(set([1, cfg.top_k + 1, nqb // 2, nqb - 1]) & set(range(nqb))):
        toks, rows, grad, pos = unit_rows(i)
        blocks = [int(x) for x in route[i] if 0 <= x < nb]
        _, lse_u = reference.attend_rows(rows, pos, k64, v64, blocks, 64, scale)
        d_rows, _, _, _ = reference.attend_rows_backward(rows, pos, k64, v64, blocks, 64, scale,
                                                         grad, lse_u)
        judge(f"dq unit {i}", dq[0, heads][:, toks].reshape(-1, d), d_rows)
    del q, k, v, dout, dq, dk, dv, sel
    torch.cuda.empty_cache()
