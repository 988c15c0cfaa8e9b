"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (whole tensors on the device, one call per stage).  The oracle
checks sampled units one by one: the pooled keys of the sampled (batch, KV
head) slabs, the tie-tolerant selection of each sampled unit along the device
trace, and the attention outputs of every row of the sampled units."""

import math

import numpy as np
import pytest
import torch

import hierarchical_block_sparse_amd as H
from hierarchical_block_sparse_amd import workloads as W
from oracle import check, reference
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu


def _sample_units(cfg, rng, n_slabs, n_per_slab):
    nqb = reference.num_query_blocks(cfg.q_len, cfg.kv_len, cfg.block)
    slabs = [(bi, hk) for bi in range(cfg.batch) for hk in range(cfg.n_kv_heads)]
    pick = [slabs[int(x)] for x in rng.choice(len(slabs), size=min(n_slabs, len(slabs)), replace=False)]
    units = []
    for bi, hk in pick:
        if nqb == 1:
            units.append((bi, hk, 0))
            continue
        fixed = [0, 1, 2, cfg.top_k - 1, cfg.top_k, cfg.top_k + 1, nqb // 2, nqb - 1]
        extra = rng.choice(nqb, size=n_per_slab, replace=False).tolist()
        for i in sorted(set(x for x in fixed + extra if 0 <= x < nqb)):
            units.append((bi, hk, int(i)))
    return pick, units


@pytest.mark.parametrize("name,n_slabs,n_per_slab,fused", [
    ("mha_32k", 2, 12, False),
    ("gqa_128k", 2, 12, False),
    ("gqa_128k", 2, 12, True),
    ("prefill_1m", 1, 16, False),
    ("decode_256k", 6, 0, False),
], ids=["mha_32k", "gqa_128k", "gqa_128k_fused", "prefill_1m", "decode_256k"])
def test_fullsize_sampled(name, n_slabs, n_per_slab, fused):
    cfg = W.CONFIGS[name]
    GH.log(f"full-size {name}{' (pyr_select_attn)' if fused else ''}: B={cfg.batch} "
           f"Hq={cfg.n_q_heads} Hk={cfg.n_kv_heads} Tq={cfg.q_len} Tk={cfg.kv_len} "
           f"b={cfg.branching} K={cfg.top_k}")
    q, k, v = W.make_inputs(cfg, "cuda")
    dev = GH.run_device(cfg, q, k, v, fused=fused)
    if fused:   # the attention half equals the separate kernel's over the same routes
        p = GH.problem(cfg)
        o2 = torch.empty_like(q)
        lse2 = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        H.pyr_block_sparse_attn(p, q, k, v, dev["sel"], o2, lse2, H.alloc_workspace(p))
        torch.cuda.synchronize()
        assert torch.equal(dev["o"].view(torch.int16), o2.view(torch.int16))
        assert torch.equal(dev["lse"], lse2)
        del o2, lse2
    rng = np.random.default_rng(77)
    slabs, units = _sample_units(cfg, rng, n_slabs, n_per_slab)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    sel = dev["sel"].cpu().numpy()
    tids = dev["tids"].cpu().numpy()
    o_dev = dev["o"]
    lse_dev = dev["lse"]
    tol_o, tol_l = GH.TOL[cfg.dtype]
    counts = {"exact": 0, "near_tie": 0, "fail": 0}
    e_o = e_l = e_p = 0.0
    pos = reference.query_positions(cfg.q_len, cfg.kv_len)
    for bi, hk in slabs:
        k64 = GH.f64(k[bi:bi + 1, hk:hk + 1])
        v64 = GH.f64(v[bi:bi + 1, hk:hk + 1])
        levels = [x[0, 0] for x in reference.build_pyramid(k64, cfg.block, cfg.branching)]
        dev_pyr = dev["pyr"][bi, hk, 0].double().cpu().numpy()
        ref_pyr = np.concatenate(levels, axis=0)
        e_p = max(e_p, float(np.abs(dev_pyr - ref_pyr).max()))
        assert e_p <= 1e-5 * max(float(np.abs(k64).max()), 1.0)
        heads = slice(hk * cfg.group, (hk + 1) * cfg.group)
        q64 = GH.f64(q[bi:bi + 1, heads])
        for (ub, uh, i) in units:
            if (ub, uh) != (bi, hk):
                continue
            toks, diag = reference.unit_tokens(i, cfg.q_len, cfg.kv_len, cfg.block)
            rows = reference.unit_rows(q64, 0, 0, cfg.group, toks)
            status, info = check.check_unit(rows, levels, diag, cfg.branching, cfg.top_k, scale,
                                            sel[bi, hk, i], [list(r) for r in tids[bi, hk, i]],
                                            tol=GH.SEL_TOL)
            counts[status] += 1
            assert status != "fail", ((bi, hk, i), info)
            if status == "exact":   # the oracle's own route row
                blocks = reference.select_unit(rows, levels, diag, cfg.branching, cfg.top_k,
                                               scale).sel
            else:                   # a near-tie row the walk above has just validated
                blocks = [int(x) for x in sel[bi, hk, i] if x >= 0]
            ob = o_dev[bi, heads][:, toks].float().cpu().numpy()
            lb = lse_dev[bi, heads][:, toks].cpu().numpy()
            for g in range(cfg.group):
                oo, ll = reference.attend_rows(q64[0, g, toks], pos[toks], k64[0, 0], v64[0, 0],
                                               blocks, cfg.block, scale)
                e_o = max(e_o, float(np.abs(ob[g] - oo).max()))
                e_l = max(e_l, float(np.abs(lb[g] - ll).max()))
    GH.log(f"  {len(units)} units: selection {counts}; pyramid err {e_p:.2e}; "
           f"O err {e_o:.3e}; LSE err {e_l:.3e}")
    assert counts["fail"] == 0
    assert e_o <= tol_o and e_l <= tol_l
    # every route row of the whole workload is well formed
    nvalid = (sel >= 0).sum(axis=-1)
    nqb = sel.shape[2]
    if cfg.decode:
        diag = (cfg.kv_len - 1) // cfg.block
        want = np.full(nvalid.shape, min(cfg.top_k, diag) + 1)
    else:
        want = np.minimum(cfg.top_k, np.arange(nqb)) + 1
    assert np.array_equal(nvalid, np.broadcast_to(want, nvalid.shape))
    del q, k, v, dev
    torch.cuda.empty_cache()
