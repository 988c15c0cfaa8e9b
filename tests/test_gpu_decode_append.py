"""GPU parity of decode-time pyramid maintenance and of the capacity layout
(reading R15), through the C ABI.

  * A pyramid laid out for a capacity larger than kv_len, over a key cache of
    capacity rows per head whose rows past kv_len hold NaN: every valid node
    matches the float64 oracle (max abs error <= 1e-5 max|k|, the pyramid bar),
    and selection and attention give the same bits as on a cache without spare
    rows.
  * pyr_append_pyramid after single-token and multi-token appends (across
    block boundaries and changes of the valid level sizes, up to the full
    capacity): every valid node matches the oracle's fresh build of the longer
    sequence, the bf16 split plane matches its fp32 means bit for bit, and
    nodes over no new token keep their bits.
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


def _problem(cfg, kv_len, cap, q_len=None):
    return H.Problem(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                     kv_len if q_len is None else q_len, kv_len, cfg.branching, cfg.top_k,
                     cfg.dtype, kv_capacity=cap)


def _cache(k, cap):
    """A key/value cache of `cap` rows per head holding k; the spare rows are NaN."""
    B, Hk, T, d = k.shape
    c = torch.full((B, Hk, cap, d), float("nan"), dtype=k.dtype, device=k.device)
    c[:, :, :T] = k
    return c


def _device_levels(pyr, p, kv_len, b):
    valid = reference.level_sizes(-(-kv_len // 64), b)
    out = []
    for lvl in range(H.pyr_num_levels(p)):
        off = H.pyr_level_offset(p, lvl)
        n = valid[lvl] if lvl < len(valid) else 1
        out.append(GH.f64(pyr[:, :, 0, off:off + n]))
    return out


def _check_levels(pyr, p, k_valid, b):
    """Device levels against the oracle's fresh build of k_valid; levels above
    the valid root must repeat the root."""
    T = k_valid.shape[2]
    k64 = GH.f64(k_valid)
    ref = reference.build_pyramid(k64, 64, b)
    dev = _device_levels(pyr, p, T, b)
    tol = 1e-5 * float(np.abs(k64).max())
    err = 0.0
    for lvl, d in enumerate(dev):
        r = ref[lvl] if lvl < len(ref) else ref[-1]
        err = max(err, float(np.abs(d - r).max()))
    GH.check_split_plane(pyr)
    return err, tol


def test_capacity_layout_build_select_attend():
    cfg = C("cap_prefill", 1, 8, 2, 64 * 20 + 17, 64 * 20 + 17, 128, torch.bfloat16, 4, 8, 4, seed=51)
    cap = 64 * 40
    q, k, v = W.make_inputs(cfg, "cuda")
    kc, vc = _cache(k, cap), _cache(v, cap)
    p0 = GH.problem(cfg)
    pc = _problem(cfg, cfg.kv_len, cap)
    GH.log(f"case {cfg.name}: T={cfg.kv_len} capacity={cap} levels {H.pyr_num_levels(p0)} -> {H.pyr_num_levels(pc)}")
    pyr0 = torch.zeros(H.pyramid_shape(p0), dtype=torch.float32, device="cuda")
    pyrc = torch.zeros(H.pyramid_shape(pc), dtype=torch.float32, device="cuda")
    H.pyr_build_pyramid(p0, k, pyr0)
    H.pyr_build_pyramid(pc, kc, pyrc)
    torch.cuda.synchronize()
    err, tol = _check_levels(pyrc, pc, k, cfg.branching)
    GH.log(f"  capacity pyramid max abs err {err:.3e} (tol {tol:.1e})")
    assert err <= tol
    sel0, selc = H.alloc_sel(p0), H.alloc_sel(pc)
    H.pyr_select_topk(p0, q, pyr0, sel0)
    H.pyr_select_topk(pc, q, pyrc, selc)
    o0, oc = torch.empty_like(q), torch.empty_like(q)
    l0 = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    lc = torch.empty_like(l0)
    H.pyr_block_sparse_attn(p0, q, k, v, sel0, o0, l0, H.alloc_workspace(p0))
    H.pyr_block_sparse_attn(pc, q, kc, vc, sel0, oc, lc, H.alloc_workspace(pc))
    torch.cuda.synchronize()
    assert torch.equal(sel0, selc)
    assert torch.equal(o0.view(torch.int16), oc.view(torch.int16))
    assert torch.equal(l0, lc)


@pytest.mark.parametrize("dtype,d,b", [(torch.bfloat16, 128, 4), (torch.float32, 64, 2)])
def test_decode_append_steps(dtype, d, b):
    cfg = C("append", 2, 8, 2, 1, 64 * 12, d, dtype, b, 8, 0, seed=52 if d == 128 else 53)
    cap = 64 * 12
    gen = torch.Generator(device="cuda").manual_seed(5200 + d)
    kc = torch.randn((cfg.batch, cfg.n_kv_heads, cap, d), generator=gen, device="cuda").to(dtype)
    t = 64 * 4 + 61
    p = _problem(cfg, t, cap, q_len=1)
    pyr = torch.zeros(H.pyramid_shape(p), dtype=torch.float32, device="cuda")
    H.pyr_build_pyramid(p, kc, pyr)
    # single tokens across a block boundary, then chunks that change the valid
    # level sizes, up to the full capacity
    steps = [t + 1, t + 2, t + 3, t + 4, 64 * 9 + 7, 64 * 9 + 8, cap]
    for new in steps:
        before = pyr.clone()
        pn = _problem(cfg, new, cap, q_len=1)
        H.pyr_append_pyramid(pn, kc, t, pyr)
        torch.cuda.synchronize()
        err, tol = _check_levels(pyr, pn, kc[:, :, :new], b)
        GH.log(f"  {dtype} append {t} -> {new}: max abs err {err:.3e} (tol {tol:.1e})")
        assert err <= tol
        # level-0 nodes before the block of token t gain nothing and keep their bits
        j0 = t // 64
        off0 = H.pyr_level_offset(pn, 0)
        assert torch.equal(pyr[:, :, :, off0:off0 + j0], before[:, :, :, off0:off0 + j0])
        t = new


@pytest.mark.parametrize("b,nblk", [(16, 4096), (2, 1000)], ids=["b16_45_siblings", "b2_10_levels"])
def test_append_inside_one_block_sibling_counts(b, nblk):
    """Appends that stay inside the last block take the on-chip fold when the
    affected nodes' older siblings number at most 32 (summed over the levels),
    and the level loop otherwise: with b = 16 and 4096 blocks the last block's
    ancestors have 15 older siblings on each of three levels (45, the level
    loop); with b = 2 and 1000 blocks they have 8 over ten levels (the fold).
    Both must match the oracle's fresh build and keep the untouched nodes."""
    cfg = C(f"append_b{b}", 2, 4, 2, 1, 64 * nblk, 64, torch.bfloat16, b, 8, 0, seed=55 + b)
    cap = 64 * nblk
    gen = torch.Generator(device="cuda").manual_seed(5500 + b)
    kc = torch.randn((cfg.batch, cfg.n_kv_heads, cap, 64), generator=gen, device="cuda").to(cfg.dtype)
    last = nblk - 1
    sib = 0
    m, lv = last, 1
    while lv < H.pyr_num_levels(_problem(cfg, cap, cap, q_len=1)):
        sib += m % b
        m //= b
        lv += 1
    GH.log(f"case b={b}: last block {last}, {sib} older siblings over the levels")
    assert (sib > 32) == (b == 16)
    t = 64 * last + 5
    p = _problem(cfg, t, cap, q_len=1)
    pyr = torch.zeros(H.pyramid_shape(p), dtype=torch.float32, device="cuda")
    H.pyr_build_pyramid(p, kc, pyr)
    for new in (t + 1, t + 2, t + 40, cap):   # one token, one token, a chunk, the rest of the block
        before = pyr.clone()
        pn = _problem(cfg, new, cap, q_len=1)
        H.pyr_append_pyramid(pn, kc, t, pyr)
        torch.cuda.synchronize()
        err, tol = _check_levels(pyr, pn, kc[:, :, :new], b)
        GH.log(f"  append {t} -> {new}: max abs err {err:.3e} (tol {tol:.1e})")
        assert err <= tol
        off0 = H.pyr_level_offset(pn, 0)
        assert torch.equal(pyr[:, :, :, off0:off0 + last], before[:, :, :, off0:off0 + last])
        t = new


def test_decode_path_over_a_cache():
    """The decode path on a cache with spare rows (build at kv_len - 1, append
    the last token, select, attend) gives the bits of the same path on a cache
    without spare rows built at kv_len."""
    cfg = C("cache_decode", 3, 8, 2, 1, 64 * 30 + 5, 128, torch.bfloat16, 4, 8, 4, seed=54)
    cap = 64 * 48
    q, k, v = W.make_inputs(cfg, "cuda")
    kc, vc = _cache(k, cap), _cache(v, cap)
    T = cfg.kv_len
    p0 = GH.problem(cfg)
    pc = _problem(cfg, T, cap, q_len=1)
    pm = _problem(cfg, T - 1, cap, q_len=1)
    pyr0 = H.alloc_pyramid(p0)
    H.pyr_build_pyramid(p0, k, pyr0)
    pyrc = torch.zeros(H.pyramid_shape(pc), dtype=torch.float32, device="cuda")
    H.pyr_build_pyramid(pm, kc, pyrc)
    H.pyr_append_pyramid(pc, kc, T - 1, pyrc)
    torch.cuda.synchronize()
    err, tol = _check_levels(pyrc, pc, k, cfg.branching)
    assert err <= tol
    sel0, selc = H.alloc_sel(p0), H.alloc_sel(pc)
    H.pyr_select_topk(p0, q, pyr0, sel0)
    H.pyr_select_topk(pc, q, pyrc, selc)
    torch.cuda.synchronize()
    GH.log(f"  decode routes equal: {bool(torch.equal(sel0, selc))}")
    assert torch.equal(sel0, selc)
    o0, oc = torch.empty_like(q), torch.empty_like(q)
    l0 = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    lc = torch.empty_like(l0)
    H.pyr_block_sparse_attn(p0, q, k, v, sel0, o0, l0, H.alloc_workspace(p0))
    H.pyr_block_sparse_attn(pc, q, kc, vc, selc, oc, lc, H.alloc_workspace(pc))
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), oc.view(torch.int16))
    assert torch.equal(l0, lc)
