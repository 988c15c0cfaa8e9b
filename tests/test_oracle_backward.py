"""Pins of the oracle's attention backward (oracle/reference.py,
attention_backward; PHBA §A.1.4, reading R14), all on the CPU:

  * central finite differences of L = sum(d_out * o) in float64;
  * torch autograd (float64, CPU) of the dense formulation with the route and
    causal mask applied as -inf scores;
  * a full budget reduces to dense causal attention: torch's
    scaled_dot_product_attention(is_causal=True) backward in float64;
  * planted mistakes (dropping the D term, the scale, the route mask) fail.
"""

import math

import numpy as np
import pytest
import torch

import oracle.reference as ref


def _case(seed, B=1, Hq=2, Hk=1, T=150, d=8, K=2, block=64):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hk, T, d))
    v = rng.standard_normal((B, Hk, T, d))
    do = rng.standard_normal((B, Hq, T, d))
    nqb = ref.num_query_blocks(T, T, block)
    sel = np.full((B, Hk, nqb, K + 1), -1, np.int32)
    for bi in range(B):
        for hk in range(Hk):
            for i in range(nqb):
                past = rng.permutation(i)[:K] if i else np.array([], int)
                blocks = sorted(int(x) for x in past) + [i]
                sel[bi, hk, i, :len(blocks)] = blocks
    return q, k, v, do, sel


def _loss(q, k, v, do, sel, block=64):
    o, _ = ref.attention(q, k, v, sel, block)
    return float((o * do).sum())


@pytest.mark.parametrize("seed", [0, 1])
def test_finite_differences(seed):
    q, k, v, do, sel = _case(seed)
    dq, dk, dv = ref.attention_backward(q, k, v, sel, 64, do)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do, sel)
            x[idx] = old - eps
            lm = _loss(q, k, v, do, sel)
            x[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def _dense_mask(sel, T, group, block=64):
    """[Hq, T, T] boolean mask: query t sees key s iff s's block is in t's
    route row and s <= t."""
    B, Hk, nqb, _ = sel.shape
    m = np.zeros((B, Hk * group, T, T), bool)
    for bi in range(B):
        for hk in range(Hk):
            for i in range(nqb):
                toks = np.arange(i * block, min((i + 1) * block, T))
                cols = np.zeros(T, bool)
                for j in sel[bi, hk, i]:
                    if j >= 0:
                        cols[j * block:min((j + 1) * block, T)] = True
                for h in range(hk * group, (hk + 1) * group):
                    for t in toks:
                        m[bi, h, t] = cols & (np.arange(T) <= t)
    return m


@pytest.mark.parametrize("seed,Hq,Hk,T,d", [(2, 2, 1, 150, 8), (3, 4, 2, 200, 16), (4, 3, 3, 64, 4)])
def test_matches_masked_dense_autograd(seed, Hq, Hk, T, d):
    q, k, v, do, sel = _case(seed, Hq=Hq, Hk=Hk, T=T, d=d, K=2)
    dq, dk, dv = ref.attention_backward(q, k, v, sel, 64, do)
    group = Hq // Hk
    mask = torch.from_numpy(_dense_mask(sel, T, group))
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    kx = tk.repeat_interleave(group, dim=1)
    vx = tv.repeat_interleave(group, dim=1)
    z = (tq @ kx.transpose(-1, -2)) / math.sqrt(d)
    z = z.masked_fill(~mask, float("-inf"))
    o = torch.softmax(z, dim=-1) @ vx
    (o * torch.from_numpy(do)).sum().backward()
    assert np.abs(tq.grad.numpy() - dq).max() <= 1e-10
    assert np.abs(tk.grad.numpy() - dk).max() <= 1e-10
    assert np.abs(tv.grad.numpy() - dv).max() <= 1e-10


def test_full_budget_equals_dense_causal_backward():
    """With every past block selected the route mask is the causal mask, so
    the gradients are those of dense causal attention."""
    T, d, Hq, Hk = 3 * 64 + 5, 8, 4, 2
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, Hq, T, d))
    k = rng.standard_normal((1, Hk, T, d))
    v = rng.standard_normal((1, Hk, T, d))
    do = rng.standard_normal((1, Hq, T, d))
    nqb = ref.num_query_blocks(T, T, 64)
    sel = np.full((1, Hk, nqb, nqb), -1, np.int32)
    for hk in range(Hk):
        for i in range(nqb):
            sel[0, hk, i, :i + 1] = np.arange(i + 1)
    dq, dk, dv = ref.attention_backward(q, k, v, sel, 64, do)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    g = Hq // Hk
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), is_causal=True)
    (o * torch.from_numpy(do)).sum().backward()
    assert np.abs(tq.grad.numpy() - dq).max() <= 1e-10
    assert np.abs(tk.grad.numpy() - dk).max() <= 1e-10
    assert np.abs(tv.grad.numpy() - dv).max() <= 1e-10


_orig = ref.attend_rows_backward


def _no_dsum(rows, row_pos, k_bh, v_bh, blocks, block, scale, d_out, lse):
    # planted: dS = P * dP (the D term dropped)
    Tk = k_bh.shape[0]
    kp = np.concatenate([np.arange(j * block, min((j + 1) * block, Tk)) for j in blocks])
    kk, vv = k_bh[kp], v_bh[kp]
    vis = kp[None, :] <= row_pos[:, None]
    p = np.where(vis, np.exp(scale * rows @ kk.T - lse[:, None]), 0.0)
    ds = p * (d_out @ vv.T)
    return scale * ds @ kk, kp, scale * ds.T @ rows, p.T @ d_out


def _no_scale(rows, row_pos, k_bh, v_bh, blocks, block, scale, d_out, lse):
    dr, kp, dk, dv = _orig(rows, row_pos, k_bh, v_bh, blocks, block, scale, d_out, lse)
    return dr / scale, kp, dk / scale, dv


def _no_causal(rows, row_pos, k_bh, v_bh, blocks, block, scale, d_out, lse):
    return _orig(rows, np.full_like(row_pos, 10 ** 9), k_bh, v_bh, blocks, block, scale, d_out,
                 lse)


@pytest.mark.parametrize("bad", [_no_dsum, _no_scale, _no_causal])
def test_planted_mistakes_fail_the_pins(bad, monkeypatch):
    monkeypatch.setattr(ref, "attend_rows_backward", bad)
    with pytest.raises(AssertionError):
        test_finite_differences(0)


def _repeat_entries(sel, seed):
    """A copy of sel with K+1 widened by two slots, where about half of the rows
    list one of their blocks a second (or third) time."""
    rng = np.random.default_rng(seed)
    B, Hk, nqb, W = sel.shape
    out = np.full((B, Hk, nqb, W + 2), -1, np.int32)
    out[..., :W] = sel
    for idx in np.ndindex(B, Hk, nqb):
        row = [int(x) for x in sel[idx] if x >= 0]
        if rng.random() < 0.5:
            extra = [row[int(rng.integers(len(row)))] for _ in range(int(rng.integers(1, 3)))]
            row = row + extra
            rng.shuffle(row)
            out[idx][:len(row)] = row
    return out


@pytest.mark.parametrize("seed,Hq,Hk,T,d", [(11, 2, 1, 150, 8), (12, 4, 2, 200, 16)])
def test_repeated_route_entries_count_once(seed, Hq, Hk, T, d):
    """Reading R18: a block listed more than once in a route row is attended
    once.  The masked dense formulation (the route as a set of columns, torch
    softmax and autograd in float64) gives the forward and the gradients."""
    q, k, v, do, sel = _case(seed, Hq=Hq, Hk=Hk, T=T, d=d, K=2)
    rsel = _repeat_entries(sel, seed)
    assert (np.sort(rsel, axis=-1)[..., 1:] == np.sort(rsel, axis=-1)[..., :-1]).any()
    group = Hq // Hk
    mask = torch.from_numpy(_dense_mask(rsel, T, group))
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    z = (tq @ tk.repeat_interleave(group, dim=1).transpose(-1, -2)) / math.sqrt(d)
    p = torch.softmax(z.masked_fill(~mask, float("-inf")), dim=-1)
    o_ref = p @ tv.repeat_interleave(group, dim=1)
    (o_ref * torch.from_numpy(do)).sum().backward()
    o, _ = ref.attention(q, k, v, rsel, 64)
    assert np.abs(o - o_ref.detach().numpy()).max() <= 1e-12
    dq, dk, dv = ref.attention_backward(q, k, v, rsel, 64, do)
    assert np.abs(tq.grad.numpy() - dq).max() <= 1e-10
    assert np.abs(tk.grad.numpy() - dk).max() <= 1e-10
    assert np.abs(tv.grad.numpy() - dv).max() <= 1e-10


def test_one_key_block_from_the_forward_output():
    """Given the forward's o and lse over the whole route, the gradients of the
    keys of any one routed block come out of attend_rows_backward over that
    block alone, equal to the rows of the whole-route computation."""
    rng = np.random.default_rng(21)
    T, d, R = 6 * 64 + 9, 16, 40
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    rows = rng.standard_normal((R, d))
    pos = np.sort(rng.integers(5 * 64, T, size=R))
    g = rng.standard_normal((R, d))
    blocks = [0, 2, 3, 6]
    scale = 1 / math.sqrt(d)
    o, lse = ref.attend_rows(rows, pos, k, v, blocks, 64, scale)
    _, kp, dk, dv = ref.attend_rows_backward(rows, pos, k, v, blocks, 64, scale, g, lse)
    for j in blocks:
        _, kpj, dkj, dvj = ref.attend_rows_backward(rows, pos, k, v, [j], 64, scale, g, lse, o=o)
        sl = np.isin(kp, kpj)
        assert np.array_equal(kp[sl], kpj)
        assert np.abs(dk[sl] - dkj).max() <= 1e-12 * max(1.0, np.abs(dk).max())
        assert np.abs(dv[sl] - dvj).max() <= 1e-12 * max(1.0, np.abs(dv).max())
    # without o the one-block call takes D from that block alone: a different
    # (wrong for a subset) value, which shows that o is what carries D
    _, _, dk0, _ = ref.attend_rows_backward(rows, pos, k, v, [0], 64, scale, g, lse)
    assert np.abs(dk0 - dk[np.isin(kp, np.arange(64))]).max() > 1e-6


def _attend_counting_repeats(rows, row_pos, k_bh, v_bh, blocks, block, scale):
    # planted: a block listed twice in a route row is attended twice
    Tk = k_bh.shape[0]
    kp = np.concatenate([np.arange(j * block, min((j + 1) * block, Tk)) for j in blocks])
    z = np.where(kp[None, :] <= row_pos[:, None], scale * rows @ k_bh[kp].T, -np.inf)
    mx = z.max(axis=1, keepdims=True)
    p = np.exp(z - mx)
    den = p.sum(axis=1, keepdims=True)
    return (p @ v_bh[kp]) / den, mx[:, 0] + np.log(den[:, 0])


def test_planted_repeat_counting_fails_the_pin(monkeypatch):
    monkeypatch.setattr(ref, "attend_rows", _attend_counting_repeats)
    with pytest.raises(AssertionError):
        test_repeated_route_entries_count_once(11, 2, 1, 150, 8)
