"""Seeded synthetic inputs for the pyramid selector and block-sparse attention.

This module only draws inputs.  It holds none of the method's arithmetic and is
shared by the tests, the benchmark and the oracle checks (which read back the
exact device tensors, so the two sides always see identical bytes).

Background: q, k, v iid N(0, 1) from a seeded ``torch.Generator`` on the target
device.  Planted retrieval (the stand-in for needle-style retrieval workloads,
PHBA §4.3 / §A.2.3 evaluate on such tasks): for every unit (batch, KV head,
query block i >= 1) pick min(n_planted, i) distinct earlier key blocks uniformly
from [0, i) and a direction u = g / |g| with g ~ N(0, I_d); add 3u to every
query row of block i in all query heads of the KV group and to every key row of
each picked block.  Plants accumulate in fp32 and the result is rounded once to
the storage dtype (round-to-nearest-even for bf16).  Plant choices and
directions come from ``numpy.random.default_rng`` with their own seed.  Decode
configurations plant n_planted blocks from [0, diag) per (sequence, KV head) and
add 3u to that sequence's single query token in every head of the group.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

PLANT_SCALE = 3.0


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    q_len: int
    kv_len: int
    head_dim: int
    dtype: torch.dtype
    branching: int
    top_k: int
    n_planted: int
    block: int = 64
    seed: int = 0

    @property
    def decode(self) -> bool:
        return self.q_len == 1 and self.kv_len > 1

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workloads the path is measured and checked on.
CONFIGS = {
    # Tiny fp32: B=1, H=2, T=2048, d=64, iid N(0,1); b=2, K=4 + diagonal.
    "tiny_fp32": Config("tiny_fp32", 1, 2, 2, 2048, 2048, 64, torch.float32, 2, 4, 0, seed=1),
    # MHA 32K: H=16, T=32768, d=128 bf16, 4 planted blocks per query block; b=4, K=16.
    "mha_32k": Config("mha_32k", 1, 16, 16, 32768, 32768, 128, torch.bfloat16, 4, 16, 4, seed=2),
    # GQA 128K: 32 q heads / 8 KV heads, T=131072, d=128 bf16, 8 planted; b=4, K=32.
    "gqa_128k": Config("gqa_128k", 1, 32, 8, 131072, 131072, 128, torch.bfloat16, 4, 32, 8, seed=3),
    # Decode: 64 sequences x 1 new token, 32/8 heads, KV 262144, d=128 bf16; b=4, K=64, 8 planted.
    "decode_256k": Config("decode_256k", 64, 32, 8, 1, 262144, 128, torch.bfloat16, 4, 64, 8, seed=4),
    # Long prefill: 8 q heads / 1 KV head, T=1048576, d=128 bf16, 16 planted; b=4, K=64.
    "prefill_1m": Config("prefill_1m", 1, 8, 1, 1048576, 1048576, 128, torch.bfloat16, 4, 64, 16, seed=5),
}


def _randn(shape, gen, device, dtype):
    return torch.randn(shape, generator=gen, device=device, dtype=dtype)


def make_inputs(cfg: Config, device="cpu"):
    """Return (q, k, v) for a config: q [B, Hq, Tq, d], k and v [B, Hk, Tk, d]."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + cfg.seed)
    rng = np.random.default_rng(2000 + cfg.seed)
    B, Hq, Hk, Tq, Tk, d = (cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.q_len, cfg.kv_len,
                            cfg.head_dim)
    blk = cfg.block
    if cfg.n_planted == 0:
        q = _randn((B, Hq, Tq, d), gen, device, torch.float32).to(cfg.dtype)
        k = _randn((B, Hk, Tk, d), gen, device, torch.float32).to(cfg.dtype)
        v = _randn((B, Hk, Tk, d), gen, device, torch.float32).to(cfg.dtype)
        return q, k, v
    if cfg.decode:
        return _make_decode(cfg, device, gen, rng)
    nb = -(-Tk // blk)
    nqb = -(-Tq // blk)
    # plant bookkeeping on the host: per-unit query direction, per-key-block sum of directions
    qdir = np.zeros((B, Hk, nqb, d), dtype=np.float64)
    kdir = np.zeros((B, Hk, nb, d), dtype=np.float64)
    for bi in range(B):
        for hk in range(Hk):
            for i in range(1, nqb):
                g = rng.standard_normal(d)
                u = g / np.linalg.norm(g)
                picks = rng.choice(i, size=min(cfg.n_planted, i), replace=False)
                qdir[bi, hk, i] = u
                np.add.at(kdir[bi, hk], picks, u)
    qd = torch.from_numpy(qdir.astype(np.float32)).to(device)
    kd = torch.from_numpy(kdir.astype(np.float32)).to(device)
    q = torch.empty((B, Hq, Tq, d), dtype=cfg.dtype, device=device)
    for h in range(Hq):      # one head at a time keeps the fp32 staging small
        x = _randn((B, Tq, d), gen, device, torch.float32)
        x += PLANT_SCALE * qd[:, h // cfg.group].repeat_interleave(blk, dim=1)[:, :Tq]
        q[:, h] = x.to(cfg.dtype)
        del x
    k = torch.empty((B, Hk, Tk, d), dtype=cfg.dtype, device=device)
    for hk in range(Hk):
        x = _randn((B, Tk, d), gen, device, torch.float32)
        x += PLANT_SCALE * kd[:, hk].repeat_interleave(blk, dim=1)[:, :Tk]
        k[:, hk] = x.to(cfg.dtype)
        del x
    v = _randn((B, Hk, Tk, d), gen, device, torch.float32).to(cfg.dtype)
    return q, k, v


def _make_decode(cfg: Config, device, gen, rng):
    B, Hq, Hk, Tk, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.kv_len, cfg.head_dim
    blk = cfg.block
    diag = (Tk - 1) // blk
    q = torch.empty((B, Hq, 1, d), dtype=cfg.dtype, device=device)
    k = torch.empty((B, Hk, Tk, d), dtype=cfg.dtype, device=device)
    v = torch.empty((B, Hk, Tk, d), dtype=cfg.dtype, device=device)
    for bi in range(B):               # one sequence at a time keeps the fp32 staging small
        qdir = np.zeros((Hk, d))
        kdir = np.zeros((Hk, -(-Tk // blk), d))
        for hk in range(Hk):
            g = rng.standard_normal(d)
            u = g / np.linalg.norm(g)
            qdir[hk] = u
            picks = rng.choice(diag, size=min(cfg.n_planted, diag), replace=False)
            np.add.at(kdir[hk], picks, u)
        qd = torch.from_numpy(qdir.astype(np.float32)).to(device)
        kd = torch.from_numpy(kdir.astype(np.float32)).to(device)
        x = _randn((Hq, 1, d), gen, device, torch.float32)
        x += PLANT_SCALE * qd.repeat_interleave(cfg.group, dim=0)[:, None, :]
        q[bi] = x.to(cfg.dtype)
        x = _randn((Hk, Tk, d), gen, device, torch.float32)
        x += PLANT_SCALE * kd.repeat_interleave(blk, dim=1)[:, :Tk]
        k[bi] = x.to(cfg.dtype)
        v[bi] = _randn((Hk, Tk, d), gen, device, torch.float32).to(cfg.dtype)
        del x
    return q, k, v


def planted_blocks(cfg: Config):
    """Replay the plant choices of ``make_inputs`` (for recall reporting only):
    dict unit -> set of planted key blocks."""
    rng = np.random.default_rng(2000 + cfg.seed)
    d, blk = cfg.head_dim, cfg.block
    out = {}
    if cfg.n_planted == 0:
        return out
    if cfg.decode:
        diag = (cfg.kv_len - 1) // blk
        for bi in range(cfg.batch):
            for hk in range(cfg.n_kv_heads):
                rng.standard_normal(d)
                out[(bi, hk, 0)] = set(int(x) for x in rng.choice(diag, size=min(cfg.n_planted, diag),
                                                                  replace=False))
        return out
    nqb = -(-cfg.q_len // blk)
    for bi in range(cfg.batch):
        for hk in range(cfg.n_kv_heads):
            for i in range(1, nqb):
                rng.standard_normal(d)
                out[(bi, hk, i)] = set(int(x) for x in rng.choice(i, size=min(cfg.n_planted, i),
                                                                  replace=False))
    return out


def make_grad_out(cfg: Config, device="cpu"):
    """dL/do for the backward: iid N(0, 1) of q's shape in the config's dtype."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(3000 + cfg.seed)
    shape = (cfg.batch, cfg.n_q_heads, cfg.q_len, cfg.head_dim)
    return _randn(shape, gen, device, torch.float32).to(cfg.dtype)


def make_route(cfg: Config, with_invalid: bool = True, repeats: bool = False):
    """A synthetic prefill route table [B, Hk, nqb, K+1] int32 (CPU): every row
    lists its diagonal block, then up to K distinct other blocks drawn uniformly
    from all blocks (future ones included: they are fully masked), in random
    order, -1 padded; with_invalid puts an out-of-range id (nb) into some rows;
    repeats lists one or two of a row's blocks a second time in about half of
    the rows that have free slots.  Used to drive the attention and its
    backward over routes the selection would not produce."""
    rng = np.random.default_rng(4000 + cfg.seed + (7 if repeats else 0))
    nb = -(-cfg.kv_len // cfg.block)
    nqb = -(-cfg.q_len // cfg.block)
    K = cfg.top_k
    out = np.full((cfg.batch, cfg.n_kv_heads, nqb, K + 1), -1, dtype=np.int32)
    for bi in range(cfg.batch):
        for hk in range(cfg.n_kv_heads):
            for i in range(nqb):
                others = [j for j in range(nb) if j != i]
                n = int(rng.integers(0, min(K, len(others)) + 1))
                row = [i] + [int(x) for x in rng.choice(others, size=n, replace=False)]
                if with_invalid and n < K and rng.random() < 0.25:
                    row.append(nb)
                if repeats and len(row) < K + 1 and rng.random() < 0.5:
                    free = K + 1 - len(row)
                    row += [row[int(rng.integers(len(row)))]
                            for _ in range(int(rng.integers(1, min(2, free) + 1)))]
                rng.shuffle(row)
                out[bi, hk, i, :len(row)] = row
    return torch.from_numpy(out)



# ---- packed batches (sequences back to back along the token axis) ----

def packed_lengths(total: int, shortest: int, longest: int, seed: int = 0) -> list[int]:
    """Sequence lengths of a packed batch of `total` rows: log-uniform in
    [shortest, longest] (numpy.random.default_rng(5000 + seed)), drawn until
    they fill `total`; the last one is cut to fit."""
    rng = np.random.default_rng(5000 + seed)
    out: list[int] = []
    while sum(out) < total:
        n = int(round(math.exp(rng.uniform(math.log(shortest), math.log(longest)))))
        out.append(min(n, total - sum(out)))
    return out


def make_packed_inputs(cfg: Config, lengths, device="cpu", spare_rows: int = 0):
    """(q, k, v, cu) of a packed batch: q [Hq, total, d], k and v [Hk, total, d]
    and cu int32 [S+1] with cu[s] = lengths[0] + ... + lengths[s-1].  Sequence
    s holds the inputs make_inputs draws for cfg at batch 1 and length
    lengths[s] with seed cfg.seed * 1000 + s (planted retrieval stays inside
    the sequence).  spare_rows rows of NaN follow the last sequence: no
    sequence owns them, so nothing may read them."""
    device = torch.device(device)
    qs, ks, vs = [], [], []
    for s, n in enumerate(lengths):
        c = replace(cfg, batch=1, q_len=n, kv_len=n, seed=cfg.seed * 1000 + s)
        q, k, v = make_inputs(c, device)
        qs.append(q[0])
        ks.append(k[0])
        vs.append(v[0])
    if spare_rows:
        nan = float("nan")
        qs.append(torch.full((cfg.n_q_heads, spare_rows, cfg.head_dim), nan, dtype=cfg.dtype,
                             device=device))
        ks.append(torch.full((cfg.n_kv_heads, spare_rows, cfg.head_dim), nan, dtype=cfg.dtype,
                             device=device))
        vs.append(ks[-1].clone())
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device=device)
    return torch.cat(qs, 1), torch.cat(ks, 1), torch.cat(vs, 1), cu
