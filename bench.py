#!/usr/bin/env python3
"""Benchmark: pyramid top-K selection + block-sparse causal attention on one MI355X.

One step = the whole hot path over one batch of synthetic input already resident
in HBM: pyr_build_pyramid -> pyr_select_topk -> pyr_block_sparse_attn (for the
decode workload the pyramid of the KV cache exists beforehand and a step is
pyr_append_pyramid of the newest token -> selection -> attention).  W untimed warm-up steps, then K timed steps
bracketed by torch.cuda.synchronize(); per-stage times come from HIP events
recorded on the stream the library launches on.

Prints one JSON line.  `value` is tokens/s of the whole path; `roofline`
describes the dominant kernel (the attention); `cpu_baseline` is the float64
CPU oracle timed on this host over a bounded sample of the same workload.

With --packed (prefill workloads) the workload's tokens are cut into a packed
batch of mixed-length sequences (log-uniform lengths in [1K, 32K] tokens), each
attending within itself through the packed-sequence form of the same entry
points; `value` is tokens/s over all of them.

With --backward (prefill workloads) a step is the training pass of the path:
build -> select -> attention -> pyr_block_sparse_attn_bwd for a seeded dL/do,
`value` is tokens/s of that pass and `roofline` describes the backward call
(its flops counted as 10 d per visible (query row, key) pair per head: the
recomputed scores, dP, dQ, dK and dV products).

With --graph one step is captured in a HIP graph after the eager, event-timed
steps, and `value` and `ms_per_step` come from K replays of that graph (no
launch gaps between the step's kernels); the stage times and the roofline stay
those of the eager steps (the kernels are the same), and
`stages.eager_ms_per_step` keeps the eager rate.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "select+sparse-attn tokens/s at T=128K; TFLOP/s & HBM GB/s as % of peak"
METRIC_BWD = "training pass (select+sparse-attn forward + attention backward) tokens/s"
METRIC_PACKED = "select+sparse-attn tokens/s over a packed batch of mixed-length sequences"
PACKED_SHORTEST, PACKED_LONGEST = 1024, 32768


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa_128k",
                    choices=["gqa_128k", "mha_32k", "prefill_1m", "decode_256k", "tiny_fp32"])
    ap.add_argument("--cpu-baseline-units", type=int, default=2048,
                    help="units of the workload the oracle runs for the CPU baseline (0: skip)")
    ap.add_argument("--packed", action="store_true",
                    help="cut the workload's tokens into a packed batch of mixed-length sequences")
    ap.add_argument("--fused", action="store_true",
                    help="selection and attention in one pyr_select_attn call per step")
    ap.add_argument("--backward", action="store_true",
                    help="time the training pass (forward + backward of the attention)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays (stage times and "
                         "the roofline still come from eagerly launched, event-timed steps)")
    ap.add_argument("--cold-steps", type=int, default=-1,
                    help="cold-cache steps timed after the warm ones (-1: as many as --steps; 0: none)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 5 device-to-device copies of 1 GiB (counter calibration)")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of known size, for scaling the HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": dt * 1e3,
                      "GB/s_read+write": 2 * n / dt / 1e9}), flush=True)


# ---------------------------------------------------------------------------
# algorithmic work (per-unit bytes and flops from the definitions of the steps)
# ---------------------------------------------------------------------------

def _num_blocks(n_tokens):
    """64-token blocks covering n_tokens tokens (the last may be ragged)."""
    return -(-n_tokens // 64)


def _level_sizes(n_blocks, b):
    """Nodes per pyramid level, finest first, down to the single root."""
    sizes = [n_blocks] if n_blocks > 0 else []
    while sizes and sizes[-1] > 1:
        sizes.append(-(-sizes[-1] // b))
    return sizes


def attn_work(cfg):
    """(flops, bytes) of the attention over the selection: every attended
    (query row, key) pair costs 4d flops (QK^T and PV); bytes = Q read + O write
    + the gathered K and V tiles of every selected block, once per unit."""
    s = 2 if cfg.dtype.itemsize == 2 else 4
    d, G, K = cfg.head_dim, cfg.group, cfg.top_k
    bh = cfg.batch * cfg.n_kv_heads
    if cfg.decode:
        diag = (cfg.kv_len - 1) // 64
        keys = min(K, diag) * 64 + (cfg.kv_len - diag * 64)
        flops = bh * G * keys * 4 * d
        byts = bh * (2 * G * d * s + 2 * keys * d * s)
        return flops, byts
    nqb = _num_blocks(cfg.q_len)
    pairs = sum(min(K, i) * 64 * 64 + 64 * 65 // 2 for i in range(nqb))
    tiles = sum(min(K, i) + 1 for i in range(nqb))
    flops = bh * G * pairs * 4 * d
    byts = bh * (2 * G * cfg.q_len * d * s + tiles * 2 * 64 * d * s)
    return flops, byts


def build_bytes(cfg, n_tot, planes):
    """Keys read once plus every pyramid plane written (fp32 means, and the
    bf16 hi/lo plane of bf16 problems)."""
    s = 2 if cfg.dtype.itemsize == 2 else 4
    bh = cfg.batch * cfg.n_kv_heads
    return bh * (cfg.kv_len * cfg.head_dim * s + planes * n_tot * cfg.head_dim * 4)


def select_work(cfg, sel_levels_cands):
    """(flops, bytes): flops = sum over scored candidates of rows * 2d (fp32
    dot products); bytes = Q read + route rows written (pooled keys are
    L2-resident and not counted)."""
    s = 2 if cfg.dtype.itemsize == 2 else 4
    rows = cfg.group * (1 if cfg.decode else 64)
    flops = sel_levels_cands * rows * 2 * cfg.head_dim
    bh = cfg.batch * cfg.n_kv_heads
    nqb = 1 if cfg.decode else -(-cfg.q_len // 64)
    byts = cfg.batch * cfg.n_q_heads * cfg.q_len * cfg.head_dim * s + bh * nqb * (cfg.top_k + 1) * 4
    return flops, byts


def scored_candidates(cfg):
    """Total candidates scored over all units (levels with more than K
    candidates), from the selection geometry: every scored level of a unit
    has b*K children of kept nodes plus the ancestor's fully-past children."""
    b, K = cfg.branching, cfg.top_k
    sizes = _level_sizes(_num_blocks(cfg.kv_len), b)
    L = len(sizes)
    diags = [(cfg.kv_len - 1) // 64] if cfg.decode else range(-(-cfg.q_len // 64))
    total = 0
    for diag in diags:
        nk = 0
        for lvl in range(L - 1, -1, -1):
            anc = diag // b ** lvl
            C = anc if lvl == L - 1 else nk * b + (anc - (diag // b ** (lvl + 1)) * b)
            if C > K:
                total += C
                nk = K
            else:
                nk = C
    return total * cfg.batch * cfg.n_kv_heads


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(cfg, q, k, v, n_units, backward=False):
    import math

    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import reference
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas_threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
        rng = np.random.default_rng(0)
        nqb = 1 if cfg.decode else -(-cfg.q_len // 64)
        bh_pairs = [(bi, hk) for bi in range(cfg.batch) for hk in range(cfg.n_kv_heads)]
        # sample: one (batch, KV head), units spread over its query blocks
        bi, hk = bh_pairs[int(rng.integers(len(bh_pairs)))]
        if cfg.decode:
            units = [(bi, hk, 0)]
        else:
            idx = sorted(set([0, 1, cfg.top_k, nqb - 1] +
                             list(rng.choice(nqb, size=min(nqb, n_units), replace=False))))
            units = [(bi, hk, int(i)) for i in idx[:max(n_units, 4)]]
        t0 = time.perf_counter()
        k64 = k[bi:bi + 1, hk:hk + 1].float().cpu().numpy().astype(np.float64)
        v64 = v[bi:bi + 1, hk:hk + 1].float().cpu().numpy().astype(np.float64)
        heads = slice(hk * cfg.group, (hk + 1) * cfg.group)
        t_copy = time.perf_counter() - t0
        t0 = time.perf_counter()
        levels = reference.build_pyramid(k64, 64, cfg.branching)
        t_pyr = time.perf_counter() - t0
        q64 = q[bi:bi + 1, heads].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        scale = 1 / math.sqrt(cfg.head_dim)
        for (_, _, i) in units:
            toks, diag = reference.unit_tokens(i, cfg.q_len, cfg.kv_len, 64)
            rows = reference.unit_rows(q64, 0, 0, cfg.group, toks)
            us = reference.select_unit(rows, [x[0, 0] for x in levels], diag, cfg.branching,
                                       cfg.top_k, scale)
            pos = reference.query_positions(cfg.q_len, cfg.kv_len)[toks]
            for h in range(cfg.group):
                o_h, lse_h = reference.attend_rows(q64[0, h, toks], pos, k64[0, 0], v64[0, 0],
                                                   us.sel, 64, scale)
                if backward:   # dL/do = o stands in for a gradient of the same shape
                    reference.attend_rows_backward(q64[0, h, toks], pos, k64[0, 0], v64[0, 0],
                                                   us.sel, 64, scale, o_h, lse_h)
        t_units = time.perf_counter() - t0
    n_bh = len(bh_pairs)
    # decode steps start from a prebuilt pyramid, as on the device
    total = (0.0 if cfg.decode else t_pyr * n_bh) + t_units / len(units) * (nqb * n_bh)
    tokens = cfg.batch * (1 if cfg.decode else cfg.q_len)
    return {
        "value": tokens / total, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
        "sample": (("forward + backward: " if backward else "") +
                   f"float64 NumPy oracle on {len(units)} of {nqb * n_bh} units (one batch/KV-head "
                   f"slab: pyramid {t_pyr:.2f}s, units {t_units:.2f}s; D2H copy {t_copy:.2f}s "
                   f"excluded); whole-workload time extrapolated as pyramid x {n_bh} slabs + "
                   f"mean unit time x {nqb * n_bh} units"),
        "host_cores_visible": cores,
    }


def attn_kernel_name(cfg, packed=False):
    """The attention kernels the library runs for this workload, in launch
    order (dense bfloat16 prefill with G a multiple of 4 and (K+1) * G/4 >= 16
    first writes the block-transposed copy of v into the workspace)."""
    if cfg.decode:
        return "attn_decode_mfma+combine" if cfg.dtype.itemsize == 2 else "attn_decode_split+combine"
    if cfg.dtype.itemsize != 2:
        return "attn_prefill_f32"
    if cfg.group % 4 == 0:
        vt = not packed and (cfg.top_k + 1) * (cfg.group // 4) >= 16
        return "attn_vt_build+attn_prefill_pp" if vt else "attn_prefill_pp"
    return "attn_prefill_mfma"


def planted_recall(cfg, sel):
    """Fraction of the planted (unit, key block) pairs whose block is in the
    unit's route row: a quality indicator of the selection, not a gate."""
    from hierarchical_block_sparse_amd import workloads as W
    plants = W.planted_blocks(cfg)
    if not plants:
        return None
    rows = sel.cpu().numpy()
    hit = total = 0
    for (bi, hk, i), blocks in plants.items():
        hit += len(blocks & set(rows[bi, hk, i].tolist()))
        total += len(blocks)
    return hit / total


def fused_kernel(cfg):
    """Whether pyr_select_attn runs as one launch for this workload (bfloat16
    prefill, four query heads per KV head, branching * (top_k + 1) <= 192)."""
    import torch
    return (cfg.dtype == torch.bfloat16 and not cfg.decode and cfg.group == 4
            and cfg.branching * (cfg.top_k + 1) <= 192)


def kernel_traffic(workload, kind="attn"):
    """HBM bytes per dispatch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_pmc.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        # the SHA-256 of the kernel's source files, concatenated in the listed order
        h = hashlib.sha256()
        for name in rec.get("sources", [f"{kind}.hip"]):
            with open(os.path.join(ROOT, "hierarchical_block_sparse_amd", "csrc", name), "rb") as f:
                h.update(f.read())
        if rec.get("attn_src_sha256") != h.hexdigest():
            return None
        return rec.get("bytes_per_dispatch")
    except (OSError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import torch

    import hierarchical_block_sparse_amd as H
    from hierarchical_block_sparse_amd import workloads as W

    cfg = W.CONFIGS[args.workload]
    if args.backward and (cfg.decode or cfg.dtype != torch.bfloat16):
        print(json.dumps({"error": "the backward runs on bfloat16 prefill workloads"}), flush=True)
        sys.exit(2)
    if args.fused and (cfg.decode or args.backward):
        print(json.dumps({"error": "--fused takes a prefill workload, forward only"}), flush=True)
        sys.exit(2)
    if args.packed and (cfg.decode or args.backward or cfg.batch != 1):
        print(json.dumps({"error": "--packed takes a batch-1 prefill workload, forward only"}),
              flush=True)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# generating {cfg.name} inputs", file=sys.stderr, flush=True)
    lengths = None
    if args.packed:
        lengths = W.packed_lengths(cfg.q_len, PACKED_SHORTEST, PACKED_LONGEST, cfg.seed)
        q, k, v, cu = W.make_packed_inputs(cfg, lengths, dev)
        p = H.problem_for_packed(q, k, cu, max(lengths), cfg.branching, cfg.top_k)
    else:
        q, k, v = W.make_inputs(cfg, dev)
        p = H.Problem(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.q_len,
                      cfg.kv_len, cfg.branching, cfg.top_k, cfg.dtype)
    # per-sequence views of the workload for the work accounting
    parts = [cfg.with_(q_len=n, kv_len=n) for n in lengths] if lengths else [cfg]
    pyr = H.alloc_pyramid(p, dev)
    sel = H.alloc_sel(p, dev)
    o = torch.empty_like(q)
    lse = torch.empty(p.lse_shape, dtype=torch.float32, device=dev)
    ws = H.alloc_workspace(p, dev)
    stream = torch.cuda.current_stream()
    if cfg.decode:
        # the cache's pyramid exists for the first kv_len - 1 tokens; every step
        # appends the newest token to it (pyramid maintenance), then selects and attends
        p_prev = H.Problem(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, 1,
                           cfg.kv_len - 1, cfg.branching, cfg.top_k, cfg.dtype,
                           kv_capacity=cfg.kv_len)
        H.pyr_build_pyramid(p_prev, k, pyr, stream)
    if args.backward:
        dout = W.make_grad_out(cfg, dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = H.alloc_bwd_workspace(p, dev)

    n_stage = 4 if args.backward else 3
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_stage + 1)]
          for _ in range(args.steps)]

    def step(events=None):
        if events:
            events[0].record(stream)
        if cfg.decode:
            H.pyr_append_pyramid(p, k, cfg.kv_len - 1, pyr, stream)
        else:
            H.pyr_build_pyramid(p, k, pyr, stream)
        if events:
            events[1].record(stream)
        if args.fused:
            H.pyr_select_attn(p, q, k, v, pyr, sel, o, lse, ws, None, None, stream)
            if events:
                events[2].record(stream)
                events[3].record(stream)
        else:
            H.pyr_select_topk(p, q, pyr, sel, None, None, stream)
            if events:
                events[2].record(stream)
            H.pyr_block_sparse_attn(p, q, k, v, sel, o, lse, ws, stream)
            if events:
                events[3].record(stream)
        if args.backward:
            H.pyr_block_sparse_attn_bwd(p, q, k, v, sel, o, lse, dout, dq, dk, dv, bws, stream)
            if events:
                events[4].record(stream)

    print(f"# warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    stage_ms = [sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
                for i in range(n_stage)]
    ms_per_step = elapsed * 1e3 / args.steps
    eager_ms_per_step = None
    if args.graph:
        # one step captured on torch's capture stream (the library launches on
        # the current stream and only launches kernels), then replayed
        print(f"# capturing one step, timing {args.steps} replays", file=sys.stderr, flush=True)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            stream = torch.cuda.current_stream()
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            stream = torch.cuda.current_stream()
            step()
        stream = torch.cuda.current_stream()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        eager_ms_per_step = ms_per_step
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # the same steps from cold caches: 1 GiB written before each step evicts the
    # L2s and the 256 MB Infinity Cache; timed by the events only
    cold_ms = None
    n_cold = min(args.steps if args.cold_steps < 0 else args.cold_steps, args.steps)
    if not args.backward and n_cold > 0:
        print(f"# timing {n_cold} cold-cache steps", file=sys.stderr, flush=True)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for s in range(n_cold):
            flush.fill_(s & 0xFF)
            step(ev[s])
        torch.cuda.synchronize()
        cold_ms = [sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(n_cold)) / n_cold
                   for i in range(n_stage)]
        del flush
    tokens = cfg.batch * (1 if cfg.decode else cfg.q_len)
    value = tokens / (ms_per_step / 1e3)

    a_flops = sum(attn_work(c)[0] for c in parts)
    a_bytes = sum(attn_work(c)[1] for c in parts)
    if lengths:
        # each sequence's pyramid: the nodes of a dense problem of its length
        b_bytes = sum(build_bytes(c, H.pyr_pyramid_nodes(H.Problem(
            1, c.n_q_heads, c.n_kv_heads, c.head_dim, c.q_len, c.kv_len, c.branching, c.top_k,
            c.dtype)), H.pyr_pyramid_planes(p)) for c in parts)
    else:
        b_bytes = build_bytes(cfg, H.pyr_pyramid_nodes(p), H.pyr_pyramid_planes(p))
    s_flops = sum(select_work(c, scored_candidates(c))[0] for c in parts)
    s_bytes = sum(select_work(c, scored_candidates(c))[1] for c in parts)
    t_build, t_sel, t_attn = (x / 1e3 for x in stage_ms[:3])
    if args.fused:   # one launch: the stage of the selection holds both
        t_sel = t_attn = stage_ms[1] / 1e3
    achieved = a_flops / t_attn / 1e12
    # the attention's matrix-core peak for its input type (bf16 or fp32 MFMA)
    peak_mfma = PEAK_BF16_TFLOPS if cfg.dtype == torch.bfloat16 else PEAK_FP32_TFLOPS
    # the attention's bound: MFMA where a gathered byte feeds many flops (bf16
    # with four or more query heads per KV head: 225 flop/B at 128K, 452 at 1M),
    # the gather bandwidth where it feeds few (bf16 with one head per KV head:
    # 59 flop/B) and for decode (one query row per head); the threshold of 100
    # flop/B for bf16 scales with the peak (6.3 flop/B for fp32)
    hbm_bound = cfg.decode or a_flops / a_bytes < 100 * peak_mfma / PEAK_BF16_TFLOPS
    traffic = kernel_traffic(cfg.name + ("_packed" if lengths else ""))
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded N(0,1) q/k/v with planted retrieval blocks)",
        "config": {
            "workload": cfg.name, "batch": cfg.batch, "q_heads": cfg.n_q_heads,
            "kv_heads": cfg.n_kv_heads, "q_len": cfg.q_len, "kv_len": cfg.kv_len,
            "head_dim": cfg.head_dim, "block": 64, "branching": cfg.branching,
            "top_k": cfg.top_k, "step": ("append+select+attn (pyramid of the cache maintained)"
                                         if cfg.decode else "build+select+attn"),
        },
        "roofline": {
            "kernel": attn_kernel_name(cfg, packed=bool(lengths)),
            "bound": "mfma" if not hbm_bound else "hbm",
            "achieved": round(achieved, 2) if not hbm_bound else round(a_bytes / t_attn / 1e9, 1),
            "peak": peak_mfma if not hbm_bound else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if not hbm_bound else "GB/s",
            "frac": round((achieved / peak_mfma) if not hbm_bound
                          else (a_bytes / t_attn / 1e9 / PEAK_HBM_GBS), 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": a_flops,
            "algorithmic_bytes_per_launch": a_bytes,
            "avg_launch_ms": round(stage_ms[2], 4),
        },
        "stages": {
            ("append" if cfg.decode else "build"): {"ms": round(stage_ms[0], 4), "GB/s": round(b_bytes / t_build / 1e9, 1) if t_build > 0 and not cfg.decode else None,
                      "hbm_frac": round(b_bytes / t_build / 1e9 / PEAK_HBM_GBS, 4) if t_build > 0 and not cfg.decode else None},
            "select": {"ms": round(stage_ms[1], 4), "GB/s": round(s_bytes / t_sel / 1e9, 1),
                       "TFLOP/s_fp32_equiv": round(s_flops / t_sel / 1e12, 2)},
            "attn": {"ms": round(stage_ms[2], 4), "TFLOP/s": round(achieved, 2),
                     "mfma_frac": round(achieved / peak_mfma, 4),
                     "GB/s_gathered": round(a_bytes / t_attn / 1e9, 1)},
            "build_plus_select_hbm_frac": (round((b_bytes + s_bytes) / (t_build + t_sel) / 1e9 / PEAK_HBM_GBS, 4)
                                           if not cfg.decode else None),
        },
        "cpu_baseline": None,
    }
    if args.graph:
        line["config"]["launch"] = "one step captured in a HIP graph, replayed"
        line["stages"]["eager_ms_per_step"] = round(eager_ms_per_step, 4)
    if not lengths:
        line["planted_recall"] = planted_recall(cfg, sel)
    tokens_sa = tokens / ((stage_ms[1] + stage_ms[2]) / 1e3)
    line["stages"]["tokens_per_s_select_attn_only"] = round(tokens_sa, 1)
    if cold_ms is not None:
        line["stages"]["cold_cache"] = {
            "note": "same steps after writing 1 GiB (L2 and Infinity Cache evicted); event time only",
            "ms_per_step": round(sum(cold_ms), 4),
            "stage_ms": [round(x, 4) for x in cold_ms],
        }
    if args.fused:
        # one kernel does the selection's scoring and the attention: its
        # algorithmic flops are both (scores counted once per dot product)
        f_flops = a_flops + s_flops
        t_f = stage_ms[1] / 1e3
        line["config"]["step"] = "build+select_attn (one fused launch)"
        line["roofline"] = {
            "kernel": "select_attend" if fused_kernel(cfg) else "select+attn (two launches)",
            "bound": "mfma",
            "achieved": round(f_flops / t_f / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(f_flops / t_f / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": kernel_traffic(cfg.name + ("_packed" if lengths else "") + "_fused"),
            "algorithmic_flops_per_launch": f_flops,
            "attention_flops": a_flops,
            "selection_flops": s_flops,
            "avg_launch_ms": round(stage_ms[1], 4),
        }
        line["stages"] = {
            "build": line["stages"]["build"],
            "select_attn": {"ms": round(stage_ms[1], 4), "TFLOP/s": round(f_flops / t_f / 1e12, 2)},
        }
    if lengths:
        line["metric"] = METRIC_PACKED
        line["config"].update({
            "workload": cfg.name + "_packed", "sequences": len(lengths),
            "q_len": max(lengths), "kv_len": max(lengths), "total_tokens": sum(lengths),
            "lengths": f"log-uniform in [{PACKED_SHORTEST}, {PACKED_LONGEST}], last cut to fit",
        })
    if args.backward:
        t_bwd = stage_ms[3] / 1e3
        b_flops = 5 * a_flops // 2
        line["metric"] = METRIC_BWD
        line["config"]["step"] = "build+select+attn+attn_bwd"
        line["roofline"] = {
            "kernel": "attn_bwd (dsum, route metadata, dq, dkdv, reduce)",
            "bound": "mfma",
            "achieved": round(b_flops / t_bwd / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(b_flops / t_bwd / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": kernel_traffic(cfg.name, "attn_bwd"),
            "algorithmic_flops_per_launch": b_flops,
            "avg_launch_ms": round(stage_ms[3], 4),
        }
        line["stages"]["attn_bwd"] = {"ms": round(stage_ms[3], 4),
                                      "TFLOP/s": round(b_flops / t_bwd / 1e12, 2)}
    if args.cpu_baseline_units > 0:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        # the backward costs the oracle about 2.5x the forward: a third of the units
        n_units = max(4, args.cpu_baseline_units // 3) if args.backward else args.cpu_baseline_units
        if lengths:
            # the oracle on the longest sequence alone, at that sequence's tokens/s
            i = max(range(len(lengths)), key=lambda j: lengths[j])
            a0 = sum(lengths[:i])
            views = [x[:, a0:a0 + lengths[i]].unsqueeze(0) for x in (q, k, v)]
            line["cpu_baseline"] = cpu_baseline(parts[i], *views, n_units)
            line["cpu_baseline"]["sample"] += f" (longest sequence, {lengths[i]} tokens)"
        else:
            line["cpu_baseline"] = cpu_baseline(cfg, q, k, v, n_units, backward=args.backward)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
