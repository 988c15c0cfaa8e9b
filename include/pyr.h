/*
 * pyr.h -- C ABI of libpyr: pyramid top-K block selection followed by
 * block-sparse causal attention, on AMD Instinct MI355X (gfx950).
 *
 * The method (PISA, peercurrent.com record of the PISA preprint, abstract):
 * keys are mean-pooled into a coarse-to-fine pyramid of O(log N) levels;
 * selection starts at the coarsest level, scores a bounded candidate set per
 * level with LogSumExp over the query block, keeps the top K and descends to
 * their children, down to 64-token key blocks; attention then runs exactly,
 * with an online softmax, over the selected blocks only.  The selected blocks
 * are strictly preceding ones and unused route slots hold -1 (PHBA:
 * Prefix-State Hybrid Block Attention, paperlayer.ai summary, §A.1.2); the
 * query's own block always supplies local causal attention (PHBA §3.1); the
 * attention writes its output and log-sum-exp (PHBA §A.1.3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, row-major [B, H, T, d]; a 64-token tile of one head is
 *    one contiguous chunk.  Query head h belongs to KV head h / (Hq / Hk).
 *  - Every tensor pointer is a DEVICE pointer, 16-byte aligned, owned by the
 *    caller.  The library never allocates, frees or synchronises, and keeps no
 *    state beyond a thread-local error string.
 *  - Work is enqueued on the given HIP stream (NULL = the default stream) and
 *    runs asynchronously; device faults surface at the caller's next
 *    synchronising call.
 *  - Outputs are fully overwritten (including -1 padding); callers need not
 *    clear them.
 *  - Arguments are validated before anything is enqueued: any status other
 *    than PYR_OK / PYR_ERR_HIP means nothing was launched.  PYR_ERR_HIP means
 *    a launch failed; pyr_last_error() holds the HIP error text.
 *  - Entry points are reentrant; concurrent calls on different streams are
 *    independent.
 *  - A unit is (batch, KV head, query block); all query heads of a KV group
 *    share the unit's selection, and the LogSumExp of a unit runs over the
 *    rows of all those heads.
 *  - Prefill: q_len == kv_len, query block i holds tokens [64i, 64i+64) and
 *    its diagonal block is i.  Decode: q_len == 1 with kv_len > 1, the single
 *    query token sits at position kv_len-1, and there is one query block whose
 *    diagonal block is (kv_len-1)/64.  Other q_len are PYR_ERR_UNSUPPORTED.
 *    kv_len need not be a multiple of 64: a ragged last block is pooled over
 *    its valid tokens and masked beyond kv_len.
 *
 * Packed sequences (pyr_problem.cu != NULL; prefill only)
 * --------------------------------------------------------
 *  - q, o are [Hq, total_len, d], k, v are [Hk, total_len, d] and lse is
 *    [Hq, total_len]: every head holds the sequences back to back, sequence s
 *    in rows [cu[s], cu[s+1]).  Rows outside every sequence are neither read
 *    nor written.
 *  - Each sequence is its own problem of length n_s = cu[s+1] - cu[s]: its
 *    64-token blocks start at its first row, its pyramid pools only its own
 *    keys, selection and attention never leave it, and a ragged last block
 *    is pooled over its valid rows.  The results are those of a dense problem
 *    of batch 1 and length n_s for every s.
 *  - The pyramid is [batch, Hk, P, nodes, d] and sel is [batch, Hk, nqb, K+1]
 *    with the layout a dense problem of length kv_len (the bound) has; route
 *    rows of query blocks past a sequence's end hold -1 only (trace rows -1
 *    and NaN), and pyramid nodes past its valid levels are left unwritten.
 *  - The offsets are read on the device, so the host cannot check them:
 *    offsets that break the rules above give unspecified results, but every
 *    access stays inside the tensors (offsets are clipped to [0, total_len]
 *    and lengths to kv_len).
 *  - pyr_append_pyramid and pyr_block_sparse_attn_bwd take no packed
 *    sequences (PYR_ERR_UNSUPPORTED).
 */
#ifndef PYR_H_
#define PYR_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PYR_ABI_VERSION 5

/* Bytes of the fixed per-device scratch array of pyr_block_sparse_attn_noalloc. */
#define PYR_NOALLOC_SCRATCH_BYTES (16u << 20)

typedef enum pyr_status {
  PYR_OK = 0,
  PYR_ERR_NULL = 1,        /* a required pointer is NULL                        */
  PYR_ERR_INVALID = 2,     /* a size or parameter is out of range               */
  PYR_ERR_UNSUPPORTED = 3, /* valid, but outside what this library implements   */
  PYR_ERR_MISALIGNED = 4,  /* a tensor pointer is not 16-byte aligned           */
  PYR_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required        */
  PYR_ERR_HIP = 6          /* a HIP launch failed (text in pyr_last_error)      */
} pyr_status;

typedef enum pyr_dtype {
  PYR_F32 = 0,  /* IEEE binary32 */
  PYR_BF16 = 1  /* bfloat16      */
} pyr_dtype;

typedef struct pyr_problem {
  int32_t batch;       /* B >= 0                                              */
  int32_t n_q_heads;   /* Hq >= 1, a multiple of n_kv_heads                   */
  int32_t n_kv_heads;  /* Hk >= 1                                             */
  int32_t head_dim;    /* d: 64 or 128                                        */
  int64_t q_len;       /* Tq: == kv_len (prefill) or 1 (decode)               */
  int64_t kv_len;      /* Tk >= 0                                             */
  int32_t block;       /* tokens per query and key block: must be 64          */
  int32_t branching;   /* b >= 2: children per pyramid node                   */
  int32_t top_k;       /* K >= 1: nodes kept per level; the diagonal block is
                          added on top, so a route row has K+1 slots          */
  int32_t dtype;       /* pyr_dtype of q, k, v and o                          */
  float scale;         /* softmax and scoring scale; 0 => 1/sqrt(head_dim)    */
  int64_t kv_capacity; /* tokens the pyramid layout is sized for: 0 => kv_len,
                          else >= kv_len.  Level count, level offsets and node
                          count follow the capacity, the valid nodes of each
                          level follow kv_len, so a pyramid can grow by
                          pyr_append_pyramid without moving (decode)          */
  const int32_t* cu;   /* NULL: a dense batch.  Else a packed batch of `batch`
                          sequences (PHBA §A.1.1-§A.1.2: packed inputs, block
                          boundaries from cu and the block size): a DEVICE
                          array of batch+1 int32 row offsets, cu[0] = 0,
                          nondecreasing, cu[batch] <= total_len; sequence s
                          owns rows [cu[s], cu[s+1]) of every head.  Needs
                          q_len == kv_len = a bound on every sequence's length
                          and kv_capacity == 0.  See "Packed sequences".      */
  int64_t total_len;   /* packed: rows per head of q, k, v, o and lse; 0 when
                          cu is NULL                                          */
} pyr_problem;

/* ---- geometry helpers (host-only, no device work; -1 on invalid input) ---- */

/* PISA abstract: keys are pooled into O(log N) levels, each coarser level
 * pooling b nodes of the one below.  Number of pyramid levels L, finest
 * (64-token blocks) to the single root:
 * n_0 = ceil(C/64), n_{l+1} = ceil(n_l / b) until n = 1, with C the capacity
 * (kv_capacity, or kv_len when that is 0).  Levels above the root of the valid
 * keys hold one node: the mean of all of them. */
int32_t pyr_num_levels(const pyr_problem* p);
/* Node offset of a level inside one (batch, KV head) pyramid slab (finest
 * level first; levels are concatenated; PISA abstract, pooled levels). */
int64_t pyr_level_offset(const pyr_problem* p, int32_t level);
/* Nodes per (batch, KV head) slab: sum of all level sizes at the capacity
 * (PISA abstract: O(N) pooled nodes over the O(log N) levels). */
int64_t pyr_pyramid_nodes(const pyr_problem* p);
/* Planes of a pyramid slab: 1 for float32 problems, 2 for bfloat16 problems
 * (plane 1 repeats plane 0 split into bfloat16 pairs, see pyr_build_pyramid;
 * PHBA §A.1.2 keeps block summaries in fp32). */
int32_t pyr_pyramid_planes(const pyr_problem* p);
/* Query blocks per (batch, KV head): ceil(q_len/64) in prefill, 1 in decode
 * (PISA abstract: selection runs per query block). */
int64_t pyr_num_query_blocks(const pyr_problem* p);
/* Bytes of device workspace pyr_block_sparse_attn uses (0 if none).
 *  - Decode splits a unit's selected blocks over several workgroups and
 *    merges their partial online-softmax states there (PHBA §A.1.3 keeps
 *    those accumulators on chip within one query tile; decode has one query
 *    token per unit, so its blocks are split to fill the GPU).  Decode
 *    requires it.
 *  - Dense bfloat16 prefill with G = q_heads / kv_heads a multiple of 4 and
 *    (top_k + 1) * G / 4 >= 16 (every block of v then feeds enough
 *    workgroups for a transposed copy to pay for its HBM round trip) may
 *    take B * kv_heads * ceil(kv_len/64) * 64 * head_dim * 2 bytes for a
 *    block-transposed copy of v, which the attention reads in place of v.
 *    Optional: with a NULL or smaller workspace the kernels read v directly,
 *    and o and lse are the same bits either way.
 * Other problems use none. */
size_t pyr_attn_workspace_bytes(const pyr_problem* p);

/* ---- the hot path ---- */

/* Pooled key pyramid (PISA abstract: pooling builds the coarse-to-fine key
 * levels; PHBA §A.1.2: block means over valid rows, fp32 accumulation).
 *   k        [B, Hk, kv_len, d] in p->dtype                          (input)
 *   pyramid  [B, Hk, P, pyr_pyramid_nodes(p), d] float32,
 *            P = pyr_pyramid_planes(p)                                (output)
 * Plane 0: node m of level l is the mean of every key token it covers (blocks
 * [m b^l, (m+1) b^l) clipped to the sequence); levels are concatenated finest
 * first at pyr_level_offset(p, l).  Plane 1 (bfloat16 problems only): the
 * 4d bytes of node row m hold the same d means as two bfloat16 rows,
 * hi = bf16(x) then lo = bf16(x - hi) (round to nearest even), which the
 * matrix-core scorer of pyr_select_topk reads; hi + lo is x to within 2^-17
 * relative. */
pyr_status pyr_build_pyramid(const pyr_problem* p, const void* k, float* pyramid,
                             hipStream_t stream);

/* Coarse-to-fine top-K selection (PISA abstract).  For every unit, starting at
 * the root: the candidates of a level are the children of the nodes kept one
 * level up plus the children of the diagonal block's ancestor that lie wholly
 * before the diagonal block's ancestor at this level; nodes that reach the
 * diagonal block are never candidates.  With more than K candidates each is
 * scored s(n) = log sum_r exp(scale * q_r . P_l[n]) over the unit's rows and
 * the K best are kept (equal scores: lower index first); otherwise all are
 * kept.  No query-by-key score matrix is written to memory.
 *   q            [B, Hq, q_len, d] in p->dtype                       (input)
 *   pyramid      output of pyr_build_pyramid for the same problem     (input)
 *   sel          [B, Hk, nqb, K+1] int32: the finest kept blocks in ascending
 *                order, then the diagonal block, then -1 padding      (output)
 *   trace_ids    NULL or [B, Hk, nqb, L, K] int32: kept node ids of every
 *                level (finest first), ascending, -1 padded           (output)
 *   trace_scores NULL or [B, Hk, nqb, L, K+1] float32: the scores of those
 *                kept nodes in the same order, then the best rejected score;
 *                NaN where a level was not scored or a slot is unused (output)
 * Ranking does not depend on the traces: with or without trace_scores the
 * kept sets, route rows and trace_ids are the same, bit for bit (without it,
 * and without a fallback, the kernel ranks by counting on all its waves
 * instead of recording scores and margins on one).
 */
pyr_status pyr_select_topk(const pyr_problem* p, const void* q, const float* pyramid,
                           int32_t* sel, int32_t* trace_ids, float* trace_scores,
                           hipStream_t stream);

/* Selection with per-head budgets and a confidence fallback (PHAROS, zensar.com
 * summary: token budgets differ between attention heads (depth-sounding budget
 * allocation) and the budget grows when the selection is not confident (fog
 * gate confidence fallback); the page gives no formulas, so the two rules
 * below are this library's).  Same as pyr_select_topk except:
 *   k_head        NULL (every unit keeps K nodes per level) or a DEVICE array
 *                 [Hk] int32: units of KV head hk keep K_h = k_head[hk] nodes
 *                 per level, clamped to [1, K] on the device  (input)
 *   fallback_k    0 (no fallback) or F in [1, K]: when the finest level was
 *                 scored (more than K_h candidates) and its margin -- the K_h-th
 *                 best score minus the best rejected score, natural-log
 *                 LogSumExp units -- is below fallback_margin, the unit keeps
 *                 the best min(F, candidates) of that level instead; F <= K_h
 *                 has no effect
 *   fallback_margin  finite; a margin below it triggers the fallback
 * Route rows keep their K+1 slots (kept blocks, diagonal, -1 padding); trace
 * rows list K_h ids per level (F at a finest level that fell back), -1 and
 * NaN after them.  The margin is computed from the kernel's fp32 scores, so a
 * unit whose margin lies within rounding of fallback_margin may go either way.
 * PYR_ERR_INVALID for fallback_k outside [0, K] or a non-finite margin,
 * PYR_ERR_MISALIGNED for a k_head that is not 4-byte aligned. */
pyr_status pyr_select_topk_budgets(const pyr_problem* p, const void* q, const float* pyramid,
                                   const int32_t* k_head, int32_t fallback_k,
                                   float fallback_margin, int32_t* sel, int32_t* trace_ids,
                                   float* trace_scores, hipStream_t stream);

/* Host-only helper for per-head budgets (no device work): K_h =
 * clamp(round(total * entropy[h] / sum(entropy)), k_min, k_max) -- budgets in
 * proportion to each head's attention entropy (a head whose attention is
 * spread out gets more blocks), an equal split when every entropy is 0.
 * entropy and k_out are HOST arrays of n_heads entries.  PYR_ERR_INVALID for
 * n_heads < 0, k_min < 1, k_max < k_min, total < 0 or an entropy that is
 * negative or not finite. */
pyr_status pyr_budgets_from_entropy(const float* entropy, int32_t n_heads, int32_t total,
                                    int32_t k_min, int32_t k_max, int32_t* k_out);

/* Exact attention over the selected blocks (PHBA §A.1.3: online-softmax
 * accumulation over routed blocks loaded straight from their original
 * layouts, writing output and log-sum-exp).  Query token t at position
 * pos(t) attends to every key s <= pos(t) of the blocks listed in its unit's
 * route row.  A route row is a set: entries < 0 are ignored and a block
 * listed more than once is attended once.
 *   q, k, v    [B, Hq, q_len, d], [B, Hk, kv_len, d] x2, p->dtype    (input)
 *   sel        [B, Hk, nqb, K+1] int32 route rows (any valid block ids;
 *              pyr_select_topk writes them)                          (input)
 *   o          [B, Hq, q_len, d] in p->dtype                         (output)
 *   lse        NULL or [B, Hq, q_len] float32, natural log            (output)
 *   workspace  device scratch, 16-byte aligned, of workspace_bytes.  Decode
 *              requires workspace_bytes >= pyr_attn_workspace_bytes(p)
 *              (PYR_ERR_WORKSPACE otherwise); for prefill the workspace is
 *              optional and used only when it holds
 *              pyr_attn_workspace_bytes(p) bytes (then the kernel reads a
 *              transposed copy of v it writes there; results are
 *              identical).  May be NULL when not required.  Its contents on
 *              entry do not matter and on return are unspecified.
 * Route entries outside [0, ceil(kv_len/64)) are ignored (the host cannot read
 * device route rows without synchronising, so they are not an error). */
pyr_status pyr_block_sparse_attn(const pyr_problem* p, const void* q, const void* k,
                                 const void* v, const int32_t* sel, void* o, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* pyr_block_sparse_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that must not call hipMalloc, and
 * harnesses that forbid allocation.  Same arguments, results and errors as
 * pyr_block_sparse_attn without the workspace (prefill reads v directly, as
 * with a NULL workspace): when the problem needs one (decode), its partial
 * states go to a
 * device array of PYR_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds
 * on every GPU it runs on until the process ends (64 sequences x 8 KV heads x
 * 4 query heads per KV head at top_k = 64 and head_dim = 128 take 9.6 MB).
 * Problems that need more return PYR_ERR_WORKSPACE before anything is
 * enqueued.  Nothing is allocated or freed; the first call on a device looks
 * up that device's array.  Every call on a GPU shares its array and leaves its
 * contents behind (each call writes every partial it reads), so calls that
 * can overlap on one GPU -- on different streams, or from several threads --
 * race and must be ordered by the caller. */
pyr_status pyr_block_sparse_attn_noalloc(const pyr_problem* p, const void* q, const void* k,
                                         const void* v, const int32_t* sel, void* o,
                                         float* lse, hipStream_t stream);

/* Selection and attention in one call (PISA abstract: the kernels fuse the
 * hierarchical routing with the LogSumExp scoring; PHBA §A.1.3: the forward
 * kernel works straight from the query-centric routes).  Arguments as in
 * pyr_select_topk and pyr_block_sparse_attn: q, k, v, pyramid (inputs), sel,
 * trace_ids, trace_scores (NULL allowed for the traces), o, lse (NULL
 * allowed) and the attention's workspace (outputs / scratch).
 * For bfloat16 prefill problems with four query heads per KV head and
 * branching * (top_k + 1) <= 192 (the selection's on-chip state then fits in
 * one of the attention's tile slots), one launch runs both steps per unit: the
 * route reaches the attention in LDS (and is written to sel), and the unit's
 * q is fetched from HBM once.  The route is the coarse-to-fine top-K of
 * pyr_select_topk; its scores are summed over the unit's rows in another
 * order, so a unit may differ from pyr_select_topk's route where two scores
 * tie within fp32 rounding.  o and lse are, bit for bit, what
 * pyr_block_sparse_attn computes over the sel written.  Other problems run
 * pyr_select_topk's and pyr_block_sparse_attn's kernels in turn.  Errors as
 * for those two calls. */
pyr_status pyr_select_attn(const pyr_problem* p, const void* q, const void* k, const void* v,
                           const float* pyramid, int32_t* sel, int32_t* trace_ids,
                           float* trace_scores, void* o, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---- decode: pyramid maintenance ---- */

/* Bring a pyramid up to date after keys were appended (PISA abstract: a node's
 * pooled key is the mean of the keys under it, so appending keys changes only
 * the nodes over the new tokens).  p describes the state after the append
 * (kv_len = new length); the pyramid was built or last appended for old_len
 * tokens with the same capacity, and k now holds tokens [0, kv_len) of every
 * (batch, KV head).  Every node whose token range meets [old_len, kv_len) is
 * recomputed — level-0 nodes as the mean of their valid keys, higher nodes as
 * the token-weighted mean of their children — and every other node is left as
 * it is, so the result equals pyr_build_pyramid for kv_len tokens (up to fp32
 * rounding order).  Requires 0 < old_len <= kv_len <= capacity (else
 * PYR_ERR_INVALID); old_len == kv_len is a no-op.  Work grows with the number
 * of new blocks: meant for decode steps and short chunks (a long prefill is
 * cheaper through pyr_build_pyramid).
 *   k        [B, Hk, kv_len, d] in p->dtype (rows of the capacity beyond kv_len
 *            may follow; only [0, kv_len) is read)                    (input)
 *   pyramid  the layout of pyr_build_pyramid for p             (input/output) */
pyr_status pyr_append_pyramid(const pyr_problem* p, const void* k, int64_t old_len,
                              float* pyramid, hipStream_t stream);

/* ---- training: backward of the attention for a fixed route table ---- */

/* Bytes of device workspace pyr_block_sparse_attn_bwd needs (0 on invalid
 * input): a 512-byte record per (batch, query head, query block), the
 * block-major route metadata (a bitmap of ceil(nqb/32) uint32 per key block,
 * counts and a work list) and fp32 partial sums for key blocks that many query
 * blocks use; the partial area is sized for the worst case the route shape
 * allows, 2 * B * Hk * nqb * (K+1) / c slots of 64 * d * 8 bytes, where c is
 * the number of query blocks per work item (1 .. 256/G, larger for larger
 * problems). */
size_t pyr_attn_bwd_workspace_bytes(const pyr_problem* p);

/* Gradients of pyr_block_sparse_attn with respect to q, k and v (PHBA §A.1.4:
 * sparse backward for a fixed route; the kernels rebuild P on chip from the
 * forward's log-sum-exp and list, for each key block, the query blocks that
 * route to it when they form the key gradients).  With P the
 * forward's probabilities over each row's visible keys, dP = dout v^T,
 * D = rowsum(dout * o) and dS = P * (dP - D):
 *   dq = scale dS k,   dk = scale dS^T q,   dv = P^T dout,
 * where dk and dv of a KV head sum the contributions of its G query heads.
 * Prefill, bfloat16 only (else PYR_ERR_UNSUPPORTED); fp32 accumulation, one
 * bfloat16 rounding per output.
 *   q, k, v    the forward's inputs, shapes as in pyr_block_sparse_attn (input)
 *   sel        the forward's route rows [B, Hk, nqb, K+1]; entries outside
 *              [0, ceil(kv_len/64)) are ignored and a block listed more
 *              than once counts once, as in the forward            (input)
 *   o, lse     the forward's output [B, Hq, q_len, d] and log-sum-exp
 *              [B, Hq, q_len] float32 (both required)                  (input)
 *   dout       dL/do, [B, Hq, q_len, d] bfloat16                       (input)
 *   dq         [B, Hq, q_len, d] bfloat16                              (output)
 *   dk, dv     [B, Hk, kv_len, d] bfloat16; keys no row sees get 0     (output)
 *   workspace  device scratch of workspace_bytes >=
 *              pyr_attn_bwd_workspace_bytes(p), 16-byte aligned; its
 *              contents on entry do not matter.
 * A row whose lse is not finite (it saw no key) gets a zero dq and adds
 * nothing to dk and dv.  The result does not depend on scheduling: no
 * gradient is accumulated with atomics, so repeated calls give identical bits. */
pyr_status pyr_block_sparse_attn_bwd(const pyr_problem* p, const void* q, const void* k,
                                     const void* v, const int32_t* sel, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk,
                                     void* dv, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* ---- diagnostics ---- */
const char* pyr_status_string(pyr_status s);
/* Thread-local detail of the last non-OK return on this thread ("" if none). */
const char* pyr_last_error(void);
int32_t pyr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PYR_H_ */
