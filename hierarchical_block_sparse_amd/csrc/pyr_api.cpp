// Host side of the libpyr C ABI: argument validation, geometry, dispatch.
// Every check runs before anything is enqueued; nothing here allocates,
// synchronises or keeps state beyond a thread-local error message.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/pyr.h"
#include "pyr_internal.h"

namespace {

thread_local char g_err[512] = "";

pyr_status fail(pyr_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Level sizes finest -> root; returns L or -1 if it would not fit.
int level_sizes(int64_t nb, int64_t b, int32_t* sizes, int64_t* offs, int64_t* n_tot) {
  if (nb <= 0) {
    *n_tot = 0;
    return 0;
  }
  int L = 0;
  int64_t n = nb, off = 0;
  for (;;) {
    if (L >= PYR_MAX_LEVELS) return -1;
    if (sizes) sizes[L] = (int32_t)n;
    if (offs) offs[L] = off;
    off += n;
    ++L;
    if (n == 1) break;
    n = (n + b - 1) / b;
  }
  *n_tot = off;
  return L;
}

// Shape checks shared by every entry point.  Fills g on success.
pyr_status resolve(const pyr_problem* p, PyrGeom* g) {
  if (!p) return fail(PYR_ERR_NULL, "problem is NULL");
  if (p->batch < 0) return fail(PYR_ERR_INVALID, "batch %d < 0", p->batch);
  if (p->n_kv_heads < 1 || p->n_q_heads < 1)
    return fail(PYR_ERR_INVALID, "head counts must be >= 1 (Hq=%d, Hk=%d)", p->n_q_heads,
                p->n_kv_heads);
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(PYR_ERR_INVALID, "n_q_heads %d is not a multiple of n_kv_heads %d",
                p->n_q_heads, p->n_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PYR_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", p->head_dim);
  if (p->block != PYR_BLOCK) return fail(PYR_ERR_UNSUPPORTED, "block %d (supported: 64)", p->block);
  if (p->branching < 2) return fail(PYR_ERR_INVALID, "branching %d < 2", p->branching);
  if (p->branching > 64) return fail(PYR_ERR_UNSUPPORTED, "branching %d > 64", p->branching);
  if (p->top_k < 1) return fail(PYR_ERR_INVALID, "top_k %d < 1", p->top_k);
  if (p->top_k > 1023) return fail(PYR_ERR_UNSUPPORTED, "top_k %d > 1023", p->top_k);
  if ((int64_t)p->branching * (p->top_k + 1) > 8192)
    return fail(PYR_ERR_UNSUPPORTED, "branching*(top_k+1) = %lld > 8192 candidates per level",
                (long long)p->branching * (p->top_k + 1));
  if (p->dtype != PYR_F32 && p->dtype != PYR_BF16)
    return fail(PYR_ERR_INVALID, "dtype %d", p->dtype);
  if (p->kv_len < 0 || p->q_len < 0) return fail(PYR_ERR_INVALID, "negative length");
  if (p->kv_len > ((int64_t)1 << 36)) return fail(PYR_ERR_UNSUPPORTED, "kv_len > 2^36");
  if (p->kv_capacity != 0 && p->kv_capacity < p->kv_len)
    return fail(PYR_ERR_INVALID, "kv_capacity %lld < kv_len %lld", (long long)p->kv_capacity,
                (long long)p->kv_len);
  if (p->kv_capacity > ((int64_t)1 << 36)) return fail(PYR_ERR_UNSUPPORTED, "kv_capacity > 2^36");
  const bool prefill = p->q_len == p->kv_len;
  const bool decode = p->q_len == 1 && p->kv_len > 1;
  if (!prefill && !decode)
    return fail(PYR_ERR_UNSUPPORTED, "q_len %lld with kv_len %lld (need q_len == kv_len or q_len == 1)",
                (long long)p->q_len, (long long)p->kv_len);
  if (!(p->scale >= 0.f) || isinf(p->scale)) return fail(PYR_ERR_INVALID, "scale must be finite and >= 0");
  if (p->cu) {
    if (!prefill)
      return fail(PYR_ERR_UNSUPPORTED,
                  "packed sequences need q_len == kv_len (the bound on every sequence's length)");
    if (p->kv_capacity != 0)
      return fail(PYR_ERR_UNSUPPORTED, "packed sequences take no kv_capacity");
    if (p->total_len < 0) return fail(PYR_ERR_INVALID, "total_len %lld < 0", (long long)p->total_len);
    if (p->total_len > ((int64_t)1 << 36)) return fail(PYR_ERR_UNSUPPORTED, "total_len > 2^36");
    if (reinterpret_cast<uintptr_t>(p->cu) & 3u)
      return fail(PYR_ERR_MISALIGNED, "cu must be 4-byte aligned");
  } else if (p->total_len != 0) {
    return fail(PYR_ERR_INVALID, "total_len %lld without cu (dense problems take 0)",
                (long long)p->total_len);
  }

  memset(g, 0, sizeof *g);
  g->Tq = p->q_len;
  g->Tk = p->kv_len;
  g->B = p->batch;
  g->Hq = p->n_q_heads;
  g->Hk = p->n_kv_heads;
  g->G = p->n_q_heads / p->n_kv_heads;
  g->D = p->head_dim;
  g->nb = (int32_t)((p->kv_len + PYR_BLOCK - 1) / PYR_BLOCK);
  g->decode = decode ? 1 : 0;
  g->nqb = decode ? 1 : (int32_t)((p->q_len + PYR_BLOCK - 1) / PYR_BLOCK);
  g->branching = p->branching;
  g->K = p->top_k;
  g->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  g->planes = p->dtype == PYR_BF16 ? 2 : 1;
  // layout (level count, offsets, node count) from the capacity; valid nodes
  // per level from kv_len (one node, the mean of everything, above its root).
  // Packed sequences: every slab is laid out for the length bound kv_len, and
  // every head of q, k, v, o and lse holds total_len rows.
  g->cu = p->cu;
  g->Tks = p->cu ? p->total_len : (p->kv_capacity ? p->kv_capacity : p->kv_len);
  g->Tqs = p->cu ? p->total_len : p->q_len;
  const int64_t nb_cap = ((p->cu ? p->kv_len : g->Tks) + PYR_BLOCK - 1) / PYR_BLOCK;
  const int L = level_sizes(nb_cap, p->branching, nullptr, g->loff, &g->n_tot);
  if (L < 0) return fail(PYR_ERR_UNSUPPORTED, "more than %d pyramid levels", PYR_MAX_LEVELS);
  g->L = L;
  for (int64_t l = 0, n = g->nb; l < L; ++l) {
    g->lsize[l] = (int32_t)n;
    n = n > 1 ? (n + p->branching - 1) / p->branching : n;
  }
  if (g->G > 128)
    return fail(PYR_ERR_UNSUPPORTED, "at most 128 query heads per KV head (G=%d)", g->G);
  if (decode && g->G > 16)
    return fail(PYR_ERR_UNSUPPORTED, "decode supports at most 16 query heads per KV head (G=%d)", g->G);
  return PYR_OK;
}

pyr_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PYR_OK;
  return fail(PYR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

pyr_status select_checked(const PyrGeom& g, int dtype, const void* q, const float* pyramid,
                          int32_t* sel, int32_t* trace_ids, float* trace_scores,
                          hipStream_t stream) {
  const bool empty = (int64_t)g.B * g.Hk * g.nqb == 0 || g.Tq == 0 || (g.cu && g.Tqs == 0);
  if (!empty && (!q || !pyramid || !sel)) return fail(PYR_ERR_NULL, "q, pyramid or sel is NULL");
  if (!empty && (!aligned16(q) || !aligned16(pyramid) || !aligned16(sel) ||
                 (trace_ids && !aligned16(trace_ids)) || (trace_scores && !aligned16(trace_scores))))
    return fail(PYR_ERR_MISALIGNED, "tensors must be 16-byte aligned");
  if (empty) return PYR_OK;
  if (pyr_select_lds_bytes(g, dtype) > 160 * 1024)
    return fail(PYR_ERR_UNSUPPORTED, "selection needs %zu bytes of LDS (> 160 KiB)",
                pyr_select_lds_bytes(g, dtype));
  return hip_status(pyr_launch_select(g, dtype, q, pyramid, sel, trace_ids, trace_scores, stream),
                    "pyr_select_topk launch");
}

}  // namespace

extern "C" {

int32_t pyr_num_levels(const pyr_problem* p) {
  PyrGeom g;
  return resolve(p, &g) == PYR_OK ? g.L : -1;
}

int64_t pyr_level_offset(const pyr_problem* p, int32_t level) {
  PyrGeom g;
  if (resolve(p, &g) != PYR_OK || level < 0 || level >= g.L) return -1;
  return g.loff[level];
}

int64_t pyr_pyramid_nodes(const pyr_problem* p) {
  PyrGeom g;
  return resolve(p, &g) == PYR_OK ? g.n_tot : -1;
}

int32_t pyr_pyramid_planes(const pyr_problem* p) {
  PyrGeom g;
  return resolve(p, &g) == PYR_OK ? g.planes : -1;
}

int64_t pyr_num_query_blocks(const pyr_problem* p) {
  PyrGeom g;
  return resolve(p, &g) == PYR_OK ? g.nqb : -1;
}

size_t pyr_attn_workspace_bytes(const pyr_problem* p) {
  PyrGeom g;
  return resolve(p, &g) == PYR_OK ? pyr_attn_ws_bytes(g) + pyr_attn_vt_bytes(g, p->dtype) : 0;
}

pyr_status pyr_build_pyramid(const pyr_problem* p, const void* k, float* pyramid,
                             hipStream_t stream) {
  g_err[0] = 0;
  PyrGeom g;
  pyr_status s = resolve(p, &g);
  if (s != PYR_OK) return s;
  const bool empty = (int64_t)g.B * g.Hk == 0 || g.nb == 0 || (g.cu && g.Tks == 0);
  if (!empty && (!k || !pyramid)) return fail(PYR_ERR_NULL, "k or pyramid is NULL");
  if (!empty && (!aligned16(k) || !aligned16(pyramid)))
    return fail(PYR_ERR_MISALIGNED, "k and pyramid must be 16-byte aligned");
  if (empty) return PYR_OK;
  return hip_status(pyr_launch_build(g, p->dtype, k, pyramid, stream), "pyr_build_pyramid launch");
}

pyr_status pyr_select_topk(const pyr_problem* p, const void* q, const float* pyramid,
                           int32_t* sel, int32_t* trace_ids, float* trace_scores,
                           hipStream_t stream) {
  g_err[0] = 0;
  PyrGeom g;
  pyr_status s = resolve(p, &g);
  if (s != PYR_OK) return s;
  return select_checked(g, p->dtype, q, pyramid, sel, trace_ids, trace_scores, stream);
}

pyr_status pyr_select_topk_budgets(const pyr_problem* p, const void* q, const float* pyramid,
                                   const int32_t* k_head, int32_t fallback_k,
                                   float fallback_margin, int32_t* sel, int32_t* trace_ids,
                                   float* trace_scores, hipStream_t stream) {
  g_err[0] = 0;
  PyrGeom g;
  pyr_status s = resolve(p, &g);
  if (s != PYR_OK) return s;
  if (fallback_k < 0 || fallback_k > g.K)
    return fail(PYR_ERR_INVALID, "fallback_k %d outside [0, top_k = %d]", fallback_k, g.K);
  if (isnan(fallback_margin) || isinf(fallback_margin))
    return fail(PYR_ERR_INVALID, "fallback_margin must be finite");
  if (k_head && (reinterpret_cast<uintptr_t>(k_head) & 3u))
    return fail(PYR_ERR_MISALIGNED, "k_head must be 4-byte aligned");
  g.k_head = k_head;
  g.fb_k = fallback_k;
  g.fb_margin = fallback_margin;
  return select_checked(g, p->dtype, q, pyramid, sel, trace_ids, trace_scores, stream);
}

pyr_status pyr_block_sparse_attn(const pyr_problem* p, const void* q, const void* k,
                                 const void* v, const int32_t* sel, void* o, float* lse,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  PyrGeom g;
  pyr_status s = resolve(p, &g);
  if (s != PYR_OK) return s;
  const bool empty = (int64_t)g.B * g.Hk * g.nqb == 0 || g.Tq == 0 || (g.cu && g.Tqs == 0);
  if (!empty && (!q || !k || !v || !sel || !o)) return fail(PYR_ERR_NULL, "q, k, v, sel or o is NULL");
  if (!empty && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sel) ||
                 !aligned16(o) || (lse && !aligned16(lse))))
    return fail(PYR_ERR_MISALIGNED, "tensors must be 16-byte aligned");
  const size_t need = pyr_attn_ws_bytes(g);
  if (!empty && need > 0 && (!workspace || workspace_bytes < need))
    return fail(PYR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!empty && workspace && (need > 0 || pyr_attn_vt_bytes(g, p->dtype) > 0) && !aligned16(workspace))
    return fail(PYR_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (empty) return PYR_OK;
  return hip_status(pyr_launch_attn(g, p->dtype, q, k, v, sel, o, lse, workspace,
                                    workspace ? workspace_bytes : 0, stream),
                    "pyr_block_sparse_attn launch");
}

pyr_status pyr_block_sparse_attn_noalloc(const pyr_problem* p, const void* q, const void* k,
                                         const void* v, const int32_t* sel, void* o,
                                         float* lse, hipStream_t stream) {
  g_err[0] = 0;
  PyrGeom g;
  pyr_status s = resolve(p, &g);
  if (s != PYR_OK) return s;
  const bool empty = (int64_t)g.B * g.Hk * g.nqb == 0 || g.Tq == 0 || (g.cu && g.Tqs == 0);
  if (!empty && (!q || !k || !v || !sel || !o)) return fail(PYR_ERR_NULL, "q, k, v, sel or o is NULL");
  if (!empty && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sel) ||
                 !aligned16(o) || (lse && !aligned16(lse))))
    return fail(PYR_ERR_MISALIGNED, "tensors must be 16-byte aligned");
  const size_t need = pyr_attn_ws_bytes(g);
  if (!empty && need > PYR_NOALLOC_SCRATCH_BYTES)
    return fail(PYR_ERR_WORKSPACE,
                "this problem needs %zu bytes of scratch; the allocation-free entry point holds "
                "%zu per device (use pyr_block_sparse_attn with a workspace)",
                need, (size_t)PYR_NOALLOC_SCRATCH_BYTES);
  if (empty) return PYR_OK;
  return hip_status(pyr_launch_attn_noalloc(g, p->dtype, q, k, v, sel, o, lse, stream),
                    "pyr_block_sparse_attn_noalloc launch");
}

pyr_status pyr_select_attn(const pyr_problem* p, const void* q, const void* k, const void* v,
                           const float* pyramid, int32_t* sel, int32_t* trace_ids,
                           float* trace_scores, void* o, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  PyrGeom g;
  pyr_status s = resolve(p, &g);
  if (s != PYR_OK) return s;
  const bool empty = (int64_t)g.B * g.Hk * g.nqb == 0 || g.Tq == 0 || (g.cu && g.Tqs == 0);
  if (!empty && (!q || !k || !v || !pyramid || !sel || !o))
    return fail(PYR_ERR_NULL, "q, k, v, pyramid, sel or o is NULL");
  if (!empty && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(pyramid) ||
                 !aligned16(sel) || !aligned16(o) || (lse && !aligned16(lse)) ||
                 (trace_ids && !aligned16(trace_ids)) ||
                 (trace_scores && !aligned16(trace_scores))))
    return fail(PYR_ERR_MISALIGNED, "tensors must be 16-byte aligned");
  const size_t need = pyr_attn_ws_bytes(g);
  if (!empty && need > 0 && (!workspace || workspace_bytes < need))
    return fail(PYR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!empty && workspace && (need > 0 || pyr_attn_vt_bytes(g, p->dtype) > 0) && !aligned16(workspace))
    return fail(PYR_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (empty) return PYR_OK;
  if (!pyr_select_attend_fused(g, p->dtype) && pyr_select_lds_bytes(g, p->dtype) > 160 * 1024)
    return fail(PYR_ERR_UNSUPPORTED, "selection needs %zu bytes of LDS (> 160 KiB)",
                pyr_select_lds_bytes(g, p->dtype));
  return hip_status(pyr_launch_select_attend(g, p->dtype, q, k, v, pyramid, sel, trace_ids,
                                             trace_scores, o, lse, workspace,
                                             workspace ? workspace_bytes : 0, stream),
                    "pyr_select_attn launch");
}

pyr_status pyr_append_pyramid(const pyr_problem* p, const void* k, int64_t old_len,
                              float* pyramid, hipStream_t stream) {
  g_err[0] = 0;
  PyrGeom g;
  pyr_status s = resolve(p, &g);
  if (s != PYR_OK) return s;
  if (g.cu) return fail(PYR_ERR_UNSUPPORTED, "pyr_append_pyramid takes no packed sequences");
  if (old_len <= 0 || old_len > g.Tk)
    return fail(PYR_ERR_INVALID, "old_len %lld outside (0, kv_len = %lld]", (long long)old_len,
                (long long)g.Tk);
  // Without a capacity the layout follows the length itself: the pyramid of
  // old_len has the layout of the new length only when both lengths cover
  // the same number of 64-token blocks (else every level above the finest
  // moves, and so does the slab stride).
  if (p->kv_capacity == 0 &&
      (old_len + PYR_BLOCK - 1) / PYR_BLOCK != (g.Tk + PYR_BLOCK - 1) / PYR_BLOCK)
    return fail(PYR_ERR_INVALID,
                "old_len %lld and kv_len %lld cover different block counts: the pyramid's "
                "layout would change; pass the same kv_capacity (>= kv_len) to the build and "
                "every append",
                (long long)old_len, (long long)g.Tk);
  if ((int64_t)g.B * g.Hk == 0 || old_len == g.Tk) return PYR_OK;
  if (!k || !pyramid) return fail(PYR_ERR_NULL, "k or pyramid is NULL");
  if (!aligned16(k) || !aligned16(pyramid))
    return fail(PYR_ERR_MISALIGNED, "tensors must be 16-byte aligned");
  return hip_status(pyr_launch_append(g, p->dtype, k, old_len, pyramid, stream),
                    "pyr_append_pyramid launch");
}

size_t pyr_attn_bwd_workspace_bytes(const pyr_problem* p) {
  PyrGeom g;
  return resolve(p, &g) == PYR_OK && !g.cu ? pyr_attn_bwd_ws_bytes(g) : 0;
}

pyr_status pyr_block_sparse_attn_bwd(const pyr_problem* p, const void* q, const void* k,
                                     const void* v, const int32_t* sel, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk,
                                     void* dv, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  g_err[0] = 0;
  PyrGeom g;
  pyr_status s = resolve(p, &g);
  if (s != PYR_OK) return s;
  if (g.decode) return fail(PYR_ERR_UNSUPPORTED, "the backward is implemented for prefill only");
  if (g.cu) return fail(PYR_ERR_UNSUPPORTED, "the backward takes no packed sequences");
  if (p->dtype != PYR_BF16)
    return fail(PYR_ERR_UNSUPPORTED, "the backward is implemented for bfloat16 only");
  if (g.Tks != g.Tk)
    return fail(PYR_ERR_UNSUPPORTED, "the backward takes k and v without spare capacity");
  if (g.K + 1 > PYR_BWD_MAX_SLOTS)
    return fail(PYR_ERR_UNSUPPORTED, "route rows of %d slots (at most %d)", g.K + 1,
                PYR_BWD_MAX_SLOTS);
  const bool empty = (int64_t)g.B * g.Hk == 0 || g.Tq == 0;
  if (!empty && pyr_attn_bwd_items_bound(g) > INT32_MAX)
    return fail(PYR_ERR_UNSUPPORTED, "problem too large for the backward's work list");
  if (!empty && (!q || !k || !v || !sel || !o || !lse || !dout || !dq || !dk || !dv))
    return fail(PYR_ERR_NULL, "q, k, v, sel, o, lse, dout, dq, dk or dv is NULL");
  if (!empty && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sel) ||
                 !aligned16(o) || !aligned16(lse) || !aligned16(dout) || !aligned16(dq) ||
                 !aligned16(dk) || !aligned16(dv)))
    return fail(PYR_ERR_MISALIGNED, "tensors must be 16-byte aligned");
  const size_t need = pyr_attn_bwd_ws_bytes(g);
  if (!empty && (!workspace || workspace_bytes < need))
    return fail(PYR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!empty && !aligned16(workspace))
    return fail(PYR_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (empty) return PYR_OK;
  return hip_status(pyr_launch_attn_bwd(g, q, k, v, sel, o, lse, dout, dq, dk, dv, workspace, stream),
                    "pyr_block_sparse_attn_bwd launch");
}

pyr_status pyr_budgets_from_entropy(const float* entropy, int32_t n_heads, int32_t total,
                                    int32_t k_min, int32_t k_max, int32_t* k_out) {
  g_err[0] = 0;
  if (n_heads < 0) return fail(PYR_ERR_INVALID, "n_heads %d < 0", n_heads);
  if (n_heads == 0) return PYR_OK;
  if (!entropy || !k_out) return fail(PYR_ERR_NULL, "entropy or k_out is NULL");
  if (k_min < 1 || k_max < k_min)
    return fail(PYR_ERR_INVALID, "need 1 <= k_min <= k_max (k_min %d, k_max %d)", k_min, k_max);
  if (total < 0) return fail(PYR_ERR_INVALID, "total %d < 0", total);
  double sum = 0.0;
  for (int32_t h = 0; h < n_heads; ++h) {
    if (!(entropy[h] >= 0.f) || isinf(entropy[h]))
      return fail(PYR_ERR_INVALID, "entropy[%d] must be finite and >= 0", h);
    sum += entropy[h];
  }
  for (int32_t h = 0; h < n_heads; ++h) {
    const double share = sum > 0.0 ? (double)total * entropy[h] / sum : (double)total / n_heads;
    double k = floor(share + 0.5);
    k = k < k_min ? k_min : (k > k_max ? k_max : k);
    k_out[h] = (int32_t)k;
  }
  return PYR_OK;
}

const char* pyr_status_string(pyr_status s) {
  switch (s) {
    case PYR_OK: return "ok";
    case PYR_ERR_NULL: return "null pointer";
    case PYR_ERR_INVALID: return "invalid argument";
    case PYR_ERR_UNSUPPORTED: return "unsupported";
    case PYR_ERR_MISALIGNED: return "misaligned pointer";
    case PYR_ERR_WORKSPACE: return "workspace too small";
    case PYR_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* pyr_last_error(void) { return g_err; }

int32_t pyr_abi_version(void) { return PYR_ABI_VERSION; }

}  // extern "C"
