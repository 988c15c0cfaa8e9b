// Internal declarations shared by the host API and the kernel translation units
// of libpyr (gfx950).  Not part of the public ABI (include/pyr.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define PYR_MAX_LEVELS 48
#define PYR_BLOCK 64

// Problem geometry resolved once on the host and passed by value to kernels.
struct PyrGeom {
  int64_t Tq, Tk;          // query / key lengths
  int64_t Tks;             // rows per head in k and v: the capacity (or Tk); packed: all rows
  int64_t Tqs;             // rows per head in q, o and lse: Tq; packed: all rows
  const int32_t* cu;       // packed sequences: device row offsets [B + 1]; dense: null
  const int32_t* k_head;   // selection budgets per KV head (device, [Hk]); null: K everywhere
  float fb_margin;         // finest-level confidence margin below which fb_k blocks are kept
  int32_t fb_k;            // fallback budget (0: no fallback)
  int64_t n_tot;           // pyramid nodes per (batch, KV head) slab
  int32_t planes;          // pyramid planes: 1 (fp32 problems) or 2 (bf16: + hi/lo split)
  int32_t B, Hq, Hk, G, D; // batch, heads, group size Hq/Hk, head dim
  int32_t nb;              // finest-level blocks: ceil(Tk / 64)
  int32_t nqb;             // query blocks per (batch, KV head)
  int32_t L;               // pyramid levels (finest .. root)
  int32_t branching, K;    // children per node, nodes kept per level
  int32_t decode;          // 1: one query token at position Tk-1
  float scale;             // scoring / softmax scale
  int32_t lsize[PYR_MAX_LEVELS];  // valid nodes per level (from Tk), finest first
  int64_t loff[PYR_MAX_LEVELS];   // node offset of each level inside a slab (from the capacity)
};

// Token count covered by node m of level `level` (blocks [m b^l, (m+1) b^l))
// of a sequence of Tk keys.
__host__ __device__ inline int64_t pyr_node_tokens(int64_t Tk, int branching, int level,
                                                   int64_t m) {
  int64_t span = PYR_BLOCK;
  for (int i = 0; i < level; ++i) span *= branching;
  int64_t t0 = m * span, t1 = t0 + span;
  if (t1 > Tk) t1 = Tk;
  return t1 > t0 ? t1 - t0 : 0;
}

// One sequence of a problem.  Row t of query head h is row q0 + h * qhs + t of
// q (and of o and lse); row t of KV head hk is row k0 + hk * khs + t of k and
// v.  Dense batches use the strides of [B, H, T, d].  In a packed batch every
// head holds all sequences back to back, sequence bi owning rows
// [cu[bi], cu[bi+1]); the offsets are clipped to the packed row count and the
// length to the problem's bound, so malformed offsets cannot reach outside the
// tensors.
struct PyrSeq {
  int64_t Tq, Tk;    // query and key lengths of the sequence
  int64_t q0, k0;    // row of token 0 of head 0
  int64_t qhs, khs;  // rows between heads
  int32_t nb, nqb;   // key blocks, query blocks
};

__device__ __forceinline__ PyrSeq pyr_seq(const PyrGeom& g, int bi) {
  PyrSeq s;
  if (g.cu) {
    const int64_t tot = g.Tks;
    int64_t a = g.cu[bi], e = g.cu[bi + 1];
    a = a < 0 ? 0 : (a > tot ? tot : a);
    e = e < a ? a : (e > tot ? tot : e);
    const int64_t n = e - a < g.Tk ? e - a : g.Tk;
    s.Tq = s.Tk = n;
    s.q0 = s.k0 = a;
    s.qhs = s.khs = tot;
    s.nb = s.nqb = (int32_t)((n + PYR_BLOCK - 1) / PYR_BLOCK);
  } else {
    s.Tq = g.Tq;
    s.Tk = g.Tk;
    s.qhs = g.Tqs;
    s.khs = g.Tks;
    s.q0 = (int64_t)bi * g.Hq * g.Tqs;
    s.k0 = (int64_t)bi * g.Hk * g.Tks;
    s.nb = g.nb;
    s.nqb = g.nqb;
  }
  return s;
}

// Launchers (each returns the hipError_t of its launches).
hipError_t pyr_launch_build(const PyrGeom& g, int dtype, const void* k, float* pyr,
                            hipStream_t st);
hipError_t pyr_launch_append(const PyrGeom& g, int dtype, const void* k, int64_t old_len,
                             float* pyr, hipStream_t st);
hipError_t pyr_launch_select(const PyrGeom& g, int dtype, const void* q, const float* pyr,
                             int32_t* sel, int32_t* trace_ids, float* trace_scores,
                             hipStream_t st);
// Workspace bytes the attention needs (decode's partial states; 0 otherwise).
size_t pyr_attn_ws_bytes(const PyrGeom& g);
// Workspace bytes the attention can use for a block-transposed copy of V
// (bf16 prefill of a dense batch, query heads per KV head G a multiple of 4,
// (top_k + 1) * G/4 >= 16; 0 otherwise).  Used when the caller's workspace
// holds that many bytes.
size_t pyr_attn_vt_bytes(const PyrGeom& g, int dtype);
// ws_bytes: the workspace's size (0: read V directly).
hipError_t pyr_launch_attn(const PyrGeom& g, int dtype, const void* q, const void* k,
                           const void* v, const int32_t* sel, void* o, float* lse, void* ws,
                           size_t ws_bytes, hipStream_t st);
// The attention with its workspace (if any) in the library's fixed per-device
// scratch array; the caller has checked pyr_attn_ws_bytes(g) against its size.
hipError_t pyr_launch_attn_noalloc(const PyrGeom& g, int dtype, const void* q, const void* k,
                                   const void* v, const int32_t* sel, void* o, float* lse,
                                   hipStream_t st);
// Selection then attention: one fused launch where pyr_select_attend_fused
// holds (bf16 prefill, four query heads per KV head, the selection's layout
// fits one tile slot), else the two launchers above in turn.
bool pyr_select_attend_fused(const PyrGeom& g, int dtype);
hipError_t pyr_launch_select_attend(const PyrGeom& g, int dtype, const void* q, const void* k,
                                    const void* v, const float* pyr, int32_t* sel,
                                    int32_t* trace_ids, float* trace_scores, void* o, float* lse,
                                    void* ws, size_t ws_bytes, hipStream_t st);
// Backward of the attention (bfloat16 prefill): workspace bytes and launcher.
size_t pyr_attn_bwd_ws_bytes(const PyrGeom& g);
// Upper bound on the work items of the key-gradient kernel (its grid size).
int64_t pyr_attn_bwd_items_bound(const PyrGeom& g);
hipError_t pyr_launch_attn_bwd(const PyrGeom& g, const void* q, const void* k, const void* v,
                               const int32_t* sel, const void* o, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, void* ws,
                               hipStream_t st);
// Route-row capacity of the backward's dQ kernel (slots K+1 it stages on chip).
#define PYR_BWD_MAX_SLOTS 1024
// Selection kernels need this much dynamic LDS (bytes); validated on the host.
size_t pyr_select_lds_bytes(const PyrGeom& g, int dtype);
