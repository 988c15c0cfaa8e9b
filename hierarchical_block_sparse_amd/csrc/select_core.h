// Selection device code shared by the selection kernels and the fused
// select-and-attend kernel: the LDS layout, unit order, ranking, candidate
// sets and the MFMA scoring of one unit.  Everything is in an unnamed
// namespace, so each translation unit that includes it has its own copy.
#pragma once

#include <math.h>

#include "pyr_device.h"
#include "pyr_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 32;   // candidates per LDS chunk (MFMA path): two 16-wide N tiles
constexpr int kZbuf = 8192;  // fp32 scratch for the generic path
constexpr int kSelStages = 2;  // candidate chunks in LDS (MFMA path): one scored while one loads
constexpr int kSelStagesDecode = 4;  // decode: one stage per wave (score_exact_dec)
// Slots after the ancestors in the layout's misc area (4 bytes each).
enum SelMisc {
  kNkept = 0,    // kept count
  kMargin = 1,   // K-th best minus best rejected score (fallback)
  kMiscSlots = 4
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Dynamic LDS layout shared by host (sizing) and device.
struct SelLayout {
  int cmax;  // candidate capacity: b*K + b - 1, rounded up to the chunk size
  int off_kept, off_kscore, off_cand, off_score, off_rank, off_part, off_misc, off_hl, off_zbuf;
  int total;  // bytes
  __host__ __device__ SelLayout(int K, int b, int D, bool mfma, int waves = kWaves) {
    cmax = (b * K + b - 1 + kChunk - 1) / kChunk * kChunk;
    const int kp = (K + 3) & ~3;
    int o = 0;
    off_kept = o;   o += 4 * kp;
    off_kscore = o; o += 4 * kp;
    off_cand = o;   o += 4 * cmax;
    off_score = o;  o += 4 * cmax;  // 16-byte aligned: read as float4
    off_rank = o;   o += 4 * cmax;
    if (mfma) {
      off_part = o;  o += 8 * waves * cmax;                 // float2 [wave][candidate]
      off_misc = o;  o += 4 * (PYR_MAX_LEVELS + kMiscSlots);  // ancestors, then SelMisc slots
      off_hl = off_zbuf = o;
    } else {
      off_part = off_hl = off_misc = o;
      off_zbuf = o;  o += 4 * kZbuf;
    }
    total = o;
  }
};

// Unit of this workgroup.  The dispatcher deals workgroups to the eight XCDs
// in turn (workgroup w runs on XCD w % 8), so XCD x takes the contiguous run
// of units [x * U8, (x + 1) * U8): its L2 then holds the pooled keys of only
// the (batch, KV head) slabs of its run.  Within a run the units go from the
// last (heaviest) query block down.  Returns false for the idle workgroups
// past the end of a short run.
__device__ __forceinline__ bool sel_unit(const PyrGeom& g, int64_t& unit) {
  const int64_t U = (int64_t)g.B * g.Hk * g.nqb;
  const int64_t U8 = (U + 7) / 8;
  const int64_t x = blockIdx.x % 8, k = blockIdx.x / 8;
  const int64_t end = min<int64_t>((x + 1) * U8, U);
  unit = end - 1 - k;
  return unit >= x * U8;
}

// Ancestor of the diagonal block at every level: anc[l] = diag / b^l.
__device__ void ancestors(const PyrGeom& g, int diag, int* s_anc) {
  if (threadIdx.x == 0) {
    int a = diag;
    for (int l = 0; l < g.L; ++l) {
      s_anc[l] = a;
      a /= g.branching;
    }
  }
}

// Order-preserving map of a score to an unsigned key: a larger score gives a
// larger key, -inf gives 0x007fffff, and 0 is left free to mark "no candidate"
// (scores are never NaN).
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One 64-candidate chunk of the in-order compaction of the kept set.
__device__ __forceinline__ void keep_chunk(int j, uint32_t kj, int C, uint32_t T, int need,
                                           unsigned long long lt, const int* cand,
                                           const float* score, int* kept, float* kscore,
                                           int& pos, int& ties, uint32_t& rej) {
  const bool eq = kj == T && j < C;
  const unsigned long long em = __ballot(eq);
  const bool keep = kj > T || (eq && ties + __popcll(em & lt) < need);
  const unsigned long long km = __ballot(keep);
  if (keep) {
    const int p = pos + __popcll(km & lt);
    kept[p] = cand[j];
    kscore[p] = score[j];
  } else if (j < C && kj > rej) {
    rej = kj;
  }
  pos += __popcll(km);
  ties += __popcll(em);
}

// Keep the top K of C >= K candidates in ascending index order and write the
// trace.  Candidates are ascending by node index, so "lower index wins a tie"
// is "lower position wins": the kept set is every candidate with a score above
// the K-th largest, T, plus the first (by position) of those equal to T until
// there are K.  Wave 0 finds T two bits at a time (the largest key with at
// least K keys >= it) with ballots over the candidates, four per lane in
// registers (more are re-read from LDS), then compacts the kept set in index
// order.  *margin gets the K-th best score minus the best rejected one (NaN
// when nothing is rejected).  The trace row is g.K wide: slots past K hold -1
// (ids) and NaN (scores), slot g.K of the scores the best rejected score.
template <int NT>
__device__ void top_k_and_trace(const PyrGeom& g, int C, int level, const int* cand,
                                const float* score, int* rank, int* kept, float* kscore,
                                int* nkept, int K, float* margin, int32_t* tr_ids,
                                float* tr_scores) {
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
  const int nch = (C + 63) / 64;
  if (w == 0) {
    uint32_t kr[4];
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int j = ch * 64 + l;
      kr[ch] = j < C ? score_key(score[j]) : 0u;
    }
    uint32_t* keys = reinterpret_cast<uint32_t*>(rank);
    for (int ch = 4; ch < nch; ++ch) {
      const int j = ch * 64 + l;
      keys[j] = j < C ? score_key(score[j]) : 0u;
    }
    // two bits per step: the largest of T | (d << bit), d = 3, 2, 1, that
    // still has at least K keys at or above it
    uint32_t T = 0;
    for (int bit = 30; bit >= 0; bit -= 2) {
      const uint32_t t1 = T | (1u << bit), t2 = T | (2u << bit), t3 = T | (3u << bit);
      int c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        c1 += __popcll(__ballot(kr[ch] >= t1));
        c2 += __popcll(__ballot(kr[ch] >= t2));
        c3 += __popcll(__ballot(kr[ch] >= t3));
      }
      for (int ch = 4; ch < nch; ++ch) {
        const uint32_t kj = keys[ch * 64 + l];
        c1 += __popcll(__ballot(kj >= t1));
        c2 += __popcll(__ballot(kj >= t2));
        c3 += __popcll(__ballot(kj >= t3));
      }
      T = c3 >= K ? t3 : (c2 >= K ? t2 : (c1 >= K ? t1 : T));
    }
    int above = 0;  // candidates strictly above T (fewer than K)
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) above += __popcll(__ballot(kr[ch] > T));
    for (int ch = 4; ch < nch; ++ch) above += __popcll(__ballot(keys[ch * 64 + l] > T));
    const int need = K - above;  // ties at T to keep, lowest positions first
    const unsigned long long lt = (1ull << l) - 1ull;
    int pos = 0, ties = 0;
    uint32_t rej = 0;  // best rejected key of this lane
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
      if (ch < nch)
        keep_chunk(ch * 64 + l, kr[ch], C, T, need, lt, cand, score, kept, kscore, pos, ties, rej);
    for (int ch = 4; ch < nch; ++ch)
      keep_chunk(ch * 64 + l, keys[ch * 64 + l], C, T, need, lt, cand, score, kept, kscore, pos,
                 ties, rej);
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t r2 = (uint32_t)__shfl_xor((int)rej, o, 64);
      rej = r2 > rej ? r2 : rej;
    }
    if (l == 0) {
      if (tr_scores) tr_scores[level * (g.K + 1) + g.K] = key_score(rej);  // best rejected
      *margin = key_score(T) - key_score(rej);
      *nkept = K;
    }
  }
  lds_barrier();
  if (tr_ids) {
    for (int j = tid; j < g.K; j += NT) tr_ids[level * g.K + j] = j < K ? kept[j] : -1;
  }
  if (tr_scores) {
    for (int j = tid; j < g.K; j += NT)
      tr_scores[level * (g.K + 1) + j] = j < K ? kscore[j] : NAN;
  }
}

// Nodes kept per level for the units of KV head hk: the head's budget when
// budgets are given (clamped to [1, K]), else K.
__device__ __forceinline__ int unit_budget(const PyrGeom& g, int hk) {
  if (!g.k_head) return g.K;
  const int k = g.k_head[hk];
  return k < 1 ? 1 : (k > g.K ? g.K : k);
}

// Confidence fallback, decided after the finest level's top-Ku: when the
// margin between the Ku-th best score and the best rejected one is below
// g.fb_margin, the level is ranked again keeping the best g.fb_k candidates
// (all of them if there are fewer).  Must be called by every thread; the
// result is uniform.
__device__ __forceinline__ bool fallback_due(const PyrGeom& g, int level, int kk, int Ku,
                                             const float* margin) {
  if (level != 0 || kk != Ku || g.fb_k <= Ku) return false;
  lds_barrier();  // the trace of the first pass has read kept[]; *margin is visible
  return *margin < g.fb_margin;
}

// Candidates of one level into cand[]; returns the count.  Must be called by
// every thread (ends with a barrier).
template <int NT>
__device__ int build_candidates(const PyrGeom& g, int level, const int* s_anc, const int* kept,
                                int nkept, int* cand) {
  const int b = g.branching;
  const int anc = s_anc[level];
  int C, base, nchild;
  if (level == g.L - 1) {
    C = anc;
    nchild = 0;
    base = 0;
  } else {
    nchild = nkept * b;
    base = s_anc[level + 1] * b;
    C = nchild + (anc - base);
  }
  for (int j = threadIdx.x; j < C; j += NT)
    cand[j] = j < nchild ? kept[j / b] * b + j % b : base + (j - nchild);
  lds_barrier();
  return C;
}

// Levels with <= K candidates keep them all (no scoring).
template <int NT>
__device__ void keep_all(const PyrGeom& g, int C, int level, const int* cand, int* kept,
                         int* nkept, int32_t* tr_ids, float* tr_scores) {
  const int K = g.K;
  for (int j = threadIdx.x; j < K; j += NT) {
    const int id = j < C ? cand[j] : -1;
    kept[j] = id;
    if (tr_ids) tr_ids[level * K + j] = id;
  }
  if (tr_scores)
    for (int j = threadIdx.x; j <= K; j += NT) tr_scores[level * (K + 1) + j] = NAN;
  if (threadIdx.x == 0) *nkept = C;
  lds_barrier();
}

template <int NT>
__device__ __forceinline__ void write_route(const PyrGeom& g, int64_t unit, const int* kept,
                                            int nk, int diag, int32_t* sel) {
  int32_t* out = sel + unit * (g.K + 1);
  for (int j = threadIdx.x; j <= g.K; j += NT) out[j] = j < nk ? kept[j] : (j == nk ? diag : -1);
}

// A unit past the end of a shorter packed sequence: its route row (and trace)
// hold nothing.
template <int NT>
__device__ void blank_unit(const PyrGeom& g, int64_t unit, int32_t* sel, int32_t* trace_ids,
                           float* trace_scores) {
  for (int j = threadIdx.x; j <= g.K; j += NT) sel[unit * (g.K + 1) + j] = -1;
  if (trace_ids)
    for (int j = threadIdx.x; j < g.L * g.K; j += NT) trace_ids[unit * g.L * g.K + j] = -1;
  if (trace_scores)
    for (int j = threadIdx.x; j < g.L * (g.K + 1); j += NT)
      trace_scores[unit * g.L * (g.K + 1) + j] = NAN;
}

// ---------------------------------------------------------------------------
// bf16 prefill path: MFMA scoring.  MT = 16-row M tiles per wave.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;

// Split rows of list entries [32c, 32c + 32) (plane 1 of the pyramid: per
// node a bf16 hi row and a bf16 lo row, 4D bytes) into one LDS stage with
// direct 16-byte loads, no register staging.  Entry jj is candidate
// cand[pos[jj]] (cand[jj] when pos is null).  Load t of a thread fills stage
// chunk p = t * NT + tid (the 64 lanes of a wave fill 1 KiB in lane order):
// entry p / CPC, row part (p % CPC) / CPR (hi, lo), stored chunk q = p % CPR,
// which holds logical chunk q ^ (entry % CPR) of that row, so the 16 entries
// of an MFMA B fragment lie in different banks.  Positions past n load entry
// 0 (finite values that are never scored).
template <int D, int NT>
__device__ __forceinline__ void issue_chunk(const unsigned char* split, const int* cand,
                                            const int* pos, int n, int c, unsigned char* stage,
                                            int w, int l) {
  constexpr int CPR = D / 8;       // 16-byte chunks per bf16 row
  constexpr int CPC = 2 * CPR;     // per candidate (hi, lo)
  constexpr int PER = kChunk * CPC / NT;
  static_assert(kChunk * CPC % NT == 0, "chunk must split evenly");
  // opaque to the optimiser, so the per-load offsets below are recomputed
  // here rather than hoisted out of the level loop into spilled registers
  uint32_t tl = (uint32_t)(w * 64 + l);
  asm volatile("" : "+v"(tl));
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const uint32_t p = t * NT + tl;
    const uint32_t cc = p / CPC, part = (p % CPC) / CPR, q = p % CPR;
    const int j = c * kChunk + (int)cc;
    const int jj = j < n ? j : 0;
    const int node = cand[pos ? pos[jj] : jj];
    const unsigned char* src =
        split + (size_t)(uint32_t)node * (4 * D) + (part * 2 * D + ((q ^ (cc % CPR)) << 4));
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (lds_void*)(stage + (t * NT + w * 64) * 16), 16, 0, 0);
  }
}

// LogSumExp (log2 domain: max m and sum s of 2^(x - m)) of one wave's rows for
// the 16 candidates of an N tile; lane l ends with the value of candidate
// l % 16.  Row j of M tile mt in the C layout is row 4*(l/16) + j, so a
// candidate's rows are spread over the four 16-lane rows: the maximum is
// taken across them first, which makes the partial sums share one reference
// and combine by plain addition.  FULL skips the per-row validity bits.
template <int MT, bool FULL>
__device__ __forceinline__ void tile_lse(const f32x4 (&acc)[MT], uint32_t rowvalid, float sl2,
                                         float& m, float& s) {
  float mr = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (FULL || (rowvalid >> (mt * 4 + j) & 1u)) mr = fmaxf(mr, acc[mt][j]);
  mr = max32(max16(mr));
  m = mr * sl2;
  s = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (FULL || (rowvalid >> (mt * 4 + j) & 1u))
          s += __builtin_amdgcn_exp2f(fmaf(acc[mt][j], sl2, -m));
  }
  s = sum32(sum16(s));
}

// Exact scores' LogSumExp partials of list entries [0, n) (entry jj is
// candidate cand[pos[jj]], cand[jj] when pos is null): both planes of the
// split contracted against the exact bf16 q on the matrix cores, chunks of 32
// entries through stages st0 / st1.  Per wave and entry the (max, sum) pair
// of the wave's rows goes to part[w * cmax + entry].  Every thread calls it;
// the caller's barrier makes the partials visible.  A candidate's partials do
// not depend on its position in the list or on the other entries.
template <int D, int MT, int NW>
__device__ __forceinline__ void score_exact(const unsigned char* lvl, const int* cand,
                                            const int* pos, int n, const uint4 (&qa)[MT][D / 32],
                                            uint32_t rowvalid, bool full, float sl2,
                                            lds_f32x2* part, int cmax, unsigned char* st0,
                                            unsigned char* st1, int w, int l) {
  constexpr int CPR = D / 8;
  const int nchunks = (n + kChunk - 1) / kChunk;
  // chunk c+1 loads while chunk c is scored; stage of chunk c is c % 2
  issue_chunk<D, NW * 64>(lvl, cand, pos, n, 0, st0, w, l);
  for (int c = 0; c < nchunks; ++c) {
    // this wave's loads of chunk c have landed; after the barrier every
    // wave's have, and the stage of chunk c-1 is free
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    lds_barrier();
    if (c + 1 < nchunks)
      issue_chunk<D, NW * 64>(lvl, cand, pos, n, c + 1, (c + 1) & 1 ? st1 : st0, w, l);
    const unsigned char* st = c & 1 ? st1 : st0;
#pragma unroll
    for (int nt = 0; nt < kChunk / 16; ++nt) {
      if (c * kChunk + nt * 16 >= n) break;  // uniform
      f32x4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // B fragment: entry r = nt*16 + l%16, logical chunk 4*ks + l/16 of its
      // hi and lo rows, stored at that chunk ^ (r % CPR)
      const int r = nt * 16 + (l % 16);
      const unsigned char* row = st + r * 4 * D;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const int off = ((4 * ks + l / 16) ^ (r % CPR)) << 4;
        const bf16x8 bhv = as_bf16x8(*reinterpret_cast<const uint4*>(row + off));
        const bf16x8 blv = as_bf16x8(*reinterpret_cast<const uint4*>(row + 2 * D + off));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[mt][ks]), bhv, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[mt][ks]), blv, acc[mt], 0, 0, 0);
        }
      }
      // this wave's LogSumExp over its rows, per entry (lane column l % 16)
      float m, s;
      if (full)
        tile_lse<MT, true>(acc, rowvalid, sl2, m, s);
      else
        tile_lse<MT, false>(acc, rowvalid, sl2, m, s);
      const int cn = c * kChunk + nt * 16 + l;
      if (l < 16 && cn < n) part[w * cmax + cn] = f32x2{m, s};
    }
  }
}

// Decode's exact scores: every wave holds the unit's G query rows (one
// 16-row tile) and scores its own chunks c = w, w + NW, ... of the list from
// a stage of its own (st + w * kChunk * 4 * D), loading a chunk and then
// scoring it with no workgroup barrier in between.  A chunk's few real rows
// take far less than its load's latency, so score_exact's barrier-paced
// pipeline (every wave on every chunk) spent a load latency per chunk.  A
// wave's (max, sum) pair of an entry is then its whole LogSumExp: it goes to
// the wave-0 slot and the other slots get the empty pair, so merged_score
// gives what score_exact gives.  Every thread calls it; the caller's barrier
// makes the partials visible.
template <int D, int NW>
__device__ __forceinline__ void score_exact_dec(const unsigned char* lvl, const int* cand, int n,
                                                const uint4 (&qa)[1][D / 32], uint32_t rowvalid,
                                                float sl2, lds_f32x2* part, int cmax,
                                                unsigned char* st, int w, int l) {
  constexpr int CPR = D / 8;
  unsigned char* mine = st + w * (kChunk * 4 * D);
  const int nchunks = (n + kChunk - 1) / kChunk;
  for (int c = w; c < nchunks; c += NW) {
    issue_chunk<D, 64>(lvl, cand, nullptr, n, c, mine, 0, l);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of chunk c
#pragma unroll
    for (int nt = 0; nt < kChunk / 16; ++nt) {
      if (c * kChunk + nt * 16 >= n) break;  // uniform
      f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
      const int r = nt * 16 + (l % 16);
      const unsigned char* row = mine + r * 4 * D;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const int off = ((4 * ks + l / 16) ^ (r % CPR)) << 4;
        const bf16x8 bhv = as_bf16x8(*reinterpret_cast<const uint4*>(row + off));
        const bf16x8 blv = as_bf16x8(*reinterpret_cast<const uint4*>(row + 2 * D + off));
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[0][ks]), bhv, acc[0], 0, 0, 0);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[0][ks]), blv, acc[0], 0, 0, 0);
      }
      float m, s;
      tile_lse<1, false>(acc, rowvalid, sl2, m, s);
      const int cn = c * kChunk + nt * 16 + l;
      if (l < 16 && cn < n) {
        part[cn] = f32x2{m, s};
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) part[ww * cmax + cn] = f32x2{-INFINITY, 0.f};
      }
    }
  }
}

// Merged score of entry j from the waves' partials (natural log; NaN ranks
// last as -inf).  The exact path and the re-scoring of undecided candidates
// both use it, so a candidate gets the same bits from either.
template <int NW>
__device__ __forceinline__ float merged_score(const lds_f32x2* part, int cmax, int j) {
  float m = -INFINITY, s = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const f32x2 p = part[ww * cmax + j];
    lse2_merge(m, s, p.x, p.y);
  }
  const float sc = (m + log2f(s)) * PYR_LN2;
  return sc == sc ? sc : -INFINITY;
}

// Number of keys among key[0, n) above kj (keys are distinct and nonzero;
// n is a multiple of 16, padded with zero keys).  Sixteen keys are read per
// batch so that one LDS latency covers them.
__device__ __forceinline__ int count_above(const uint64_t* key, int n, uint64_t kj) {
  int cnt = 0;
  for (int i = 0; i < n; i += 16) {
    ulonglong2 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = *reinterpret_cast<const ulonglong2*>(key + i + 2 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) cnt += (a[u].x > kj) + (a[u].y > kj);
  }
  return cnt;
}

// Number of the 16 keys at key[0..16) above kj.
__device__ __forceinline__ int count16(const uint64_t* key, uint64_t kj) {
  ulonglong2 a[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) a[u] = *reinterpret_cast<const ulonglong2*>(key + 2 * u);
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) cnt += (a[u].x > kj) + (a[u].y > kj);
  return cnt;
}

// Rank key of a score at candidate position j: larger score first, then the
// lower position (the lower node index: candidates ascend by index).
__device__ __forceinline__ uint64_t rank_key(float sc, int j) {
  return ((uint64_t)score_key(sc) << 32) | (uint32_t)~(uint32_t)j;
}

// Ranking of one scored level without a score trace or fallback, after
// score_exact and its barrier: every candidate's merged score gets a 64-bit
// key (score, then the lower position), the keys above each candidate's are
// counted (its rank; the counting is spread over all threads), and wave 0
// compacts the candidates ranked below Ku in index order into kept[].
// The kept set is the one top_k_and_trace keeps from the same scores.
template <int NW, bool BAL = false>
__device__ __forceinline__ void rank_level(const PyrGeom& g, int level, int C, int Ku,
                                           const SelLayout& lay, unsigned char* smem,
                                           int32_t* tr_ids, int w, int l) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, cmax = lay.cmax;
  int* kept = reinterpret_cast<int*>(smem + lay.off_kept);
  const int* cand = reinterpret_cast<const int*>(smem + lay.off_cand);
  int* flag = reinterpret_cast<int*>(smem + lay.off_rank);
  const lds_f32x2* part = (const lds_f32x2*)(smem + lay.off_part);
  // a key overwrites the wave-0 partial of its own candidate, read just before
  uint64_t* key = reinterpret_cast<uint64_t*>(smem + lay.off_part);
  int* misc = reinterpret_cast<int*>(smem + lay.off_misc) + PYR_MAX_LEVELS;
  const int C16 = (C + 15) & ~15;  // <= cmax, a multiple of 32
  for (int j = tid; j < C16; j += NT) key[j] = j < C ? rank_key(merged_score<NW>(part, cmax, j), j) : 0ull;
  if (BAL && C > NT)  // the counts of candidates NT .. C-1 are accumulated below
    for (int j = NT + tid; j < C; j += NT) flag[j] = 0;
  lds_barrier();
  if (NW == 4 && !BAL && 2 * C16 <= NT) {
    // at most half a candidate per thread (four waves; with eight the
    // kernel's extra registers for this path cost more than it saves): the
    // first half of the threads
    // counts the keys above each candidate's in the first half of the list,
    // the second half in the rest (the lanes of a wave read the same keys:
    // LDS broadcast), and the two counts meet in LDS
    const int hh = 2 * tid >= NT, j = tid - hh * (NT / 2);
    const int nh = ((C16 / 2) + 15) & ~15;  // keys of the first half, a multiple of 16
    int cnt = 0;
    if (j < C) cnt = count_above(key + hh * nh, hh ? C16 - nh : nh, key[j]);
    if (hh && j < C) flag[j] = cnt;
    lds_barrier();
    if (!hh && j < C) flag[j] += cnt;
  } else if (!BAL || C <= NT) {
    // a candidate per thread: its rank (the keys above its key); the lanes of
    // a wave read the same keys (LDS broadcast)
    for (int j = tid; j < C; j += NT) flag[j] = count_above(key, C16, key[j]);
  } else {
    // BAL, more candidates than threads (decode: C = b*K + b - 1 just over
    // the threads): candidate tid as above, and the 16-key batches of the
    // candidates past NT spread one per thread and added into their ranks,
    // instead of a few threads counting a second candidate in full
    flag[tid] = count_above(key, C16, key[tid]);
    const int nbt = C16 / 16;
    for (int t = tid; t < (C - NT) * nbt; t += NT) {
      const int j = NT + t / nbt, bt = t % nbt;
      atomicAdd(&flag[j], count16(key + 16 * bt, key[j]));
    }
  }
  lds_barrier();
  if (w == 0) {
    const uint64_t lt = (1ull << l) - 1ull;
    int nk = 0;
    for (int j0 = 0; j0 < C; j0 += 256) {
      // four chunks' flags and ids read together
      bool f[4];
      int id[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + 64 * u + l;
        f[u] = j < C && flag[j] < Ku;
        id[u] = j < C ? cand[j] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t mk = __ballot(f[u]);
        if (f[u]) kept[nk + __popcll(mk & lt)] = id[u];
        nk += __popcll(mk);
      }
    }
    if (l == 0) misc[kNkept] = Ku;
  }
  lds_barrier();
  if (tr_ids)
    for (int j = tid; j < g.K; j += NT) tr_ids[level * g.K + j] = j < Ku ? kept[j] : -1;
}

// Selection of one unit on the matrix cores by NW waves of MT M tiles each.
// smem: the dynamic layout SelLayout(K, b, D, true, NW); st0 and st1: the two
// candidate stages (kChunk * 4 * D bytes each), LDS of their own so that
// writes to the layout do not wait for the stage loads in flight.  Must be
// called by every thread of the workgroup.  Leaves the finest kept set in
// the layout's kept[] and its size in the kept count, and writes the route
// row (and trace) of the unit.  Without a score trace and without a
// fallback, scored levels are ranked by rank_level; otherwise by
// top_k_and_trace, which also records scores and the margin.
template <int D, int MT, int NW, bool DEC = false>
__device__ __forceinline__ void select_mfma_unit(const bf16_t* __restrict__ q,
                                                 const float* __restrict__ pyr,
                                                 int32_t* __restrict__ sel,
                                                 int32_t* __restrict__ trace_ids,
                                                 float* __restrict__ trace_scores,
                                                 const PyrGeom& g, int64_t unit,
                                                 unsigned char* smem, unsigned char* st0,
                                                 unsigned char* st1) {
  constexpr int NT = NW * 64;
  const SelLayout lay(g.K, g.branching, D, true, NW);
  int* kept = reinterpret_cast<int*>(smem + lay.off_kept);
  float* kscore = reinterpret_cast<float*>(smem + lay.off_kscore);
  int* cand = reinterpret_cast<int*>(smem + lay.off_cand);
  float* score = reinterpret_cast<float*>(smem + lay.off_score);
  int* rank = reinterpret_cast<int*>(smem + lay.off_rank);
  lds_f32x2* part = (lds_f32x2*)(smem + lay.off_part);
  int* s_anc = reinterpret_cast<int*>(smem + lay.off_misc);
  int* misc = s_anc + PYR_MAX_LEVELS;
  float* miscf = reinterpret_cast<float*>(misc);
  int& s_nkept = misc[kNkept];
  float* s_margin = miscf + kMargin;

  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int i = (int)(unit % g.nqb);
  const int64_t bhk = unit / g.nqb;  // b * Hk + hk
  const int bi = (int)(bhk / g.Hk), hk = (int)(bhk % g.Hk);
  const PyrSeq sq = pyr_seq(g, bi);
  if (i >= sq.nqb) {
    blank_unit<NT>(g, unit, sel, trace_ids, trace_scores);
    return;
  }
  // decode: one query block whose token sits at kv_len - 1; its G rows (one
  // per query head) fill the first M tile of wave 0, every other row is idle
  const int diag = g.decode ? (int)((g.Tk - 1) / PYR_BLOCK) : i;
  const int Ku = unit_budget(g, hk);
  const int RW = MT * 16;  // rows per wave
  const float sl2 = g.scale * PYR_LOG2E;
  // no score trace and no fallback: the kept sets come from rank_level
  const bool ranked = !trace_scores && g.fb_k <= Ku;

  ancestors(g, diag, s_anc);

  // Q fragments (A operand): lane holds row (l % 16) of each M tile and the
  // 8 consecutive d at 32*ks + 8*(l/16).
  uint4 qa[MT][D / 32];
  uint32_t rowvalid = 0;  // bit (mt*4 + j): C-layout row 4*(l/16)+j of tile mt is a real row
  // (DEC: every wave holds the same rows, the G real ones in its first tile)
  const int rbase = DEC ? 0 : w * RW;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ra = rbase + mt * 16 + (l % 16);
    int h;
    int64_t tok;
    if (g.decode) {
      h = ra < g.G ? ra : g.G - 1;
      tok = 0;
    } else {
      h = ra / PYR_BLOCK;
      tok = min<int64_t>((int64_t)i * PYR_BLOCK + ra % PYR_BLOCK, sq.Tq - 1);
    }
    const bf16_t* qrow = q + (sq.q0 + ((int64_t)hk * g.G + h) * sq.qhs + tok) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qa[mt][ks] = ld16(qrow + ks * 32 + 8 * (l / 16));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rc = rbase + mt * 16 + 4 * (l / 16) + j;
      const bool real = g.decode ? rc < g.G : (int64_t)i * PYR_BLOCK + rc % PYR_BLOCK < sq.Tq;
      if (real) rowvalid |= 1u << (mt * 4 + j);
    }
  }
  // every row of the unit is real
  const bool full = !g.decode && (int64_t)(i + 1) * PYR_BLOCK <= sq.Tq;
  // plane 1 of the slab: the split rows
  const unsigned char* split =
      reinterpret_cast<const unsigned char*>(pyr + (bhk * g.planes + 1) * g.n_tot * D);
  int32_t* tr_ids = trace_ids ? trace_ids + unit * g.L * g.K : nullptr;
  float* tr_sc = trace_scores ? trace_scores + unit * g.L * (g.K + 1) : nullptr;
  lds_barrier();
  // Coarse levels with at most Ku candidates keep them all.  While every
  // level above keeps all, the candidates of level l are the nodes before
  // the diagonal's ancestor, [0, anc[l]); so the first scored level is the
  // coarsest with anc[l] > Ku, and the kept set above it is [0, anc[top+1]).
  int top = g.L - 1;
  while (top >= 0 && s_anc[top] <= Ku) --top;
  for (int lv = g.L - 1; lv > top; --lv) {
    if (tr_ids)
      for (int j = tid; j < g.K; j += NT) tr_ids[lv * g.K + j] = j < s_anc[lv] ? j : -1;
    if (tr_sc)
      for (int j = tid; j <= g.K; j += NT) tr_sc[lv * (g.K + 1) + j] = NAN;
  }
  const int nabove = top + 1 < g.L ? s_anc[top + 1] : 0;
  for (int j = tid; j < nabove; j += NT) kept[j] = j;
  if (tid == 0) s_nkept = nabove;
  lds_barrier();

  for (int level = top; level >= 0; --level) {
    const int C = build_candidates<NT>(g, level, s_anc, kept, s_nkept, cand);
    if (C <= Ku) {
      keep_all<NT>(g, C, level, cand, kept, &s_nkept, tr_ids, tr_sc);
      continue;
    }
    const unsigned char* lvl = split + g.loff[level] * 4 * D;
    if constexpr (DEC)
      score_exact_dec<D, NW>(lvl, cand, C, qa, rowvalid, sl2, part, lay.cmax, st0, w, l);
    else
      score_exact<D, MT, NW>(lvl, cand, nullptr, C, qa, rowvalid, full, sl2, part, lay.cmax, st0,
                             st1, w, l);
    lds_barrier();
    if (ranked) {
      rank_level<NW, DEC>(g, level, C, Ku, lay, smem, tr_ids, w, l);
      continue;
    }
    for (int j = tid; j < C; j += NT) score[j] = merged_score<NW>(part, lay.cmax, j);
    lds_barrier();
    for (int kk = Ku;;) {
      top_k_and_trace<NT>(g, C, level, cand, score, rank, kept, kscore, &s_nkept, kk, s_margin,
                          tr_ids, tr_sc);
      if (!fallback_due(g, level, kk, Ku, s_margin)) break;
      kk = C < g.fb_k ? C : g.fb_k;  // keep more of the same candidates
    }
  }
  write_route<NT>(g, unit, kept, s_nkept, diag, sel);
}

// NW waves of MT M tiles each, at most 128 VGPRs (four waves per SIMD):
// four four-wave workgroups (G = 4) or two eight-wave ones (G = 8) share a
// CU, so other units' scoring fills a unit's ranking and load latency.
template <int D, int MT, int NW, bool DEC = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void select_mfma(
    const bf16_t* __restrict__ q, const float* __restrict__ pyr, int32_t* __restrict__ sel,
    int32_t* __restrict__ trace_ids, float* __restrict__ trace_scores, PyrGeom g) {
  constexpr int STAGE = kChunk * 4 * D;  // bytes per LDS stage
  static_assert(kSelStages == 2, "two candidate stages");
  static_assert(!DEC || (MT == 1 && NW <= kSelStagesDecode), "decode: one tile, a stage per wave");
  // The layout is the one dynamic array: with a second __shared__ variable
  // the compiler would give each its own alias scope and wait for every chunk
  // load in flight before any LDS read, undoing the prefetch.
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ __attribute__((aligned(16))) unsigned char stages[(DEC ? kSelStagesDecode : kSelStages) * STAGE];
  int64_t unit;
  if (!sel_unit(g, unit)) return;
  select_mfma_unit<D, MT, NW, DEC>(q, pyr, sel, trace_ids, trace_scores, g, unit, smem, stages,
                                   stages + STAGE);
}

}  // namespace
