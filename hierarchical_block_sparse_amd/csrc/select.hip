// Coarse-to-fine top-K block selection on gfx950.
//
// PISA (peercurrent.com record), abstract: start at the coarsest pooled level,
// score a bounded candidate set with LogSumExp, keep the top K, continue with
// their children at the next finer level until the finest; the query-key score
// matrix is never materialised.  PHBA (Prefix-State Hybrid Block Attention)
// §A.1.2: only strictly preceding blocks are routed, unused slots hold -1.
//
// One workgroup per unit (batch, KV head, query block).  Per level:
//   1. candidates = children of the nodes kept one level up, then the children
//      of the diagonal block's ancestor that lie wholly before the diagonal's
//      ancestor at this level (ascending by construction);
//   2. with more than K candidates, every candidate n is scored
//      s(n) = log sum_r exp(scale * q_r . P_l[n]) over the unit's rows
//      (G heads x the block's tokens) -- the scores live only in LDS;
//   3. the K best (score desc, index asc) are kept, in ascending index order.
// The route row is the finest kept set, the diagonal block, then -1.
//
// Scoring, bf16 prefill path: rows are the M side of v_mfma_f32_16x16x32_bf16
// and candidates the N side; each wave keeps its rows of Q in VGPRs for the
// whole unit.  Pooled keys are fp32; each is split into hi = bf16(x) and
// lo = bf16(x - hi) and both are contracted against the exact bf16 q, so a dot
// product carries ~2^-17 relative error instead of bf16's 2^-9.  Candidates go
// through LDS in chunks of 32: the pooled keys of the next chunk are loaded
// into registers while the current chunk's MFMAs run, then converted to hi/lo
// into the other LDS buffer (one barrier per chunk).  Each wave reduces its
// rows' LogSumExp per candidate in-lane and across its 4 lane groups with
// shuffles, as (max, sum) pairs in the log2 domain; the waves' partials are
// merged once per level.  Generic path (fp32 inputs, decode, other group
// sizes): fp32 dot products on the vector ALUs, same selection logic.
#include <math.h>

#include "pyr_device.h"
#include "pyr_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 32;   // candidates per LDS chunk (MFMA path): two 16-wide N tiles
constexpr int kZbuf = 8192;  // fp32 scratch for the generic path

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Dynamic LDS layout shared by host (sizing) and device.
struct SelLayout {
  int cmax;  // candidate capacity: b*K + b - 1, rounded up to the chunk size
  int off_kept, off_kscore, off_cand, off_score, off_rank, off_part, off_hl, off_zbuf;
  int total;  // bytes
  __host__ __device__ SelLayout(int K, int b, int D, bool mfma) {
    cmax = (b * K + b - 1 + kChunk - 1) / kChunk * kChunk;
    const int kp = (K + 3) & ~3;
    int o = 0;
    off_kept = o;   o += 4 * kp;
    off_kscore = o; o += 4 * kp;
    off_cand = o;   o += 4 * cmax;
    off_score = o;  o += 4 * cmax;  // 16-byte aligned: read as float4
    off_rank = o;   o += 4 * cmax;
    if (mfma) {
      off_part = o;  o += 8 * kWaves * cmax;             // float2 [wave][candidate]
      off_hl = o;    o += 2 * 2 * kChunk * (D + 8) * 2;  // bf16 [stage][hi, lo][cand][D + 8]
      off_zbuf = o;
    } else {
      off_part = off_hl = o;
      off_zbuf = o;  o += 4 * kZbuf;
    }
    total = o;
  }
};

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

// Keep the top K of C > K candidates in ascending index order and write the
// trace.  Candidates are ascending by node index, so "lower index wins a tie"
// is "lower position wins": the kept set is every candidate with a score above
// the K-th largest, T, plus the first (by position) of those equal to T until
// there are K.  Wave 0 finds T bit by bit (the largest key with at least K
// keys >= it) with ballots over the candidates, four per lane in registers
// (more are re-read from LDS), then compacts the kept set in index order.
__device__ void top_k_and_trace(const PyrGeom& g, int C, int level, const int* cand,
                                const float* score, int* rank, int* kept, float* kscore,
                                int* nkept, int32_t* tr_ids, float* tr_scores) {
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
  const int K = g.K;
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
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) cnt += __popcll(__ballot(kr[ch] >= t));
      for (int ch = 4; ch < nch; ++ch) cnt += __popcll(__ballot(keys[ch * 64 + l] >= t));
      if (cnt >= K) T = t;
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
      if (tr_scores) tr_scores[level * (K + 1) + K] = key_score(rej);  // best rejected candidate
      *nkept = K;
    }
  }
  __syncthreads();
  if (tr_ids) {
    for (int j = tid; j < K; j += kThreads) tr_ids[level * K + j] = kept[j];
  }
  if (tr_scores) {
    for (int j = tid; j < K; j += kThreads) tr_scores[level * (K + 1) + j] = kscore[j];
  }
}

// Candidates of one level into cand[]; returns the count.  Must be called by
// every thread (ends with a barrier).
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
  for (int j = threadIdx.x; j < C; j += kThreads)
    cand[j] = j < nchild ? kept[j / b] * b + j % b : base + (j - nchild);
  __syncthreads();
  return C;
}

// Levels with <= K candidates keep them all (no scoring).
__device__ void keep_all(const PyrGeom& g, int C, int level, const int* cand, int* kept,
                         int* nkept, int32_t* tr_ids, float* tr_scores) {
  const int K = g.K;
  for (int j = threadIdx.x; j < K; j += kThreads) {
    const int id = j < C ? cand[j] : -1;
    kept[j] = id;
    if (tr_ids) tr_ids[level * K + j] = id;
  }
  if (tr_scores)
    for (int j = threadIdx.x; j <= K; j += kThreads) tr_scores[level * (K + 1) + j] = NAN;
  if (threadIdx.x == 0) *nkept = C;
  __syncthreads();
}

__device__ __forceinline__ void write_route(const PyrGeom& g, int64_t unit, const int* kept,
                                            int nk, int diag, int32_t* sel) {
  int32_t* out = sel + unit * (g.K + 1);
  for (int j = threadIdx.x; j <= g.K; j += kThreads) out[j] = j < nk ? kept[j] : (j == nk ? diag : -1);
}

// ---------------------------------------------------------------------------
// bf16 prefill path: MFMA scoring.  MT = 16-row M tiles per wave.
// ---------------------------------------------------------------------------

// Pooled keys of chunk c (fp32 rows of the level) -> registers.  Slot s of a
// thread is float4 number tid + s*kThreads of the chunk's kChunk x D block.
template <int D>
__device__ __forceinline__ void load_chunk(const float* lvl, const int* cand, int C, int c,
                                           float4* stg) {
  constexpr int SLOTS = kChunk * (D / 4) / kThreads;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int idx = threadIdx.x + s * kThreads;
    const int cc = idx / (D / 4), d4 = idx % (D / 4);
    const int j = c * kChunk + cc;
    stg[s] = j < C ? *reinterpret_cast<const float4*>(lvl + (int64_t)cand[j] * D + d4 * 4)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Registers -> hi/lo bf16 rows of one LDS stage.
template <int D>
__device__ __forceinline__ void store_chunk(const float4* stg, bf16_t* hi, bf16_t* lo) {
  constexpr int SLOTS = kChunk * (D / 4) / kThreads;
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int idx = threadIdx.x + s * kThreads;
    const int cc = idx / (D / 4), d4 = idx % (D / 4);
    const float4 x = stg[s];
    bf16x4 h, r;
    h[0] = (__bf16)x.x;
    h[1] = (__bf16)x.y;
    h[2] = (__bf16)x.z;
    h[3] = (__bf16)x.w;
    r[0] = (__bf16)(x.x - (float)h[0]);
    r[1] = (__bf16)(x.y - (float)h[1]);
    r[2] = (__bf16)(x.z - (float)h[2]);
    r[3] = (__bf16)(x.w - (float)h[3]);
    *reinterpret_cast<bf16x4*>(hi + cc * (D + 8) + d4 * 4) = h;
    *reinterpret_cast<bf16x4*>(lo + cc * (D + 8) + d4 * 4) = r;
  }
}

// Values of a lane's partner in the other 16-lane row (xor 16) or the other
// 32-lane half (xor 32): the swap hands each lane the pair (even, odd) of the
// two lanes, so a symmetric merge of the pair needs no select.
__device__ __forceinline__ void lse_swap_merge16(float& m, float& s) {
  const auto rm = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  const auto rs = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  m = __uint_as_float(rm[0]);
  s = __uint_as_float(rs[0]);
  lse2_merge(m, s, __uint_as_float(rm[1]), __uint_as_float(rs[1]));
}
__device__ __forceinline__ void lse_swap_merge32(float& m, float& s) {
  const auto rm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  const auto rs = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  m = __uint_as_float(rm[0]);
  s = __uint_as_float(rs[0]);
  lse2_merge(m, s, __uint_as_float(rm[1]), __uint_as_float(rs[1]));
}

// LogSumExp (log2 domain: max m and sum s of 2^(x - m)) of one wave's rows for
// the 16 candidates of an N tile; lane l ends with the value of candidate
// l % 16.  Row j of M tile mt in the C layout is row 4*(l/16) + j; FULL skips
// the per-row validity bits.
template <int MT, bool FULL>
__device__ __forceinline__ void tile_lse(const f32x4 (&acc)[MT], uint32_t rowvalid, float sl2,
                                         float& m, float& s) {
  m = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (FULL || (rowvalid >> (mt * 4 + j) & 1u)) m = fmaxf(m, acc[mt][j]);
  s = 0.f;
  m *= sl2;
  if (m != -INFINITY) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (FULL || (rowvalid >> (mt * 4 + j) & 1u))
          s += __builtin_amdgcn_exp2f(fmaf(acc[mt][j], sl2, -m));
  }
  lse_swap_merge16(m, s);
  lse_swap_merge32(m, s);
}

template <int D, int MT>
__global__ __launch_bounds__(kThreads) void select_mfma(const bf16_t* __restrict__ q,
                                                        const float* __restrict__ pyr,
                                                        int32_t* __restrict__ sel,
                                                        int32_t* __restrict__ trace_ids,
                                                        float* __restrict__ trace_scores,
                                                        PyrGeom g) {
  static_assert(kChunk * (D / 4) % kThreads == 0, "chunk must split evenly");
  constexpr int SLOTS = kChunk * (D / 4) / kThreads;
  constexpr int STAGE = 2 * kChunk * (D + 8);  // bf16 elements per stage (hi then lo)
  extern __shared__ __align__(16) unsigned char smem[];
  const SelLayout lay(g.K, g.branching, D, true);
  int* kept = reinterpret_cast<int*>(smem + lay.off_kept);
  float* kscore = reinterpret_cast<float*>(smem + lay.off_kscore);
  int* cand = reinterpret_cast<int*>(smem + lay.off_cand);
  float* score = reinterpret_cast<float*>(smem + lay.off_score);
  int* rank = reinterpret_cast<int*>(smem + lay.off_rank);
  float2* part = reinterpret_cast<float2*>(smem + lay.off_part);
  bf16_t* hl = reinterpret_cast<bf16_t*>(smem + lay.off_hl);
  __shared__ int s_nkept;
  __shared__ int s_anc[PYR_MAX_LEVELS];

  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
  const int64_t unit = blockIdx.x;
  const int i = (int)(unit % g.nqb);
  const int64_t bhk = unit / g.nqb;  // b * Hk + hk
  const int bi = (int)(bhk / g.Hk), hk = (int)(bhk % g.Hk);
  const int diag = i;
  const int RW = MT * 16;  // rows per wave
  const float sl2 = g.scale * PYR_LOG2E;
  const int cmax = lay.cmax;

  if (tid == 0) s_nkept = 0;
  ancestors(g, diag, s_anc);

  // Q fragments (A operand): lane holds row (l % 16) of each M tile and the
  // 8 consecutive d at 32*ks + 8*(l/16).
  uint4 qa[MT][D / 32];
  uint32_t rowvalid = 0;  // bit (mt*4 + j): C-layout row 4*(l/16)+j of tile mt is a real row
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ra = w * RW + mt * 16 + (l % 16);
    const int h = ra / PYR_BLOCK, t = ra % PYR_BLOCK;
    const int64_t tok = min<int64_t>((int64_t)i * PYR_BLOCK + t, g.Tq - 1);
    const bf16_t* qrow = q + (((int64_t)bi * g.Hq + (int64_t)hk * g.G + h) * g.Tq + tok) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qa[mt][ks] = ld16(qrow + ks * 32 + 8 * (l / 16));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rc = w * RW + mt * 16 + 4 * (l / 16) + j;
      if ((int64_t)i * PYR_BLOCK + rc % PYR_BLOCK < g.Tq) rowvalid |= 1u << (mt * 4 + j);
    }
  }

  const bool full = (int64_t)(i + 1) * PYR_BLOCK <= g.Tq;  // every row of the unit is real
  const float* slab = pyr + bhk * g.n_tot * D;
  int32_t* tr_ids = trace_ids ? trace_ids + unit * g.L * g.K : nullptr;
  float* tr_sc = trace_scores ? trace_scores + unit * g.L * (g.K + 1) : nullptr;
  __syncthreads();

  for (int level = g.L - 1; level >= 0; --level) {
    const int C = build_candidates(g, level, s_anc, kept, s_nkept, cand);
    if (C <= g.K) {
      keep_all(g, C, level, cand, kept, &s_nkept, tr_ids, tr_sc);
      continue;
    }
    const float* lvl = slab + g.loff[level] * D;
    const int nchunks = (C + kChunk - 1) / kChunk;
    float4 stg[SLOTS];
    load_chunk<D>(lvl, cand, C, 0, stg);
    store_chunk<D>(stg, hl, hl + kChunk * (D + 8));
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      if (c + 1 < nchunks) load_chunk<D>(lvl, cand, C, c + 1, stg);  // in flight during the MFMAs
      const bf16_t* hi = hl + (c & 1) * STAGE;
      const bf16_t* lo = hi + kChunk * (D + 8);
#pragma unroll
      for (int nt = 0; nt < kChunk / 16; ++nt) {
        if (c * kChunk + nt * 16 >= C) break;  // uniform
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const bf16_t* bh_row = hi + (nt * 16 + (l % 16)) * (D + 8) + 8 * (l / 16);
        const bf16_t* bl_row = lo + (nt * 16 + (l % 16)) * (D + 8) + 8 * (l / 16);
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 bhv = as_bf16x8(*reinterpret_cast<const uint4*>(bh_row + ks * 32));
          const bf16x8 blv = as_bf16x8(*reinterpret_cast<const uint4*>(bl_row + ks * 32));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[mt][ks]), bhv, acc[mt], 0, 0, 0);
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[mt][ks]), blv, acc[mt], 0, 0, 0);
          }
        }
        // this wave's LogSumExp over its rows, per candidate (lane column l % 16)
        float m, s;
        if (full)
          tile_lse<MT, true>(acc, rowvalid, sl2, m, s);
        else
          tile_lse<MT, false>(acc, rowvalid, sl2, m, s);
        if (l < 16) part[w * cmax + c * kChunk + nt * 16 + l] = make_float2(m, s);
      }
      if (c + 1 < nchunks) {
        bf16_t* nhi = hl + ((c + 1) & 1) * STAGE;
        store_chunk<D>(stg, nhi, nhi + kChunk * (D + 8));
      }
      __syncthreads();
    }
    for (int j = tid; j < C; j += kThreads) {
      float m = -INFINITY, s = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float2 p = part[ww * cmax + j];
        lse2_merge(m, s, p.x, p.y);
      }
      const float sc = (m + log2f(s)) * PYR_LN2;
      score[j] = sc == sc ? sc : -INFINITY;  // a NaN score ranks last
    }
    __syncthreads();
    top_k_and_trace(g, C, level, cand, score, rank, kept, kscore, &s_nkept, tr_ids, tr_sc);
  }
  write_route(g, unit, kept, s_nkept, diag, sel);
}

// ---------------------------------------------------------------------------
// Generic path: fp32 dot products on the vector ALUs (fp32 inputs, decode,
// group sizes the MFMA path does not tile).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void select_valu(const T* __restrict__ q,
                                                        const float* __restrict__ pyr,
                                                        int32_t* __restrict__ sel,
                                                        int32_t* __restrict__ trace_ids,
                                                        float* __restrict__ trace_scores,
                                                        PyrGeom g) {
  extern __shared__ __align__(16) unsigned char smem[];
  const SelLayout lay(g.K, g.branching, D, false);
  int* kept = reinterpret_cast<int*>(smem + lay.off_kept);
  float* kscore = reinterpret_cast<float*>(smem + lay.off_kscore);
  int* cand = reinterpret_cast<int*>(smem + lay.off_cand);
  float* score = reinterpret_cast<float*>(smem + lay.off_score);
  int* rank = reinterpret_cast<int*>(smem + lay.off_rank);
  float* zbuf = reinterpret_cast<float*>(smem + lay.off_zbuf);
  __shared__ int s_nkept;
  __shared__ int s_anc[PYR_MAX_LEVELS];

  const int tid = threadIdx.x;
  const int64_t unit = blockIdx.x;
  const int i = (int)(unit % g.nqb);
  const int64_t bhk = unit / g.nqb;
  const int bi = (int)(bhk / g.Hk), hk = (int)(bhk % g.Hk);
  int64_t tok0, ntok;
  int diag;
  if (g.decode) {
    tok0 = 0;
    ntok = 1;
    diag = (int)((g.Tk - 1) / PYR_BLOCK);
  } else {
    tok0 = (int64_t)i * PYR_BLOCK;
    ntok = min<int64_t>(PYR_BLOCK, g.Tq - tok0);
    diag = i;
  }
  const int R = (int)(g.G * ntok);
  const float sl2 = g.scale * PYR_LOG2E;
  const float* slab = pyr + bhk * g.n_tot * D;
  int32_t* tr_ids = trace_ids ? trace_ids + unit * g.L * g.K : nullptr;
  float* tr_sc = trace_scores ? trace_scores + unit * g.L * (g.K + 1) : nullptr;
  const int chv = max(1, kZbuf / R);
  if (tid == 0) s_nkept = 0;
  ancestors(g, diag, s_anc);
  __syncthreads();

  for (int level = g.L - 1; level >= 0; --level) {
    const int C = build_candidates(g, level, s_anc, kept, s_nkept, cand);
    if (C <= g.K) {
      keep_all(g, C, level, cand, kept, &s_nkept, tr_ids, tr_sc);
      continue;
    }
    const float* lvl = slab + g.loff[level] * D;
    for (int c0 = 0; c0 < C; c0 += chv) {
      const int nch = min(chv, C - c0);
      for (int p = tid; p < nch * R; p += kThreads) {
        const int cc = p / R, r = p % R;
        const int h = (int)(r / ntok);
        const int64_t tok = tok0 + r % ntok;
        const T* qrow = q + (((int64_t)bi * g.Hq + (int64_t)hk * g.G + h) * g.Tq + tok) * D;
        const float* krow = lvl + (int64_t)cand[c0 + cc] * D;
        float acc = 0.f;
        for (int d0 = 0; d0 < D; d0 += 16 / (int)sizeof(T)) {
          float x[16 / sizeof(T)];
          unpack16<T>(ld16(qrow + d0), x);
#pragma unroll
          for (int e = 0; e < (int)(16 / sizeof(T)); ++e) acc = fmaf(x[e], krow[d0 + e], acc);
        }
        zbuf[cc * R + r] = acc * sl2;
      }
      __syncthreads();
      for (int cc = tid; cc < nch; cc += kThreads) {
        float m = -INFINITY;
        for (int r = 0; r < R; ++r) m = fmaxf(m, zbuf[cc * R + r]);
        float s = 0.f;
        for (int r = 0; r < R; ++r) s += exp2f(zbuf[cc * R + r] - m);
        const float sc = (m + log2f(s)) * PYR_LN2;
        score[c0 + cc] = sc == sc ? sc : -INFINITY;  // a NaN score ranks last
      }
      __syncthreads();
    }
    top_k_and_trace(g, C, level, cand, score, rank, kept, kscore, &s_nkept, tr_ids, tr_sc);
  }
  write_route(g, unit, kept, s_nkept, diag, sel);
}

int mfma_tiles(const PyrGeom& g, int dtype) {
  if (dtype != 1 || g.decode) return 0;
  switch (g.G) {
    case 1: return 1;
    case 2: return 2;
    case 4: return 4;
    case 8: return 8;
    default: return 0;
  }
}

template <int D>
hipError_t launch_select_d(const PyrGeom& g, int dtype, const void* q, const float* pyr,
                           int32_t* sel, int32_t* tid_, float* tsc, hipStream_t st) {
  const int64_t units = (int64_t)g.B * g.Hk * g.nqb;
  if (units == 0) return hipSuccess;
  const int mt = mfma_tiles(g, dtype);
  const dim3 grid((unsigned)units), block(kThreads);
  const size_t lds = SelLayout(g.K, g.branching, D, mt != 0).total;
  if (mt) {
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    switch (mt) {
      case 1: hipLaunchKernelGGL((select_mfma<D, 1>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
      case 2: hipLaunchKernelGGL((select_mfma<D, 2>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
      case 4: hipLaunchKernelGGL((select_mfma<D, 4>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
      default: hipLaunchKernelGGL((select_mfma<D, 8>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
    }
  } else if (dtype == 1) {
    hipLaunchKernelGGL((select_valu<bf16_t, D>), grid, block, lds, st,
                       static_cast<const bf16_t*>(q), pyr, sel, tid_, tsc, g);
  } else {
    hipLaunchKernelGGL((select_valu<float, D>), grid, block, lds, st,
                       static_cast<const float*>(q), pyr, sel, tid_, tsc, g);
  }
  return hipGetLastError();
}

}  // namespace

size_t pyr_select_lds_bytes(const PyrGeom& g, int dtype) {
  return SelLayout(g.K, g.branching, g.D, mfma_tiles(g, dtype) != 0).total;
}

hipError_t pyr_launch_select(const PyrGeom& g, int dtype, const void* q, const float* pyr,
                             int32_t* sel, int32_t* trace_ids, float* trace_scores,
                             hipStream_t st) {
  return g.D == 64 ? launch_select_d<64>(g, dtype, q, pyr, sel, trace_ids, trace_scores, st)
                   : launch_select_d<128>(g, dtype, q, pyr, sel, trace_ids, trace_scores, st);
}
