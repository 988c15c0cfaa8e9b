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
// lo = bf16(x - hi) in LDS and both are contracted against the exact bf16 q,
// so a dot product carries ~2^-17 relative error instead of bf16's 2^-9.  The
// LogSumExp over rows is reduced in-lane, across the 4 lane groups with
// shuffles, and across waves through LDS, as (max, sum) pairs in the log2
// domain.  Generic path (fp32 inputs, decode, other group sizes): fp32 dot
// products on the vector ALUs, same selection logic.
#include <math.h>

#include "pyr_device.h"
#include "pyr_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 64;        // candidates staged per round (MFMA path)
constexpr int kZbuf = 8192;       // fp32 scratch for the generic path

struct SelLayout {
  int cmax;   // candidate capacity: b*K + b - 1, rounded up to 4
  int off_kept, off_kscore, off_cand, off_score, off_rank, off_pos, off_scratch;
  int total;  // bytes
  __host__ __device__ SelLayout(int K, int b, int scratch_bytes) {
    cmax = (b * K + b - 1 + 3) & ~3;
    int o = 0;
    off_kept = o;   o += 4 * ((K + 3) & ~3);
    off_kscore = o; o += 4 * ((K + 3) & ~3);
    off_cand = o;   o += 4 * cmax;
    off_score = o;  o += 4 * cmax;
    off_rank = o;   o += 4 * cmax;
    off_pos = o;    o += 4 * cmax;
    o = (o + 15) & ~15;
    off_scratch = o;
    total = o + scratch_bytes;
  }
};

template <int D>
constexpr int mfma_scratch_bytes() {
  // part[kWaves][kChunk] float2 + khi/klo[kChunk][D+8] bf16
  return kWaves * kChunk * 8 + 2 * kChunk * (D + 8) * 2;
}

__device__ __forceinline__ int64_t ipow(int b, int e) {
  int64_t r = 1;
  for (int i = 0; i < e; ++i) r *= b;
  return r;
}

// Rank every candidate, keep the top K in ascending index order, write trace.
__device__ void top_k_and_trace(const PyrGeom& g, int C, int level, const int* cand,
                                float* score, int* rank, int* pos, int* kept, float* kscore,
                                int* nkept, int32_t* tr_ids, float* tr_scores) {
  const int tid = threadIdx.x;
  const int K = g.K;
  for (int j = tid; j < C; j += kThreads) {
    float s = score[j];
    if (s != s) score[j] = -INFINITY;  // a NaN score ranks last
  }
  __syncthreads();
  for (int j = tid; j < C; j += kThreads) {
    const float sj = score[j];
    const int cj = cand[j];
    int r = 0;
    for (int jj = 0; jj < C; ++jj) {
      const float s2 = score[jj];
      r += (s2 > sj) || (s2 == sj && cand[jj] < cj);
    }
    rank[j] = r;
  }
  __syncthreads();
  // position among kept, in candidate (= ascending index) order
  for (int j = tid; j < C; j += kThreads) {
    int p = 0;
    if (rank[j] < K)
      for (int jj = 0; jj < j; ++jj) p += rank[jj] < K;
    pos[j] = p;
  }
  __syncthreads();
  for (int j = tid; j < C; j += kThreads) {
    if (rank[j] < K) {
      kept[pos[j]] = cand[j];
      kscore[pos[j]] = score[j];
    } else if (rank[j] == K && tr_scores) {
      tr_scores[level * (K + 1) + K] = score[j];  // best rejected candidate
    }
  }
  __syncthreads();
  if (tr_ids) {
    for (int j = tid; j < K; j += kThreads) tr_ids[level * K + j] = kept[j];
  }
  if (tr_scores) {
    for (int j = tid; j < K; j += kThreads) tr_scores[level * (K + 1) + j] = kscore[j];
  }
  if (tid == 0) *nkept = K;
  __syncthreads();
}

// Candidates of one level into cand[]; returns the count.  Must be called by
// every thread (ends with a barrier).
__device__ int build_candidates(const PyrGeom& g, int level, int64_t diag, const int* kept,
                                int nkept, int* cand) {
  const int b = g.branching;
  const int64_t anc = diag / ipow(b, level);
  int C;
  int64_t base;
  int nchild;
  if (level == g.L - 1) {
    C = (int)anc;
    nchild = 0;
    base = 0;
  } else {
    const int64_t anc_up = diag / ipow(b, level + 1);
    nchild = nkept * b;
    base = anc_up * b;
    C = nchild + (int)(anc - base);
  }
  for (int j = threadIdx.x; j < C; j += kThreads) {
    cand[j] = j < nchild ? kept[j / b] * b + j % b : (int)(base + (j - nchild));
  }
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

// ---------------------------------------------------------------------------
// bf16 prefill path: MFMA scoring.  MT = 16-row M tiles per wave.
// ---------------------------------------------------------------------------
template <int D, int MT>
__global__ __launch_bounds__(kThreads) void select_mfma(const bf16_t* __restrict__ q,
                                                        const float* __restrict__ pyr,
                                                        int32_t* __restrict__ sel,
                                                        int32_t* __restrict__ trace_ids,
                                                        float* __restrict__ trace_scores,
                                                        PyrGeom g) {
  extern __shared__ __align__(16) unsigned char smem[];
  const SelLayout lay(g.K, g.branching, mfma_scratch_bytes<D>());
  int* kept = reinterpret_cast<int*>(smem + lay.off_kept);
  float* kscore = reinterpret_cast<float*>(smem + lay.off_kscore);
  int* cand = reinterpret_cast<int*>(smem + lay.off_cand);
  float* score = reinterpret_cast<float*>(smem + lay.off_score);
  int* rank = reinterpret_cast<int*>(smem + lay.off_rank);
  int* pos = reinterpret_cast<int*>(smem + lay.off_pos);
  float2* part = reinterpret_cast<float2*>(smem + lay.off_scratch);
  bf16_t* khi = reinterpret_cast<bf16_t*>(smem + lay.off_scratch + kWaves * kChunk * 8);
  bf16_t* klo = khi + kChunk * (D + 8);
  __shared__ int s_nkept;

  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
  const int64_t unit = blockIdx.x;
  const int i = (int)(unit % g.nqb);
  const int64_t bhk = unit / g.nqb;  // b * Hk + hk
  const int bi = (int)(bhk / g.Hk), hk = (int)(bhk % g.Hk);
  const int64_t diag = i;
  const int RW = MT * 16;  // rows per wave
  const float sl2 = g.scale * PYR_LOG2E;

  // Q fragments (A operand): lane holds row (l % 16) of each M tile and the
  // 8 consecutive d at 32*ks + 8*(l/16).
  uint4 qa[MT][D / 32];
  uint32_t rowvalid = 0;  // bit (mt*4 + j): C-layout row 4*(l/16)+j of tile mt is a real row
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int ra = w * RW + mt * 16 + (l % 16);
    const int h = ra / PYR_BLOCK, t = ra % PYR_BLOCK;
    const int64_t tok = (int64_t)i * PYR_BLOCK + t;
    const bf16_t* qrow = q + (((int64_t)bi * g.Hq + (int64_t)hk * g.G + h) * g.Tq + tok) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qa[mt][ks] = tok < g.Tq ? ld16(qrow + ks * 32 + 8 * (l / 16)) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rc = w * RW + mt * 16 + 4 * (l / 16) + j;
      const int64_t tc = (int64_t)i * PYR_BLOCK + rc % PYR_BLOCK;
      if (tc < g.Tq) rowvalid |= 1u << (mt * 4 + j);
    }
  }

  const float* slab = pyr + bhk * g.n_tot * D;
  int32_t* tr_ids = trace_ids ? trace_ids + unit * g.L * g.K : nullptr;
  float* tr_sc = trace_scores ? trace_scores + unit * g.L * (g.K + 1) : nullptr;
  if (tid == 0) s_nkept = 0;
  __syncthreads();

  for (int level = g.L - 1; level >= 0; --level) {
    const int C = build_candidates(g, level, diag, kept, s_nkept, cand);
    if (C <= g.K) {
      keep_all(g, C, level, cand, kept, &s_nkept, tr_ids, tr_sc);
      continue;
    }
    const float* lvl = slab + g.loff[level] * D;
    for (int c0 = 0; c0 < C; c0 += kChunk) {
      const int nch = min(kChunk, C - c0);
      // stage pooled keys of this chunk as hi/lo bf16 pairs
      for (int idx = tid; idx < kChunk * (D / 4); idx += kThreads) {
        const int cc = idx / (D / 4), d4 = idx % (D / 4);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (cc < nch) x = *reinterpret_cast<const float4*>(lvl + (int64_t)cand[c0 + cc] * D + d4 * 4);
        const uint32_t h0 = f32_to_bf16_bits(x.x), h1 = f32_to_bf16_bits(x.y);
        const uint32_t h2 = f32_to_bf16_bits(x.z), h3 = f32_to_bf16_bits(x.w);
        const uint32_t l0 = f32_to_bf16_bits(x.x - bf16_to_f32(h0));
        const uint32_t l1 = f32_to_bf16_bits(x.y - bf16_to_f32(h1));
        const uint32_t l2 = f32_to_bf16_bits(x.z - bf16_to_f32(h2));
        const uint32_t l3 = f32_to_bf16_bits(x.w - bf16_to_f32(h3));
        *reinterpret_cast<uint2*>(khi + cc * (D + 8) + d4 * 4) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        *reinterpret_cast<uint2*>(klo + cc * (D + 8) + d4 * 4) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
      }
      __syncthreads();
      for (int nt = 0; nt * 16 < nch; ++nt) {
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const bf16_t* bh_row = khi + (nt * 16 + (l % 16)) * (D + 8) + 8 * (l / 16);
        const bf16_t* bl_row = klo + (nt * 16 + (l % 16)) * (D + 8) + 8 * (l / 16);
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
        float m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (rowvalid >> (mt * 4 + j) & 1u) m = fmaxf(m, acc[mt][j] * sl2);
        float s = 0.f;
        if (m != -INFINITY) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (rowvalid >> (mt * 4 + j) & 1u) s += exp2f(acc[mt][j] * sl2 - m);
        }
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
          const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
          lse2_merge(m, s, m2, s2);
        }
        if (l < 16) part[w * kChunk + nt * 16 + l] = make_float2(m, s);
      }
      __syncthreads();
      for (int cc = tid; cc < nch; cc += kThreads) {
        float m = -INFINITY, s = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          const float2 p = part[ww * kChunk + cc];
          lse2_merge(m, s, p.x, p.y);
        }
        score[c0 + cc] = (m + log2f(s)) * PYR_LN2;
      }
      __syncthreads();
    }
    top_k_and_trace(g, C, level, cand, score, rank, pos, kept, kscore, &s_nkept, tr_ids, tr_sc);
  }

  int32_t* out = sel + unit * (g.K + 1);
  const int nk = s_nkept;
  for (int j = tid; j <= g.K; j += kThreads) out[j] = j < nk ? kept[j] : (j == nk ? (int)diag : -1);
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
  const SelLayout lay(g.K, g.branching, kZbuf * 4);
  int* kept = reinterpret_cast<int*>(smem + lay.off_kept);
  float* kscore = reinterpret_cast<float*>(smem + lay.off_kscore);
  int* cand = reinterpret_cast<int*>(smem + lay.off_cand);
  float* score = reinterpret_cast<float*>(smem + lay.off_score);
  int* rank = reinterpret_cast<int*>(smem + lay.off_rank);
  int* pos = reinterpret_cast<int*>(smem + lay.off_pos);
  float* zbuf = reinterpret_cast<float*>(smem + lay.off_scratch);
  __shared__ int s_nkept;

  const int tid = threadIdx.x;
  const int64_t unit = blockIdx.x;
  const int i = (int)(unit % g.nqb);
  const int64_t bhk = unit / g.nqb;
  const int bi = (int)(bhk / g.Hk), hk = (int)(bhk % g.Hk);
  int64_t tok0, ntok, diag;
  if (g.decode) {
    tok0 = 0;
    ntok = 1;
    diag = (g.Tk - 1) / PYR_BLOCK;
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
  __syncthreads();

  for (int level = g.L - 1; level >= 0; --level) {
    const int C = build_candidates(g, level, diag, kept, s_nkept, cand);
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
        score[c0 + cc] = (m + log2f(s)) * PYR_LN2;
      }
      __syncthreads();
    }
    top_k_and_trace(g, C, level, cand, score, rank, pos, kept, kscore, &s_nkept, tr_ids, tr_sc);
  }

  int32_t* out = sel + unit * (g.K + 1);
  const int nk = s_nkept;
  for (int j = tid; j <= g.K; j += kThreads) out[j] = j < nk ? kept[j] : (j == nk ? (int)diag : -1);
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
  if (mt) {
    const size_t lds = SelLayout(g.K, g.branching, mfma_scratch_bytes<D>()).total;
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    switch (mt) {
      case 1: hipLaunchKernelGGL((select_mfma<D, 1>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
      case 2: hipLaunchKernelGGL((select_mfma<D, 2>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
      case 4: hipLaunchKernelGGL((select_mfma<D, 4>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
      default: hipLaunchKernelGGL((select_mfma<D, 8>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
    }
  } else {
    const size_t lds = SelLayout(g.K, g.branching, kZbuf * 4).total;
    if (dtype == 1)
      hipLaunchKernelGGL((select_valu<bf16_t, D>), grid, block, lds, st,
                         static_cast<const bf16_t*>(q), pyr, sel, tid_, tsc, g);
    else
      hipLaunchKernelGGL((select_valu<float, D>), grid, block, lds, st,
                         static_cast<const float*>(q), pyr, sel, tid_, tsc, g);
  }
  return hipGetLastError();
}

}  // namespace

size_t pyr_select_lds_bytes(const PyrGeom& g, int dtype) {
  if (mfma_tiles(g, dtype))
    return SelLayout(g.K, g.branching,
                     g.D == 64 ? mfma_scratch_bytes<64>() : mfma_scratch_bytes<128>()).total;
  return SelLayout(g.K, g.branching, kZbuf * 4).total;
}

hipError_t pyr_launch_select(const PyrGeom& g, int dtype, const void* q, const float* pyr,
                             int32_t* sel, int32_t* trace_ids, float* trace_scores,
                             hipStream_t st) {
  return g.D == 64 ? launch_select_d<64>(g, dtype, q, pyr, sel, trace_ids, trace_scores, st)
                   : launch_select_d<128>(g, dtype, q, pyr, sel, trace_ids, trace_scores, st);
}
