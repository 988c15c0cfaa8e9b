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
// Scoring, bf16 path: rows are the M side of v_mfma_f32_16x16x32_bf16 and
// candidates the N side; each wave keeps its rows of Q in VGPRs for the whole
// unit.  Pooled keys are fp32; each is split into hi = bf16(x) and
// lo = bf16(x - hi) and both are contracted against the exact bf16 q, so a dot
// product carries ~2^-17 relative error instead of bf16's 2^-9.  The build
// stores the hi/lo rows beside the means (plane 1), and candidates go through
// LDS in chunks of 32 with direct global-to-LDS loads, two stages deep (one
// barrier per chunk); in decode (a 16-row tile holding the G query rows) each
// wave scores its own chunks instead.  Each wave reduces its rows' LogSumExp
// per candidate in-lane and across its 4 lane groups with shuffles, as (max,
// sum) pairs in the log2 domain; the waves' partials are merged once per
// level.  Generic path (fp32 inputs, and bf16 group sizes the MFMA tiles do
// not cover): fp32 dot products on the vector ALUs, same selection logic.
#include <math.h>

#include "pyr_device.h"
#include "pyr_internal.h"

#include "select_core.h"

namespace {

// ---------------------------------------------------------------------------
// Generic path: fp32 dot products on the vector ALUs (fp32 inputs, prefill
// and decode; bf16 group sizes the MFMA path does not tile).
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
  __shared__ float s_margin[1];
  __shared__ int s_anc[PYR_MAX_LEVELS];

  const int tid = threadIdx.x;
  int64_t unit;
  if (!sel_unit(g, unit)) return;
  const int i = (int)(unit % g.nqb);
  const int64_t bhk = unit / g.nqb;
  const int bi = (int)(bhk / g.Hk), hk = (int)(bhk % g.Hk);
  const PyrSeq sq = pyr_seq(g, bi);
  if (i >= sq.nqb) {
    blank_unit<kThreads>(g, unit, sel, trace_ids, trace_scores);
    return;
  }
  int64_t tok0, ntok;
  int diag;
  if (g.decode) {
    tok0 = 0;
    ntok = 1;
    diag = (int)((g.Tk - 1) / PYR_BLOCK);
  } else {
    tok0 = (int64_t)i * PYR_BLOCK;
    ntok = min<int64_t>(PYR_BLOCK, sq.Tq - tok0);
    diag = i;
  }
  const int R = (int)(g.G * ntok);
  const int Ku = unit_budget(g, hk);
  const float sl2 = g.scale * PYR_LOG2E;
  const float* slab = pyr + bhk * g.planes * g.n_tot * D;  // plane 0: fp32 means
  int32_t* tr_ids = trace_ids ? trace_ids + unit * g.L * g.K : nullptr;
  float* tr_sc = trace_scores ? trace_scores + unit * g.L * (g.K + 1) : nullptr;
  const int chv = max(1, kZbuf / R);
  if (tid == 0) s_nkept = 0;
  ancestors(g, diag, s_anc);
  __syncthreads();

  for (int level = g.L - 1; level >= 0; --level) {
    const int C = build_candidates<kThreads>(g, level, s_anc, kept, s_nkept, cand);
    if (C <= Ku) {
      keep_all<kThreads>(g, C, level, cand, kept, &s_nkept, tr_ids, tr_sc);
      continue;
    }
    const float* lvl = slab + g.loff[level] * D;
    for (int c0 = 0; c0 < C; c0 += chv) {
      const int nch = min(chv, C - c0);
      for (int p = tid; p < nch * R; p += kThreads) {
        const int cc = p / R, r = p % R;
        const int h = (int)(r / ntok);
        const int64_t tok = tok0 + r % ntok;
        const T* qrow = q + (sq.q0 + ((int64_t)hk * g.G + h) * sq.qhs + tok) * D;
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
    for (int kk = Ku;;) {
      top_k_and_trace<kThreads>(g, C, level, cand, score, rank, kept, kscore, &s_nkept, kk, s_margin,
                      tr_ids, tr_sc);
      if (!fallback_due(g, level, kk, Ku, s_margin)) break;
      kk = C < g.fb_k ? C : g.fb_k;  // keep more of the same candidates
    }
  }
  write_route<kThreads>(g, unit, kept, s_nkept, diag, sel);
}

int mfma_tiles(const PyrGeom& g, int dtype) {
  if (dtype != 1) return 0;
  if (g.decode) return g.G <= 16 ? 1 : 0;  // the G rows in one 16-row tile
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
  const dim3 grid((unsigned)((units + 7) / 8 * 8)), block(kThreads);  // whole runs per XCD
  const size_t lds = SelLayout(g.K, g.branching, D, mt != 0, mt == 8 ? 8 : kWaves).total;
  if (mt) {
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    switch (mt) {
      case 1:
        if (g.decode)
          hipLaunchKernelGGL((select_mfma<D, 1, 4, true>), grid, block, lds, st, qq, pyr, sel, tid_,
                             tsc, g);
        else
          hipLaunchKernelGGL((select_mfma<D, 1, 4>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g);
        break;
      case 2: hipLaunchKernelGGL((select_mfma<D, 2, 4>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
      case 4: hipLaunchKernelGGL((select_mfma<D, 4, 4>), grid, block, lds, st, qq, pyr, sel, tid_, tsc, g); break;
      default:  // G = 8: eight waves of four M tiles
        hipLaunchKernelGGL((select_mfma<D, 4, 8>), grid, dim3(512), lds, st, qq, pyr, sel, tid_, tsc, g);
        break;
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
  const bool mfma = mfma_tiles(g, dtype) != 0;
  // dynamic layout, plus the candidate stages of the MFMA path (a static array)
  return SelLayout(g.K, g.branching, g.D, mfma, mfma_tiles(g, dtype) == 8 ? 8 : kWaves).total +
         (mfma ? (size_t)(g.decode ? kSelStagesDecode : kSelStages) * kChunk * 4 * g.D : 0);
}

hipError_t pyr_launch_select(const PyrGeom& g, int dtype, const void* q, const float* pyr,
                             int32_t* sel, int32_t* trace_ids, float* trace_scores,
                             hipStream_t st) {
  return g.D == 64 ? launch_select_d<64>(g, dtype, q, pyr, sel, trace_ids, trace_scores, st)
                   : launch_select_d<128>(g, dtype, q, pyr, sel, trace_ids, trace_scores, st);
}
