// Pooled key pyramid on gfx950.
//
// PISA (peercurrent.com record), abstract: keys are pooled into a
// coarse-to-fine hierarchy of O(log N) levels.  PHBA (Prefix-State Hybrid
// Block Attention), §A.1.2: a block summary is the mean of the block's valid
// key rows, accumulated in fp32 registers.  Here node m of level l is the mean
// of all key tokens under it; levels are stored finest first in one fp32 plane
// per (batch, KV head).  For bf16 problems a second plane repeats every mean
// as a bf16 pair (hi = bf16(x), lo = bf16(x - hi)), the operands of the
// selection's matrix-core scorer, so that the scorer can stream them into LDS
// without converting.
//
// Two kernels:
//  * build_chunk: one workgroup per chunk of `chunk` = b^s consecutive 64-token
//    blocks of one (batch, KV head).  It streams the chunk's keys from HBM once
//    (16-byte loads, several blocks in flight per thread), reduces each block
//    to its mean, then folds the chunk's nodes up s levels inside LDS.  This is
//    the HBM-bound pass: every key byte is read exactly once.
//  * build_level: one launch per remaining level (above level s), one thread
//    per (node, column) of every slab, reading the children from the output
//    slab (a few hundred KiB at most, in L2).
// A parent is the token-weighted mean of its children, so a ragged last block
// or a ragged last node gives the exact token mean.
#include "pyr_device.h"
#include "pyr_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunkMax = 16;  // finest blocks per workgroup (b^s <= 16)
constexpr int kBatch = 4;      // blocks whose loads are in flight together

// Store the mean x of column dcol of node `node` of a slab: plane 0 in fp32,
// and for two-plane slabs the bf16 pair in plane 1 (the hi row, then the lo
// row, in the node's 4D bytes).
template <int D>
__device__ __forceinline__ void put_node(const PyrGeom& g, float* slab, int64_t node, int dcol,
                                         float x) {
  slab[node * D + dcol] = x;
  if (g.planes == 2) {
    bf16_t* split = reinterpret_cast<bf16_t*>(slab + g.n_tot * D) + node * 2 * D;
    const __bf16 hi = (__bf16)x;
    const __bf16 lo = (__bf16)(x - (float)hi);
    split[dcol] = __builtin_bit_cast(bf16_t, hi);
    split[D + dcol] = __builtin_bit_cast(bf16_t, lo);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void build_chunk(const T* __restrict__ k,
                                                        float* __restrict__ pyr, PyrGeom g,
                                                        int chunk, int s_levels,
                                                        int chunks_per_bh) {
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte load
  constexpr int TPR = D / VEC;          // threads per key row
  constexpr int RPP = kThreads / TPR;   // rows per pass of the workgroup
  constexpr int PASSES = PYR_BLOCK / RPP;
  static_assert(PYR_BLOCK % RPP == 0, "rows per pass must divide the block");

  __shared__ float part[kBatch][RPP][D];
  __shared__ float nodes[2][kChunkMax][D];

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / chunks_per_bh;
  const int c = blockIdx.x % chunks_per_bh;
  const PyrSeq sq = pyr_seq(g, (int)(bh / g.Hk));
  const int64_t blk0 = (int64_t)c * chunk;
  const int nblk = (int)min<int64_t>(chunk, sq.nb - blk0);
  if (nblk <= 0) return;  // past the end of a shorter packed sequence
  const T* kb = k + (sq.k0 + (bh % g.Hk) * sq.khs) * D;
  float* slab = pyr + bh * g.planes * g.n_tot * D;

  const int col = (tid % TPR) * VEC;
  const int r0 = tid / TPR;

  for (int jb = 0; jb < nblk; jb += kBatch) {
    uint4 raw[kBatch][PASSES];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const int64_t tok = (blk0 + jb + u) * PYR_BLOCK + r0 + p * RPP;
        if (jb + u < nblk && tok < sq.Tk)
          raw[u][p] = ld16_nt(kb + tok * D + col);
        else
          raw[u][p] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      float acc[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        float x[VEC];
        unpack16<T>(raw[u][p], x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += x[e];
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) part[u][r0][col + e] = acc[e];
    }
    __syncthreads();
    for (int idx = tid; idx < kBatch * D; idx += kThreads) {
      const int u = idx / D, dcol = idx % D;
      if (jb + u < nblk) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < RPP; ++r) s += part[u][r][dcol];
        const int64_t m = blk0 + jb + u;
        const float mean = s / (float)pyr_node_tokens(sq.Tk, g.branching, 0, m);
        nodes[0][jb + u][dcol] = mean;
        put_node<D>(g, slab, g.loff[0] + m, dcol, mean);
      }
    }
    __syncthreads();
  }

  // Fold the chunk up s levels inside LDS (token-weighted means).
  int cur = 0;
  int n_below = nblk;
  int64_t first_below = blk0;  // global index of the chunk's first node one level down
  for (int lvl = 1; lvl <= s_levels; ++lvl) {
    const int b = g.branching;
    const int n_here = (n_below + b - 1) / b;
    const int64_t first_here = first_below / b;
    for (int idx = tid; idx < n_here * D; idx += kThreads) {
      const int m = idx / D, dcol = idx % D;
      float num = 0.f, den = 0.f;
      for (int j = 0; j < b; ++j) {
        const int cidx = m * b + j;
        if (cidx < n_below) {
          const float w = (float)pyr_node_tokens(sq.Tk, b, lvl - 1, first_below + cidx);
          num += nodes[cur][cidx][dcol] * w;
          den += w;
        }
      }
      const float mean = num / den;
      nodes[cur ^ 1][m][dcol] = mean;
      put_node<D>(g, slab, g.loff[lvl] + first_here + m, dcol, mean);
    }
    __syncthreads();
    cur ^= 1;
    n_below = n_here;
    first_below = first_here;
  }
}

// Valid nodes of level `lvl` for a sequence of nb blocks (one above its root).
__device__ __forceinline__ int64_t level_valid(int64_t nb, int b, int lvl) {
  for (int l = 0; l < lvl; ++l) nb = nb > 1 ? (nb + b - 1) / b : 1;
  return nb;
}

// One level above the chunks: one thread per (node, column), nodes of every
// slab spread over the whole grid (a level is one launch, the launches of
// consecutive levels are ordered by the stream).
template <int D>
__global__ __launch_bounds__(kThreads) void build_level(float* __restrict__ pyr, PyrGeom g,
                                                        int lvl, int wg_per_bh) {
  const int64_t bh = blockIdx.x / wg_per_bh;
  const int64_t idx = (int64_t)(blockIdx.x % wg_per_bh) * kThreads + threadIdx.x;
  const PyrSeq sq = pyr_seq(g, (int)(bh / g.Hk));
  const int b = g.branching;
  const int64_t n_below = level_valid(sq.nb, b, lvl - 1);
  const int64_t n_here = sq.nb ? level_valid(sq.nb, b, lvl) : 0;
  const int64_t m = idx / D;
  if (m >= n_here) return;
  const int dcol = (int)(idx % D);
  float* slab = pyr + bh * g.planes * g.n_tot * D;
  const float* below = slab + g.loff[lvl - 1] * D;
  float num = 0.f, den = 0.f;
  for (int j = 0; j < b; ++j) {
    const int64_t cidx = m * b + j;
    if (cidx < n_below) {
      const float w = (float)pyr_node_tokens(sq.Tk, b, lvl - 1, cidx);
      num += below[cidx * D + dcol] * w;
      den += w;
    }
  }
  put_node<D>(g, slab, g.loff[lvl] + m, dcol, num / den);
}

__device__ __forceinline__ float key_f32(float x) { return x; }
__device__ __forceinline__ float key_f32(bf16_t x) { return bf16_to_f32(x); }

// Decode-time maintenance: one workgroup per (batch, KV head) recomputes every
// node over the tokens [old_len, Tk): the level-0 nodes of the affected blocks
// as the mean of their valid key rows, then, level by level, the affected
// ancestors as token-weighted means of their children (the children are up to
// date by then).  Nodes outside those ranges are not touched.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void append_nodes(const T* __restrict__ k,
                                                         float* __restrict__ pyr, PyrGeom g,
                                                         int64_t old_len) {
  constexpr int NG = kThreads / D;  // row groups of the level-0 reduction
  __shared__ float part[NG][D];
  const int64_t bh = blockIdx.x;
  const T* kb = k + bh * g.Tks * D;
  float* slab = pyr + bh * g.planes * g.n_tot * D;
  const int tid = threadIdx.x, dcol = tid % D, rg = tid / D;
  int64_t a0 = old_len / PYR_BLOCK, a1 = (g.Tk - 1) / PYR_BLOCK;  // affected blocks
  for (int64_t j = a0; j <= a1; ++j) {
    const int64_t t0 = j * PYR_BLOCK;
    const int64_t t1 = t0 + PYR_BLOCK < g.Tk ? t0 + PYR_BLOCK : g.Tk;
    float s = 0.f;
    for (int64_t t = t0 + rg; t < t1; t += NG) s += key_f32(kb[t * D + dcol]);
    part[rg][dcol] = s;
    __syncthreads();
    if (rg == 0) {
      float tot = 0.f;
#pragma unroll
      for (int r = 0; r < NG; ++r) tot += part[r][dcol];
      put_node<D>(g, slab, g.loff[0] + j, dcol, tot / (float)(t1 - t0));
    }
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();
  const int b = g.branching;
  for (int lvl = 1; lvl < g.L; ++lvl) {
    a0 /= b;
    a1 /= b;
    const int64_t n_below = g.lsize[lvl - 1];
    const float* below = slab + g.loff[lvl - 1] * D;
    for (int64_t idx = tid; idx < (a1 - a0 + 1) * D; idx += kThreads) {
      const int64_t m = a0 + idx / D;
      const int c = (int)(idx % D);
      float num = 0.f, den = 0.f;
      for (int jj = 0; jj < b; ++jj) {
        const int64_t cidx = m * b + jj;
        if (cidx < n_below) {
          const float w = (float)pyr_node_tokens(g.Tk, b, lvl - 1, cidx);
          num += below[cidx * D + c] * w;
          den += w;
        }
      }
      put_node<D>(g, slab, g.loff[lvl] + m, c, num / den);
    }
    __threadfence_block();
    __syncthreads();
  }
}

template <typename T, int D>
hipError_t launch_append_t(const PyrGeom& g, const void* k, int64_t old_len, float* pyr,
                           hipStream_t st) {
  const int64_t n_bh = (int64_t)g.B * g.Hk;
  if (n_bh == 0 || old_len >= g.Tk) return hipSuccess;
  hipLaunchKernelGGL((append_nodes<T, D>), dim3((unsigned)n_bh), dim3(kThreads), 0, st,
                     static_cast<const T*>(k), pyr, g, old_len);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_build_t(const PyrGeom& g, const void* k, float* pyr, hipStream_t st) {
  const int64_t n_bh = (int64_t)g.B * g.Hk;
  if (n_bh == 0 || g.nb == 0) return hipSuccess;
  // s = levels folded inside a workgroup: the largest s with b^s <= kChunkMax
  // and s < L (never past the root).
  int s = 0, chunk = 1;
  while ((int64_t)chunk * g.branching <= kChunkMax && s + 1 < g.L) {
    chunk *= g.branching;
    ++s;
  }
  const int chunks_per_bh = (g.nb + chunk - 1) / chunk;
  hipLaunchKernelGGL((build_chunk<T, D>), dim3((unsigned)(n_bh * chunks_per_bh)),
                     dim3(kThreads), 0, st, static_cast<const T*>(k), pyr, g, chunk, s,
                     chunks_per_bh);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int lvl = s + 1; lvl < g.L && e == hipSuccess; ++lvl) {
    const int64_t wg = ((int64_t)g.lsize[lvl] * D + kThreads - 1) / kThreads;  // longest sequence
    hipLaunchKernelGGL((build_level<D>), dim3((unsigned)(n_bh * wg)), dim3(kThreads), 0, st, pyr,
                       g, lvl, (int)wg);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t pyr_launch_build(const PyrGeom& g, int dtype, const void* k, float* pyr,
                            hipStream_t st) {
  if (dtype == 1) {
    return g.D == 64 ? launch_build_t<bf16_t, 64>(g, k, pyr, st)
                     : launch_build_t<bf16_t, 128>(g, k, pyr, st);
  }
  return g.D == 64 ? launch_build_t<float, 64>(g, k, pyr, st)
                   : launch_build_t<float, 128>(g, k, pyr, st);
}

hipError_t pyr_launch_append(const PyrGeom& g, int dtype, const void* k, int64_t old_len,
                             float* pyr, hipStream_t st) {
  if (dtype == 1) {
    return g.D == 64 ? launch_append_t<bf16_t, 64>(g, k, old_len, pyr, st)
                     : launch_append_t<bf16_t, 128>(g, k, old_len, pyr, st);
  }
  return g.D == 64 ? launch_append_t<float, 64>(g, k, old_len, pyr, st)
                   : launch_append_t<float, 128>(g, k, old_len, pyr, st);
}
