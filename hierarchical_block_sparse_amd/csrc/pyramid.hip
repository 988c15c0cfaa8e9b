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
// Launches:
//  * build_chunk: one workgroup per chunk of `chunk` = b^s consecutive 64-token
//    blocks of one (batch, KV head).  It streams the chunk's keys from HBM once
//    (16-byte loads, several blocks in flight per thread), reduces each block
//    to its mean -- the rows a wave holds are summed across its lanes with
//    lane swaps, the waves' sums through LDS -- then folds the chunk's nodes
//    up s levels inside LDS.  This is the HBM-bound pass: every key byte is
//    read exactly once.
//  * build_fold: the levels above s, t per launch (b^(t-1) <= 64): one
//    workgroup per group of b^t nodes of the level below computes the first
//    level from the children in the slab (in L2) and folds the rest in LDS.
//    At 128K tokens (b = 4) one launch covers levels 3..6; at 1M, two.
// A parent is the token-weighted mean of its children, so a ragged last block
// or a ragged last node gives the exact token mean.
#include "pyr_device.h"
#include "pyr_internal.h"

namespace {

typedef __attribute__((address_space(3))) void lds_void;

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

// Sum of x over the lanes of a wave that share lane % TPR (the row groups of
// one column slice): lane swaps for the 16- and 32-lane partners, a shuffle
// below that.  Every lane of the group ends with the same sum.
template <int TPR>
__device__ __forceinline__ float rowgroup_sum(float x) {
#pragma unroll
  for (int o = TPR; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
  if (TPR <= 16) x = sum16(x);
  return sum32(x);
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
  constexpr int NWV = kThreads / 64;    // waves
  static_assert(PYR_BLOCK % RPP == 0, "rows per pass must divide the block");
  static_assert(TPR >= 8 && TPR <= 32 && 64 % TPR == 0, "a row spans 8 to 32 lanes");

  // per-wave row sums; rows padded by 4 floats so that the 4 waves' sums of a
  // column sit in 4 different banks when one lane reads them
  __shared__ __align__(16) float part[kBatch][NWV][D + 4];
  __shared__ float nodes[2][kChunkMax][D];

  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
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

  // The keys of batch jb+kBatch are loaded while batch jb's sums cross the
  // waves through LDS: a batch's registers are free once reduced, and the
  // LDS-only barriers do not wait for loads in flight.
  uint4 raw[kBatch][PASSES];
  auto load_batch = [&](int jb) {
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
  };
  load_batch(0);
  for (int jb = 0; jb < nblk; jb += kBatch) {
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
      for (int e = 0; e < VEC; ++e) acc[e] = rowgroup_sum<TPR>(acc[e]);
      if (l < TPR) {
        // with two 16-byte halves per lane (VEC = 8), lane l stores half
        // ((l >> 2) ^ (l >> 3)) & 1 first: each store's 16-byte chunks
        // 2l + h are then distinct modulo 8 within lanes 0-7 and 8-15, and
        // modulo 16 over lanes 0-15 (no bank conflict at 128 or 256 bytes
        // per LDS cycle)
        float4* dst = reinterpret_cast<float4*>(&part[u][w][col]);
        constexpr int NH = VEC / 4;
        const int flip = NH == 2 ? ((l >> 2) ^ (l >> 3)) & 1 : 0;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          const int h = hh ^ flip;
          dst[h] = make_float4(acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]);
        }
      }
    }
    if (jb + kBatch < nblk) load_batch(jb + kBatch);
    lds_barrier();
    for (int idx = tid; idx < kBatch * D; idx += kThreads) {
      const int u = idx / D, dcol = idx % D;
      if (jb + u < nblk) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NWV; ++ww) s += part[u][ww][dcol];
        const int64_t m = blk0 + jb + u;
        const float mean = s / (float)pyr_node_tokens(sq.Tk, g.branching, 0, m);
        nodes[0][jb + u][dcol] = mean;
        put_node<D>(g, slab, g.loff[0] + m, dcol, mean);
      }
    }
    lds_barrier();
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

constexpr int kFoldThreads = 512;
constexpr int kFoldNodes = 64;  // nodes of the first folded level one workgroup holds in LDS

// Levels lo+1 .. lo+t of one (batch, KV head), one workgroup per group of
// b^t consecutive level-lo nodes (b^(t-1) <= kFoldNodes).  The first level
// is computed from the children read from the slab (in L2: written by the
// previous launch), with every thread's loads in flight together; the
// remaining t-1 levels are folded in LDS.  Every level produced is written.
template <int D>
__global__ __launch_bounds__(kFoldThreads) void build_fold(float* __restrict__ pyr, PyrGeom g,
                                                           int lo, int t, int groups_per_bh) {
  __shared__ __align__(16) float nodes[2][kFoldNodes][D];
  constexpr int C4 = D / 4;  // float4 column groups per node
  const int b = g.branching;
  int gn1 = 1;  // first-level nodes per group: b^(t-1)
  for (int i = 1; i < t; ++i) gn1 *= b;
  const int64_t bh = blockIdx.x / groups_per_bh;
  const int grp = blockIdx.x % groups_per_bh;
  const PyrSeq sq = pyr_seq(g, (int)(bh / g.Hk));
  if (sq.nb == 0) return;
  const int64_t n_lo = level_valid(sq.nb, b, lo);
  const int64_t n_hi = level_valid(sq.nb, b, lo + 1);
  const int64_t first1 = (int64_t)grp * gn1;  // first level-(lo+1) node of the group
  if (first1 >= n_hi) return;
  const int cnt1 = (int)min<int64_t>(gn1, n_hi - first1);
  float* slab = pyr + bh * g.planes * g.n_tot * D;
  const float* below = slab + g.loff[lo] * D;

  // level lo+1: one float4 column group of one node per work item; a
  // thread's PER items read their children four at a time, loads first
  constexpr int PER = kFoldNodes * C4 / kFoldThreads;
  static_assert(kFoldNodes * C4 % kFoldThreads == 0, "items must split evenly");
  float4 num[PER];
  float den[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    num[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    den[u] = 0.f;
  }
  for (int j0 = 0; j0 < b; j0 += 4) {
    float4 x[PER][4];
    float wv[PER][4];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int idx = u * kFoldThreads + threadIdx.x;
      const int64_t node = first1 + idx / C4;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t cidx = node * b + j0 + jj;
        const bool ok = idx < cnt1 * C4 && j0 + jj < b && cidx < n_lo;
        x[u][jj] = ok ? *reinterpret_cast<const float4*>(below + cidx * D + 4 * (idx % C4))
                      : make_float4(0.f, 0.f, 0.f, 0.f);
        wv[u][jj] = ok ? (float)pyr_node_tokens(sq.Tk, b, lo, cidx) : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < PER; ++u)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        num[u].x += x[u][jj].x * wv[u][jj];
        num[u].y += x[u][jj].y * wv[u][jj];
        num[u].z += x[u][jj].z * wv[u][jj];
        num[u].w += x[u][jj].w * wv[u][jj];
        den[u] += wv[u][jj];
      }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = u * kFoldThreads + threadIdx.x;
    if (idx < cnt1 * C4) {
      const int m = idx / C4, c4 = idx % C4;
      const float mean[4] = {num[u].x / den[u], num[u].y / den[u], num[u].z / den[u],
                             num[u].w / den[u]};
      *reinterpret_cast<float4*>(&nodes[0][m][4 * c4]) = make_float4(mean[0], mean[1], mean[2], mean[3]);
#pragma unroll
      for (int e = 0; e < 4; ++e) put_node<D>(g, slab, g.loff[lo + 1] + first1 + m, 4 * c4 + e, mean[e]);
    }
  }
  __syncthreads();
  // levels lo+2 .. lo+t in LDS
  int cur = 0, n_below = cnt1;
  int64_t first_below = first1;
  for (int lvl = lo + 2; lvl <= lo + t; ++lvl) {
    const int n_here = (n_below + b - 1) / b;
    const int64_t first_here = first_below / b;
    for (int idx = threadIdx.x; idx < n_here * D; idx += kFoldThreads) {
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

__device__ __forceinline__ float key_f32(float x) { return x; }
__device__ __forceinline__ float key_f32(bf16_t x) { return bf16_to_f32(x); }

// Sum of column dcol over the rows t0 + rg, t0 + rg + NG, ... below t1 of one
// block, in that order; every row's load is issued before the first add.
template <typename T, int D, int NG>
__device__ __forceinline__ float block_col_sum(const T* kb, int64_t t0, int64_t t1, int rg,
                                               int dcol) {
  constexpr int RPT = PYR_BLOCK / NG;
  float x[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int64_t t = t0 + rg + (int64_t)r * NG;
    x[r] = key_f32(kb[(t < t1 ? t : t1 - 1) * D + dcol]);  // rows past t1: loaded, not added
  }
  __builtin_amdgcn_sched_barrier(0);  // every load issued before the first add waits
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    if (t0 + rg + (int64_t)r * NG < t1) s += x[r];
  return s;
}

// Siblings an append to one block can need: the children before the affected
// one, summed over the levels (b - 1 per level at most).
constexpr int kSibMax = 32;

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
  __shared__ float sib[kSibMax][D];
  const int64_t bh = blockIdx.x;
  const T* kb = k + bh * g.Tks * D;
  float* slab = pyr + bh * g.planes * g.n_tot * D;
  const int tid = threadIdx.x, dcol = tid % D, rg = tid / D;
  const int b = g.branching;
  int64_t a0 = old_len / PYR_BLOCK, a1 = (g.Tk - 1) / PYR_BLOCK;  // affected blocks

  // One affected block (every decode step that stays inside a block).  It is
  // the last block, so the affected node of each level is the last valid one:
  // its children are the p = anc % b nodes before the affected child (older
  // tokens only, untouched here) and that child.  Those siblings load together
  // with the block's rows, and the thread of each column then folds the levels
  // in registers -- the same operations in the same order as the general loop
  // below, without a round trip through memory per level.
  if (a0 == a1) {
    // block ids stay below 2^30, so 32-bit arithmetic suffices here
    const uint32_t ub = (uint32_t)b;
    int nsib = 0;
    for (uint32_t an = (uint32_t)a0, lvl = 1; lvl < (uint32_t)g.L; ++lvl, an /= ub) nsib += (int)(an % ub);
    if (nsib <= kSibMax) {
      const int64_t t0 = a0 * PYR_BLOCK;
      const int64_t t1 = t0 + PYR_BLOCK < g.Tk ? t0 + PYR_BLOCK : g.Tk;
      // sibling e (levels in order, children in order) goes straight to LDS
      // row sib[e], loaded by row group e % NG; a row group is whole waves,
      // each wave taking 64 consecutive columns
      const int wrg = __builtin_amdgcn_readfirstlane(rg);
      const int c0 = __builtin_amdgcn_readfirstlane(dcol - (tid % 64));
      uint32_t an = (uint32_t)a0;
      for (int lvl = 1, e = 0; lvl < g.L; ++lvl, an /= ub) {
        const uint32_t p = an % ub;
        const int64_t first = g.loff[lvl - 1] + (an - p);
        for (uint32_t jj = 0; jj < p; ++jj, ++e)
          if (e % NG == wrg)
            __builtin_amdgcn_global_load_lds((const void*)(slab + (first + jj) * D + dcol),
                                             (lds_void*)&sib[e][c0], 4, 0, 0);
      }
      part[rg][dcol] = block_col_sum<T, D, NG>(kb, t0, t1, rg, dcol);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's siblings are in LDS
      __syncthreads();
      if (rg != 0) return;
      float tot = 0.f;
#pragma unroll
      for (int r = 0; r < NG; ++r) tot += part[r][dcol];
      float v = tot / (float)(t1 - t0);
      put_node<D>(g, slab, g.loff[0] + a0, dcol, v);
      uint32_t m = (uint32_t)a0;  // the affected node of the level below
      for (int lvl = 1, e = 0; lvl < g.L; ++lvl) {
        const uint32_t p = m % ub;
        float num = 0.f, den = 0.f;
        for (uint32_t jj = 0; jj < p; ++jj, ++e) {
          const float w = (float)pyr_node_tokens(g.Tk, b, lvl - 1, (int64_t)(m - p + jj));
          num += sib[e][dcol] * w;
          den += w;
        }
        const float w = (float)pyr_node_tokens(g.Tk, b, lvl - 1, (int64_t)m);
        num += v * w;
        den += w;
        v = num / den;
        m /= ub;
        put_node<D>(g, slab, g.loff[lvl] + m, dcol, v);
      }
      return;
    }
  }

  for (int64_t j = a0; j <= a1; ++j) {
    const int64_t t0 = j * PYR_BLOCK;
    const int64_t t1 = t0 + PYR_BLOCK < g.Tk ? t0 + PYR_BLOCK : g.Tk;
    part[rg][dcol] = block_col_sum<T, D, NG>(kb, t0, t1, rg, dcol);
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
  // the levels above s, as many per launch as one workgroup's LDS allows
  for (int lo = s; lo + 1 < g.L && e == hipSuccess;) {
    int t = 1, gn1 = 1;
    while (lo + t + 1 < g.L && (int64_t)gn1 * g.branching <= kFoldNodes) {
      gn1 *= g.branching;
      ++t;
    }
    const int64_t groups = ((int64_t)g.lsize[lo + 1] + gn1 - 1) / gn1;  // longest sequence
    hipLaunchKernelGGL((build_fold<D>), dim3((unsigned)(n_bh * groups)), dim3(kFoldThreads), 0, st,
                       pyr, g, lo, t, (int)groups);
    e = hipGetLastError();
    lo += t;
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
