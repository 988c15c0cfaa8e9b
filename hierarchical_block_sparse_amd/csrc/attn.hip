// Block-sparse causal attention over the selected blocks, on gfx950.
//
// PHBA (Prefix-State Hybrid Block Attention) §A.1.3: a query tile streams its
// routed key/value blocks straight from their original HBM layout and keeps
// online-softmax accumulators on chip, writing the output and its log-sum-exp;
// §3.1: the current block gives local causal attention.  PHAROS notes that
// selected keys and values go through FlashAttention-style kernels.
//
// Kernels:
//  * attn_prefill_mfma (bf16): one workgroup per (unit, group of NW heads);
//    each wave owns one head's 64 query rows of the unit.  For every selected
//    block the K tile is staged in LDS row-major and the V tile transposed
//    (so PV reads keys contiguously), then S^T = K Q^T and O^T += V^T P^T run on
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  With keys on the M side
//    of S^T, each lane holds one query row: the row max and sum need a single
//    cross-half shuffle, and P^T feeds the PV MFMA as its B operand straight from
//    registers.  Online softmax in fp32, log2 domain.  Q stays in VGPRs.
//  * attn_prefill_valu: fp32 (or any dtype) reference-precision path, one
//    thread per query row, fp32 dot products.
//  * attn_decode_split + attn_decode_combine: decode (one query token per
//    sequence).  The selected blocks of a unit are split across workgroups so
//    the HBM-bound KV stream fills the chip; partial (max, sum, O) triples go to
//    the workspace and are merged with the LogSumExp rule.
#include <math.h>

#include "pyr_device.h"
#include "pyr_internal.h"

namespace {

constexpr int kMaxSel = 1024;  // route-row capacity staged in LDS (K+1 <= this)

// Heavy-first unit order: query blocks with more selected blocks start first;
// consecutive workgroups cycle over (batch, KV head), so workgroup w lands on
// XCD w % 8 together with the other query blocks of the same KV heads.
__device__ __forceinline__ void unit_of(const PyrGeom& g, int64_t u_ord, int& bi, int& hk,
                                        int& i, int64_t& unit) {
  const int64_t nbhk = (int64_t)g.B * g.Hk;
  i = g.nqb - 1 - (int)(u_ord / nbhk);
  const int64_t bhk = u_ord % nbhk;
  bi = (int)(bhk / g.Hk);
  hk = (int)(bhk % g.Hk);
  unit = bhk * g.nqb + i;
}

// ---------------------------------------------------------------------------
// bf16 prefill, MFMA
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_prefill_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ sel, bf16_t* __restrict__ o, float* __restrict__ lse, PyrGeom g,
    int wg_per_unit) {
  constexpr int NT = NW * 64;
  constexpr int KS = D + 8;   // K tile row stride (elements): 16-byte pad
  constexpr int VS = 64 + 4;  // V^T tile row stride (elements): 8-byte pad
  constexpr int SEG = D / 8;  // 16-byte segments per row
  __shared__ __align__(16) bf16_t Ks[64 * KS];
  __shared__ __align__(16) bf16_t Vt[D * VS];
  __shared__ int s_sel[kMaxSel];

  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
  const int half = l / 32, lr = l % 32;
  const int sub = (int)(blockIdx.x % wg_per_unit);
  int bi, hk, i;
  int64_t unit;
  unit_of(g, blockIdx.x / wg_per_unit, bi, hk, i, unit);
  const int h = hk * g.G + sub * NW + w;
  const float sl2 = g.scale * PYR_LOG2E;
  const int64_t row0 = (int64_t)i * PYR_BLOCK;  // first query token of the unit

  // route row -> LDS (entries outside [0, nb) are skipped below)
  for (int jj = tid; jj <= g.K; jj += NT) s_sel[jj] = sel[unit * (g.K + 1) + jj];

  // Q^T fragments (B operand): lane holds query row rt*32 + lr and d = ks*16 + 8*half .. +7
  const bf16_t* qh = q + ((int64_t)bi * g.Hq + h) * g.Tq * D;
  uint4 qb[2][D / 16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int64_t tok = row0 + rt * 32 + lr;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qb[rt][ks] = tok < g.Tq ? ld16(qh + tok * D + ks * 16 + 8 * half) : make_uint4(0, 0, 0, 0);
  }

  f32x16 oacc[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][rt][e] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const bf16_t* kh = k + ((int64_t)bi * g.Hk + hk) * g.Tk * D;
  const bf16_t* vh = v + ((int64_t)bi * g.Hk + hk) * g.Tk * D;
  __syncthreads();

  for (int jj = 0; jj <= g.K; ++jj) {
    const int j = s_sel[jj];
    if (j < 0 || j >= g.nb) continue;  // uniform across the workgroup
    const int64_t key0 = (int64_t)j * PYR_BLOCK;
    __syncthreads();  // previous tile fully consumed
    // K tile, row-major
    for (int s = tid; s < 64 * SEG; s += NT) {
      const int key = s / SEG, seg = s % SEG;
      const int64_t kp = key0 + key;
      const uint4 x = kp < g.Tk ? ld16(kh + kp * D + seg * 8) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(Ks + key * KS + seg * 8) = x;
    }
    // V tile, transposed: 4 keys x 8 dims per slot
    for (int s = tid; s < 16 * SEG; s += NT) {
      const int kg = s / SEG, seg = s % SEG;
      uint4 r[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int64_t kp = key0 + kg * 4 + rr;
        r[rr] = kp < g.Tk ? ld16(vh + kp * D + seg * 8) : make_uint4(0, 0, 0, 0);
      }
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&r[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&r[1]);
      const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&r[2]);
      const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e / 2, sh = (e % 2) * 16;
        const uint32_t a0 = (r0[wd] >> sh) & 0xffffu, a1 = (r1[wd] >> sh) & 0xffffu;
        const uint32_t a2 = (r2[wd] >> sh) & 0xffffu, a3 = (r3[wd] >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(Vt + (seg * 8 + e) * VS + kg * 4) =
            make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
      }
    }
    __syncthreads();

    // S^T = K Q^T: [64 keys x 64 rows] as 2x2 tiles of 32x32
    f32x16 sacc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kt][rt][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(Ks + (kt * 32 + lr) * KS + ks * 16 + 8 * half));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          sacc[kt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(qb[rt][ks]), sacc[kt][rt], 0, 0, 0);
      }
    }

    // online softmax per query row (lane's row = rt*32 + lr)
    const bool need_mask = key0 + PYR_BLOCK - 1 > row0;  // only the diagonal (or later) block
    uint4 pb[2][2][2];  // [rt][kt][ks2] P^T fragments as bf16x8
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t rp = row0 + rt * 32 + lr;
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = sacc[kt][rt][e] * sl2;
          if (need_mask) {
            const int64_t kp = key0 + kt * 32 + (e / 4) * 8 + half * 4 + (e % 4);
            if (kp > rp) x = -INFINITY;
          }
          sacc[kt][rt][e] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[rt], mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run[rt] - m_new);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = m_new == -INFINITY ? 0.f : exp2f(sacc[kt][rt][e] - m_new);
          sacc[kt][rt][e] = p;
          psum += p;
        }
      l_run[rt] = l_run[rt] * alpha + psum;
      m_run[rt] = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][rt][e] *= alpha;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int e0 = k2 * 8;
          pb[rt][kt][k2] = make_uint4(pack_bf16x2(sacc[kt][rt][e0 + 0], sacc[kt][rt][e0 + 1]),
                                      pack_bf16x2(sacc[kt][rt][e0 + 2], sacc[kt][rt][e0 + 3]),
                                      pack_bf16x2(sacc[kt][rt][e0 + 4], sacc[kt][rt][e0 + 5]),
                                      pack_bf16x2(sacc[kt][rt][e0 + 6], sacc[kt][rt][e0 + 7]));
        }
    }

    // O^T += V^T P^T.  MFMA k index 8*half + jj maps to key
    // kt*32 + 16*k2 + 4*half + jj (jj < 4) or + 8 + (jj - 4) (jj >= 4), the
    // order in which the S^T accumulator holds P.
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const bf16_t* vrow = Vt + (dt * 32 + lr) * VS + kt * 32 + 16 * k2 + 4 * half;
          const uint2 a0 = *reinterpret_cast<const uint2*>(vrow);
          const uint2 a1 = *reinterpret_cast<const uint2*>(vrow + 8);
          const bf16x8 a = as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y));
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            oacc[dt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(pb[rt][kt][k2]), oacc[dt][rt], 0, 0, 0);
        }
    }
  }

  // finalize: rows of this lane = rt*32 + lr; dims of oacc[dt][rt][e] =
  // dt*32 + (e/4)*8 + half*4 + e%4
  bf16_t* oh = o + ((int64_t)bi * g.Hq + h) * g.Tq * D;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float lt = l_run[rt] + __shfl_xor(l_run[rt], 32, 64);
    const int64_t tok = row0 + rt * 32 + lr;
    if (tok >= g.Tq) continue;
    const float inv = 1.f / lt;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dt * 32 + g4 * 8 + half * 4;
        const uint2 pk = make_uint2(pack_bf16x2(oacc[dt][rt][g4 * 4 + 0] * inv, oacc[dt][rt][g4 * 4 + 1] * inv),
                                    pack_bf16x2(oacc[dt][rt][g4 * 4 + 2] * inv, oacc[dt][rt][g4 * 4 + 3] * inv));
        *reinterpret_cast<uint2*>(oh + tok * D + d0) = pk;
      }
    if (lse && half == 0) lse[((int64_t)bi * g.Hq + h) * g.Tq + tok] = (m_run[rt] + log2f(lt)) * PYR_LN2;
  }
}

// ---------------------------------------------------------------------------
// fp32 (any dtype) prefill on the vector ALUs: one thread per query row.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_prefill_valu(const T* __restrict__ q,
                                                        const T* __restrict__ k,
                                                        const T* __restrict__ v,
                                                        const int32_t* __restrict__ sel,
                                                        T* __restrict__ o, float* __restrict__ lse,
                                                        PyrGeom g) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ float Kt[64][D];
  __shared__ float Vt[64][D];
  __shared__ int s_sel[kMaxSel];
  const int t = threadIdx.x;
  const int hsub = (int)(blockIdx.x % g.G);
  int bi, hk, i;
  int64_t unit;
  unit_of(g, blockIdx.x / g.G, bi, hk, i, unit);
  const int h = hk * g.G + hsub;
  const float sl2 = g.scale * PYR_LOG2E;
  const int64_t rp = (int64_t)i * PYR_BLOCK + t;
  const bool valid = rp < g.Tq;
  for (int jj = t; jj <= g.K; jj += 64) s_sel[jj] = sel[unit * (g.K + 1) + jj];
  float qr[D], acc[D];
  const T* qrow = q + (((int64_t)bi * g.Hq + h) * g.Tq + (valid ? rp : 0)) * D;
  for (int d0 = 0; d0 < D; d0 += VEC) {
    float x[VEC];
    unpack16<T>(ld16(qrow + d0), x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qr[d0 + e] = x[e] * sl2;
  }
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const T* kh = k + ((int64_t)bi * g.Hk + hk) * g.Tk * D;
  const T* vh = v + ((int64_t)bi * g.Hk + hk) * g.Tk * D;
  __syncthreads();
  for (int jj = 0; jj <= g.K; ++jj) {
    const int j = s_sel[jj];
    if (j < 0 || j >= g.nb) continue;  // uniform across the workgroup
    const int64_t key0 = (int64_t)j * PYR_BLOCK;
    __syncthreads();
    for (int s = t; s < 64 * (D / VEC); s += 64) {
      const int key = s / (D / VEC), c = (s % (D / VEC)) * VEC;
      const int64_t kp = key0 + key;
      float xk[VEC], xv[VEC];
      if (kp < g.Tk) {
        unpack16<T>(ld16(kh + kp * D + c), xk);
        unpack16<T>(ld16(vh + kp * D + c), xv);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) xk[e] = xv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        Kt[key][c + e] = xk[e];
        Vt[key][c + e] = xv[e];
      }
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int key = 0; key < 64; ++key) {
      if (key0 + key > rp) break;  // keys are ascending: the rest are in the future
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qr[d], Kt[key][d], s);
      mx = fmaxf(mx, s);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;
    const float alpha = exp2f(m - m_new);
    lsum *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
    for (int key = 0; key < 64; ++key) {
      if (key0 + key > rp) break;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qr[d], Kt[key][d], s);
      const float p = exp2f(s - m_new);
      lsum += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vt[key][d], acc[d]);
    }
    m = m_new;
  }
  if (!valid) return;
  T* orow = o + (((int64_t)bi * g.Hq + h) * g.Tq + rp) * D;
  const float inv = 1.f / lsum;
  for (int d = 0; d < D; ++d) {
    const float y = acc[d] * inv;
    if constexpr (sizeof(T) == 4)
      orow[d] = y;
    else
      orow[d] = (T)f32_to_bf16_bits(y);
  }
  if (lse) lse[((int64_t)bi * g.Hq + h) * g.Tq + rp] = (m + log2f(lsum)) * PYR_LN2;
}

// ---------------------------------------------------------------------------
// Decode: split selected blocks across workgroups, then merge.
// ---------------------------------------------------------------------------
constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecMaxRows = 4 * kDecWaves;  // G <= 16
constexpr int kDecBlocksPerSplit = 8;

__host__ __device__ inline int decode_splits(int K) {
  return (K + 1 + kDecBlocksPerSplit - 1) / kDecBlocksPerSplit;
}

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void attn_decode_split(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ sel, float* __restrict__ ws, PyrGeom g, int nsplit) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int SEG = D / VEC;
  constexpr int SLOTS = 64 * SEG / kDecThreads;  // 16-byte loads per thread per tile
  constexpr int DPL = D / 64;                    // output dims per lane
  static_assert(SLOTS * kDecThreads == 64 * SEG, "tile must split evenly");
  __shared__ float Ks[64][D + 4];
  __shared__ float Vs[64][D];
  __shared__ float qs[kDecMaxRows][D];
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
  const int split = (int)(blockIdx.x % nsplit);
  const int64_t bhk = blockIdx.x / nsplit;  // unit (decode: one query block)
  const int bi = (int)(bhk / g.Hk), hk = (int)(bhk % g.Hk);
  const int G = g.G;
  const float sl2 = g.scale * PYR_LOG2E;
  const int64_t qpos = g.Tk - 1;
  for (int idx = tid; idx < G * D; idx += kDecThreads) {
    const int r = idx / D, d = idx % D;
    const T* qrow = q + ((int64_t)bi * g.Hq + (int64_t)hk * G + r) * D;  // Tq == 1
    float x;
    if constexpr (sizeof(T) == 4)
      x = reinterpret_cast<const float*>(qrow)[d];
    else
      x = bf16_to_f32(reinterpret_cast<const uint16_t*>(qrow)[d]);
    qs[r][d] = x * sl2;
  }
  // this split's blocks
  const int32_t* srow = sel + bhk * (g.K + 1);
  const int jb0 = split * kDecBlocksPerSplit;
  const int jb1 = min(g.K + 1, jb0 + kDecBlocksPerSplit);
  const T* kh = k + ((int64_t)bi * g.Hk + hk) * g.Tk * D;
  const T* vh = v + ((int64_t)bi * g.Hk + hk) * g.Tk * D;

  float m_r[4], l_r[4], acc[4][DPL];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    m_r[rr] = -INFINITY;
    l_r[rr] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[rr][e] = 0.f;
  }

  uint4 rk[SLOTS], rv[SLOTS];
  auto fetch = [&](int j) {
#pragma unroll
    for (int sl = 0; sl < SLOTS; ++sl) {
      const int s = tid + sl * kDecThreads;
      const int key = s / SEG, c = (s % SEG) * VEC;
      const int64_t kp = (int64_t)j * PYR_BLOCK + key;
      const bool ok = j >= 0 && j < g.nb && kp < g.Tk;
      rk[sl] = ok ? ld16_nt(kh + kp * D + c) : make_uint4(0, 0, 0, 0);
      rv[sl] = ok ? ld16_nt(vh + kp * D + c) : make_uint4(0, 0, 0, 0);
    }
  };
  int jj = jb0;
  while (jj < jb1 && !(srow[jj] >= 0 && srow[jj] < g.nb)) ++jj;
  if (jj < jb1) fetch(srow[jj]);
  while (jj < jb1) {
    const int j = srow[jj];
    int nx = jj + 1;
    while (nx < jb1 && !(srow[nx] >= 0 && srow[nx] < g.nb)) ++nx;
    __syncthreads();  // previous tile consumed, q staged
#pragma unroll
    for (int sl = 0; sl < SLOTS; ++sl) {
      const int s = tid + sl * kDecThreads;
      const int key = s / SEG, c = (s % SEG) * VEC;
      float xk[VEC], xv[VEC];
      unpack16<T>(rk[sl], xk);
      unpack16<T>(rv[sl], xv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        Ks[key][c + e] = xk[e];
        Vs[key][c + e] = xv[e];
      }
    }
    __syncthreads();
    if (nx < jb1) fetch(srow[nx]);
    const int64_t kp = (int64_t)j * PYR_BLOCK + l;
    const bool vis = kp <= qpos;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = w + rr * kDecWaves;
      if (r >= G) break;
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; d += 4) {
        const float4 kk = *reinterpret_cast<const float4*>(&Ks[l][d]);
        const float4 qq = *reinterpret_cast<const float4*>(&qs[r][d]);
        s = fmaf(qq.x, kk.x, s);
        s = fmaf(qq.y, kk.y, s);
        s = fmaf(qq.z, kk.z, s);
        s = fmaf(qq.w, kk.w, s);
      }
      const float x = vis ? s : -INFINITY;
      const float mb = wave_max(x);
      const float m_new = fmaxf(m_r[rr], mb);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_r[rr] - m_new);
      const float p = m_new == -INFINITY ? 0.f : exp2f(x - m_new);
      l_r[rr] = l_r[rr] * alpha + wave_sum(p);
      m_r[rr] = m_new;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[rr][e] *= alpha;
#pragma unroll 16
      for (int key = 0; key < 64; ++key) {
        const float pk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), key));
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[rr][e] = fmaf(pk, Vs[key][l * DPL + e], acc[rr][e]);
      }
    }
    jj = nx;
  }
  // partial results: ws[((bhk*G + r)*nsplit + split)*(D+2) + {0: m, 1: l, 2..: acc}]
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = w + rr * kDecWaves;
    if (r >= G) break;
    float* dst = ws + (((int64_t)bhk * G + r) * nsplit + split) * (D + 2);
    if (l == 0) {
      dst[0] = m_r[rr];
      dst[1] = l_r[rr];
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) dst[2 + l * DPL + e] = acc[rr][e];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_decode_combine(const float* __restrict__ ws,
                                                          T* __restrict__ o,
                                                          float* __restrict__ lse, PyrGeom g,
                                                          int nsplit) {
  constexpr int DPL = D / 64;
  const int64_t row = blockIdx.x;  // (bhk * G + r)
  const int l = threadIdx.x;
  float m = -INFINITY, s = 0.f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* src = ws + (row * nsplit + sp) * (D + 2);
    const float m2 = src[0], s2 = src[1];
    const float mx = fmaxf(m, m2);
    if (mx == -INFINITY) continue;
    const float a1 = exp2f(m - mx), a2 = exp2f(m2 - mx);
    s = s * a1 + s2 * a2;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = acc[e] * a1 + src[2 + l * DPL + e] * a2;
    m = mx;
  }
  const int64_t bhk = row / g.G;
  const int r = (int)(row % g.G);
  const int bi = (int)(bhk / g.Hk), hk = (int)(bhk % g.Hk);
  const int64_t qh = (int64_t)bi * g.Hq + (int64_t)hk * g.G + r;  // Tq == 1
  const float inv = 1.f / s;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const float y = acc[e] * inv;
    if constexpr (sizeof(T) == 4)
      o[qh * D + l * DPL + e] = y;
    else
      o[qh * D + l * DPL + e] = (T)f32_to_bf16_bits(y);
  }
  if (lse && l == 0) lse[qh] = (m + log2f(s)) * PYR_LN2;
}

template <int D>
hipError_t launch_attn_d(const PyrGeom& g, int dtype, const void* q, const void* k,
                         const void* v, const int32_t* sel, void* o, float* lse, void* ws,
                         hipStream_t st) {
  const int64_t units = (int64_t)g.B * g.Hk * g.nqb;
  if (units == 0 || g.Tq == 0) return hipSuccess;
  if (g.decode) {
    const int ns = decode_splits(g.K);
    float* wsf = static_cast<float*>(ws);
    if (dtype == 1) {
      hipLaunchKernelGGL((attn_decode_split<bf16_t, D>), dim3((unsigned)(units * ns)),
                         dim3(kDecThreads), 0, st, static_cast<const bf16_t*>(q),
                         static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), sel, wsf,
                         g, ns);
      hipLaunchKernelGGL((attn_decode_combine<bf16_t, D>), dim3((unsigned)(units * g.G)),
                         dim3(64), 0, st, wsf, static_cast<bf16_t*>(o), lse, g, ns);
    } else {
      hipLaunchKernelGGL((attn_decode_split<float, D>), dim3((unsigned)(units * ns)),
                         dim3(kDecThreads), 0, st, static_cast<const float*>(q),
                         static_cast<const float*>(k), static_cast<const float*>(v), sel, wsf, g,
                         ns);
      hipLaunchKernelGGL((attn_decode_combine<float, D>), dim3((unsigned)(units * g.G)),
                         dim3(64), 0, st, wsf, static_cast<float*>(o), lse, g, ns);
    }
    return hipGetLastError();
  }
  if (dtype == 1) {
    const int nw = g.G % 4 == 0 ? 4 : (g.G % 2 == 0 ? 2 : 1);
    const int wpu = g.G / nw;
    const dim3 grid((unsigned)(units * wpu));
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    const bf16_t* kk = static_cast<const bf16_t*>(k);
    const bf16_t* vv = static_cast<const bf16_t*>(v);
    bf16_t* oo = static_cast<bf16_t*>(o);
    if (nw == 4)
      hipLaunchKernelGGL((attn_prefill_mfma<D, 4>), grid, dim3(256), 0, st, qq, kk, vv, sel, oo, lse, g, wpu);
    else if (nw == 2)
      hipLaunchKernelGGL((attn_prefill_mfma<D, 2>), grid, dim3(128), 0, st, qq, kk, vv, sel, oo, lse, g, wpu);
    else
      hipLaunchKernelGGL((attn_prefill_mfma<D, 1>), grid, dim3(64), 0, st, qq, kk, vv, sel, oo, lse, g, wpu);
  } else {
    hipLaunchKernelGGL((attn_prefill_valu<float, D>), dim3((unsigned)(units * g.G)), dim3(64), 0,
                       st, static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), sel, static_cast<float*>(o), lse, g);
  }
  return hipGetLastError();
}

}  // namespace

size_t pyr_attn_ws_bytes(const PyrGeom& g) {
  if (!g.decode) return 0;
  return (size_t)g.B * g.Hk * g.G * decode_splits(g.K) * (g.D + 2) * sizeof(float);
}

hipError_t pyr_launch_attn(const PyrGeom& g, int dtype, const void* q, const void* k,
                           const void* v, const int32_t* sel, void* o, float* lse, void* ws,
                           hipStream_t st) {
  return g.D == 64 ? launch_attn_d<64>(g, dtype, q, k, v, sel, o, lse, ws, st)
                   : launch_attn_d<128>(g, dtype, q, k, v, sel, o, lse, ws, st);
}
