// Block-sparse causal attention over the selected blocks, on gfx950.
//
// PHBA (Prefix-State Hybrid Block Attention) §A.1.3: a query tile streams its
// routed key/value blocks straight from their original HBM layout and keeps
// online-softmax accumulators on chip, writing the output and its log-sum-exp;
// §3.1: the current block gives local causal attention.  PHAROS notes that
// selected keys and values go through FlashAttention-style kernels.
//
// Kernels:
//  * attn_prefill_mfma (bf16): one workgroup per (unit, group of heads); each
//    wave owns 32 * RT query rows of one head.  For every selected block the K
//    and V tiles are staged in LDS row-major (swizzled), V^T fragments come from
//    transposed LDS reads, and S^T = K Q^T and O^T += V^T P^T run on
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  With keys on the M side
//    of S^T, each lane holds one query row: the row max and sum need a single
//    cross-half shuffle, and P^T feeds the PV MFMA as its B operand straight from
//    registers.  Online softmax in fp32, log2 domain.  Q stays in VGPRs.
//  * attn_prefill_pp (bf16, query heads per KV head a multiple of 4): the same
//    data layout and MFMA shapes with 8 waves of 32 rows in two groups that
//    take turns: while one wave of a SIMD runs the matrix work of a block (its
//    LDS fragment reads and MFMAs), the other runs the vector work (row max,
//    exponentials, bf16 packing), then they swap.
//  * attn_prefill_f32 (fp32): the layout of attn_prefill_mfma with fp32 tiles
//    on v_mfma_f32_32x32x2_f32, fp32 products and accumulation.
//  * attn_decode_mfma (bf16) / attn_decode_split (fp32) + attn_decode_combine:
//    decode (one query token per sequence).  The selected blocks of a unit are
//    split across workgroups so the HBM-bound KV stream fills the chip; partial
//    (max, sum, O) triples go to the workspace and are merged with the
//    LogSumExp rule.  The bf16 kernel scores and accumulates on the matrix
//    cores, the query rows padded to a 16-wide tile.
#include <math.h>

#include <mutex>

#include "../../include/pyr.h"
#include "pyr_device.h"
#include "pyr_internal.h"
#include "select_core.h"

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
//
// K and V tiles of the selected blocks stream global -> LDS with direct
// 16-byte loads (no VGPR staging), double-buffered: the tiles of the next
// selected block are in flight while the current one is computed, and one
// barrier per block separates the two.  Tiles keep the global row-major layout
// with a per-row XOR swizzle of the 16-byte chunks, chosen so that the K reads
// (one row per lane) and the transposed V reads are both free of bank
// conflicts.  V^T fragments for the PV MFMA come from ds_read_b64_tr_b16:
// within each 16-lane group, lane i receives element (i % 4) of the 8-byte
// chunk that lane 4j + i/4 addresses, j = 0..3, so lanes that address a 4-key x
// 16-dim patch row by row receive 4 consecutive keys of one dim each.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kRescaleLog2 = 8.f;  // rescale O only when a row max grows by > 2^8
constexpr int kVtRow = PYR_BLOCK * 2;  // bytes per row of a transposed V tile (attn_vt_build)

template <int D>
struct TileGeom {
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int ROW = 2 * D;            // bytes per row
  static constexpr int TILE = 64 * ROW;        // bytes per K or V tile
  static constexpr int RP = 256 / ROW;         // rows per 256-byte bank sweep
  __device__ static int swz_k(int r) { return (r / RP) % CPR; }
  __device__ static int swz_v(int r) { return 4 * ((r / RP) % (CPR / 4)); }
};

// Issue the K and V tiles of block j into stage st.  Instruction t of a tile
// fills LDS chunks [64t, 64t+64): lane l writes chunk p = 64t + l, i.e. row
// p / CPR, stored chunk p % CPR, which holds logical chunk (p % CPR) ^ swz(row).
// Rows past the sequence end re-read its last row (finite values that the
// causal mask gives zero weight).
template <int D, int NW>
__device__ __forceinline__ void issue_tiles(const bf16_t* kh, const bf16_t* vh, int64_t Tk, int j,
                                            unsigned char* ktile, unsigned char* vtile, int w,
                                            int l) {
  using TG = TileGeom<D>;
  const int64_t key0 = (int64_t)__builtin_amdgcn_readfirstlane(j) * PYR_BLOCK;
  const bf16_t* kb = kh + key0 * D;
  const bf16_t* vb = vh + key0 * D;
  const int64_t lim = Tk - 1 - key0;
  const int last = lim < PYR_BLOCK - 1 ? (int)lim : PYR_BLOCK - 1;
#pragma unroll
  for (int tt = 0; tt < TG::CPR / NW; ++tt) {
    const int t = tt * NW + w;
    const int p = t * 64 + l, row = p / TG::CPR, sc = p % TG::CPR;
    const int rr = row < last ? row : last;
    const uint32_t ko = (uint32_t)(rr * D + (sc ^ TG::swz_k(row)) * 8) * 2;
    const uint32_t vo = (uint32_t)(rr * D + (sc ^ TG::swz_v(row)) * 8) * 2;
    lds_dma16(kb, TG::TILE, ko, (lds_dma_void*)(ktile + t * 1024));
    lds_dma16(vb, TG::TILE, vo, (lds_dma_void*)(vtile + t * 1024));
  }
}

template <int D, int NW, int RT>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_prefill_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ sel, bf16_t* __restrict__ o, float* __restrict__ lse, PyrGeom g,
    int wg_per_unit) {
  using TG = TileGeom<D>;
  constexpr int NT = NW * 64;
  // one 8-wave workgroup per CU keeps three tile stages in flight; smaller
  // workgroups share a CU and keep two
  constexpr int NSTAGE = NW >= 8 ? 3 : 2;
  constexpr int NLOAD = 2 * (TG::CPR / NW);  // tile-load instructions per block per wave
  constexpr int WAIT_ONE = 0x0F70 | (NLOAD & 15) | ((NLOAD >> 4) << 14);  // vmcnt(NLOAD)
  __shared__ __align__(16) unsigned char tiles[NSTAGE][2][TG::TILE];  // [stage][K, V]
  __shared__ int s_sel[kMaxSel];
  __shared__ int s_n;
  // the raw route row, in the last stage's V tile (free until its first load)
  static_assert(kMaxSel * 4 <= TG::TILE, "route row fits a tile");
  int* s_raw = reinterpret_cast<int*>(tiles[NSTAGE - 1][1]);

  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
  const int half = l / 32, lr = l % 32;
  // RT row tiles of 32 per wave: a wave covers rows [rsub, rsub + 32*RT) of one head
  constexpr int WPH = 2 / RT;  // waves per head
  const int sub = (int)(blockIdx.x % wg_per_unit);
  int bi, hk, i;
  int64_t unit;
  unit_of(g, blockIdx.x / wg_per_unit, bi, hk, i, unit);
  const PyrSeq sq = pyr_seq(g, bi);
  if (i >= sq.nqb) return;  // past the end of a shorter packed sequence
  const int h = hk * g.G + sub * (NW / WPH) + w / WPH;
  const int rsub = (w % WPH) * 32;
  const float sl2 = g.scale * PYR_LOG2E;
  const int64_t row0 = (int64_t)i * PYR_BLOCK + rsub;  // first query token of this wave
  const bf16_t* kh = k + (sq.k0 + hk * sq.khs) * D;
  const bf16_t* vh = v + (sq.k0 + hk * sq.khs) * D;

  for (int jj = tid; jj <= g.K; jj += NT) s_raw[jj] = sel[unit * (g.K + 1) + jj];

  __syncthreads();  // s_raw visible
  if (w == 0) {     // compact the route row: entries outside [0, nb) and repeats are skipped
    const int n = route_compact_wave(s_raw, g.K + 1, sq.nb, s_sel, 0, [](int) { return true; });
    if (l == 0) s_n = n;
  }
  __syncthreads();
  const int nsel = s_n;
#pragma unroll
  for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
    if (s0 < nsel) issue_tiles<D, NW>(kh, vh, sq.Tk, s_sel[s0], tiles[s0][0], tiles[s0][1], w, l);

  // Q^T fragments (B operand): lane holds query row rt*32 + lr and d = ks*16 + 8*half .. +7.
  // Rows past the end of a ragged last block load the last row instead; they are never stored.
  const bf16_t* qh = q + (sq.q0 + h * sq.qhs) * D;
  uint4 qb[RT][D / 16];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t tok = min<int64_t>(row0 + rt * 32 + lr, sq.Tq - 1);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qb[rt][ks] = ld16(qh + tok * D + ks * 16 + 8 * half);
  }

  f32x16 oacc[D / 32][RT];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][rt][e] = 0.f;
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
  }

  // per-lane LDS offsets that do not depend on the block
  const int g16 = l / 16, s16 = l % 16;
  int vrow[2][2];   // [kt][k2] first V row this lane addresses for the transposed reads
  int vcol[D / 32]; // byte offset of the lane's 8-byte V chunk per 32-dim tile (row-dependent swizzle applied below)
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) vrow[kt][k2] = kt * 32 + 16 * k2 + 4 * half + s16 / 4;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) vcol[dt] = dt * 32 + (g16 % 2) * 16 + 4 * (s16 % 4);

  int st = 0;
  for (int jj = 0; jj < nsel; ++jj) {
    const int j = s_sel[jj];
    // this wave's loads of block jj have landed once at most the loads of the
    // blocks issued after it are outstanding (loads complete in order)
    if (NSTAGE > 2 && jj + 1 < nsel)
      __builtin_amdgcn_s_waitcnt(WAIT_ONE);
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();  // every wave's loads of block jj landed; the oldest stage is free
    const int nx = jj + NSTAGE - 1;
    const int nst = st + NSTAGE - 1 >= NSTAGE ? st - 1 : st + NSTAGE - 1;
    if (nx < nsel) issue_tiles<D, NW>(kh, vh, sq.Tk, s_sel[nx], tiles[nst][0], tiles[nst][1], w, l);
    const unsigned char* Kt = tiles[st][0];
    const unsigned char* Vt = tiles[st][1];
    const int64_t key0 = (int64_t)j * PYR_BLOCK;

    // Two halves of 32 keys: S^T = K Q^T for the half, online softmax, then
    // O^T += V^T P^T for the half (keeps only one half's scores live).
    const bool need_mask = key0 + PYR_BLOCK - 1 > row0;  // only the diagonal (or later) block
    // (row0 here is the wave's first row; rows of the wave run to row0 + 32*RT - 1)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 sacc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[rt][e] = 0.f;
      const int krow = kt * 32 + lr;
      const unsigned char* kbase = Kt + krow * TG::ROW;
      const int kswz = TG::swz_k(krow);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(kbase + (((2 * ks + half) ^ kswz) << 4)));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sacc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(qb[rt][ks]), sacc[rt], 0, 0, 0);
      }

      // online softmax per query row (lane's row = rt*32 + lr), log2 domain
      bf16x8 pb[RT][2];  // [rt][k2] P^T fragments
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (need_mask) {
          // key position minus row position, in the block's local coordinates
          const int rel = (int)(row0 - key0) + rt * 32 + lr;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (kt * 32 + (e / 4) * 8 + half * 4 + (e % 4) > rel) sacc[rt][e] = -INFINITY;
        }
        float mraw = sacc[rt][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mraw = fmaxf(mraw, sacc[rt][e]);
        mraw = fmaxf(mraw, __shfl_xor(mraw, 32, 64));
        const float mx = mraw * sl2;
        const bool need = mx > m_run[rt] + kRescaleLog2;
        if (__any(need)) {
          const float m_new = need ? mx : m_run[rt];
          const float alpha = m_new == m_run[rt] ? 1.f : __builtin_amdgcn_exp2f(m_run[rt] - m_new);
          l_run[rt] *= alpha;
          m_run[rt] = m_new;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[dt][rt][e] *= alpha;
        }
        // a row that has seen no visible key yet keeps m_run = -inf: all its p are 0
        const float mneg = m_run[rt] == -INFINITY ? 0.f : -m_run[rt];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[rt][e], sl2, mneg));
          sacc[rt][e] = p;
          psum += p;
        }
        l_run[rt] += psum;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[rt][k2][e] = (__bf16)sacc[rt][k2 * 8 + e];
      }

      // O^T += V^T P^T.  MFMA k index 8*half + jj maps to key
      // kt*32 + 16*k2 + 4*half + jj (jj < 4) or + 8 + (jj - 4) (jj >= 4), the
      // order in which the S^T accumulator holds P.
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int r1 = vrow[kt][k2];
        const unsigned char* vbase = Vt + r1 * TG::ROW;
        const int vswz = TG::swz_v(r1);  // row + 8 has the same swizzle
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int c = vcol[dt];
          const int off1 = (((c >> 3) ^ vswz) << 4) + (c & 7) * 2;
          const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + off1));
          const s16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbase + off1 + 8 * TG::ROW));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            oacc[dt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[rt][k2], oacc[dt][rt], 0, 0, 0);
        }
      }
    }
    st = st + 1 == NSTAGE ? 0 : st + 1;
  }

  // finalize: rows of this lane = rt*32 + lr; dims of oacc[dt][rt][e] =
  // dt*32 + (e/4)*8 + half*4 + e%4
  bf16_t* oh = o + (sq.q0 + h * sq.qhs) * D;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lt = l_run[rt] + __shfl_xor(l_run[rt], 32, 64);
    const int64_t tok = row0 + rt * 32 + lr;
    if (tok >= sq.Tq) continue;
    const float inv = 1.f / lt;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = dt * 32 + g4 * 8 + half * 4;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(oacc[dt][rt][g4 * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(oh + tok * D + d0) = pk;
      }
    if (lse && half == 0) lse[sq.q0 + h * sq.qhs + tok] = (m_run[rt] + log2f(lt)) * PYR_LN2;
  }
}
// ---------------------------------------------------------------------------
// Helpers of the 8-wave bf16 prefill kernel: fragment offsets, tile loads,
// the row maximum of a 32-key half and the exponentials of P^T.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4v lds_u32x4;

// Per-lane LDS byte offsets of the MFMA fragments in a tile.  A row's swizzle
// repeats every 4 rows (V) and within 32 rows (K), so the two 32-key halves and
// the 16-key groups of a half differ by constant offsets.
template <int D>
struct FragOffsets {
  // K fragment of step ks: row lr, 16-byte chunk 2*ks + half, stored at chunk
  // (2*ks + half) ^ swz = 2*ks ^ (swz ^ half): byte offset krow + (32*ks ^ kx)
  int krow, kx;
  int v[D / 32];  // V^T fragment of dim tile dt: keys 4*half + l%16/4 (and + 8)
  // transposed V tiles (VT, see attn_vt_build): row d = dt*32 + lr of the tile
  // holds chunk c at c ^ vsw(d), vsw(d) = (d / 2) % 8 = (lr / 2) % 8; the lane's
  // fragment chunk is 4*kt + 2*k2 + half, read at that ^ vsw: (4*kt + 2*k2) ^ vx
  int vt[D / 32], vx;
  __device__ FragOffsets(int l) {
    using TG = TileGeom<D>;
    const int half = l / 32, lr = l % 32, g16 = l / 16, s16 = l % 16;
    krow = lr * TG::ROW;
    kx = (TG::swz_k(lr) ^ half) << 4;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) vt[dt] = (dt * 32 + lr) * kVtRow;
    vx = half ^ ((lr / 2) % 8);
    const int r1 = 4 * half + s16 / 4;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int c = dt * 32 + (g16 % 2) * 16 + 4 * (s16 % 4);
      v[dt] = r1 * TG::ROW + (((c >> 3) ^ TG::swz_v(r1)) << 4) + (c & 7) * 2;
    }
  }
};

// Tile loads of block j for the 8-wave kernel (same layout as issue_tiles):
// the block's first row is a uniform base and each lane adds a 32-bit
// offset, clamped to the last row of the sequence.  VT: vh is the (batch, KV
// head)'s transposed V (attn_vt_build), block j's tile the 64*D elements at
// vh + j*64*D, D rows of 128 bytes stored with chunk q of row r at q ^ ((r/2) % 8).
template <int D, bool VT = false>
__device__ __forceinline__ void tile_loads8(const bf16_t* kh, const bf16_t* vh, int64_t Tk, int j,
                                          int w, int l, unsigned char* ktile,
                                          unsigned char* vtile) {
  using TG = TileGeom<D>;
  // j is uniform; taking it from lane 0 keeps the tile bases in scalar registers
  const int64_t key0 = (int64_t)__builtin_amdgcn_readfirstlane(j) * PYR_BLOCK;
  const bf16_t* kb = kh + key0 * D;
  const bf16_t* vb = vh + key0 * D;
  const int64_t lim = Tk - 1 - key0;
  const int last = lim < PYR_BLOCK - 1 ? (int)lim : PYR_BLOCK - 1;
#pragma unroll
  for (int tt = 0; tt < TG::CPR / 8; ++tt) {
    const int t = tt * 8 + w;
    const int p = t * 64 + l, row = p / TG::CPR, sc = p % TG::CPR;
    const int rr = row < last ? row : last;
    const uint32_t ko = (uint32_t)(rr * D + (sc ^ TG::swz_k(row)) * 8) * 2;
    uint32_t vo;
    if constexpr (VT) {
      const int vr = p / 8, vq = p % 8;
      vo = (uint32_t)(vr * PYR_BLOCK + (vq ^ ((vr / 2) % 8)) * 8) * 2;
    } else {
      vo = (uint32_t)(rr * D + (sc ^ TG::swz_v(row)) * 8) * 2;
    }
    // buffer form of the LDS DMA: LDS reads of the other slots keep
    // per-read waits while these loads are in flight
    lds_dma16(kb, TG::TILE, ko, (lds_dma_void*)(ktile + t * 1024));
    lds_dma16(vb, TG::TILE, vo, (lds_dma_void*)(vtile + t * 1024));
  }
}

// Exponential of score e (of the lane's 16) of the current half, in place,
// with its share of the row sum and, for odd e, the packed bf16 pair of P^T.
// Empty asm uses keep each result in the slot that computes it (IR passes
// would otherwise sink the work past the sequence, to its first real use).
__device__ __forceinline__ void exp_pair(int e, f32x16& sc, float sl2, float mneg, float& ps0,
                                        float& ps1, uint32_t (&pw)[8]) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const float p = __builtin_amdgcn_exp2f(fmaf(sc[e], sl2, mneg));
  sc[e] = p;
  if (e & 1) {
    ps1 += p;
    const bf16x2_t pr = {(__bf16)sc[e - 1], (__bf16)p};
    pw[e / 2] = __builtin_bit_cast(uint32_t, pr);
    asm volatile("" ::"v"(pw[e / 2]), "v"(ps1));
  } else {
    ps0 += p;
    asm volatile("" ::"v"(ps0));
  }
}

// P^T fragment k2 (keys 16*k2 .. of the half) from the packed pairs.
__device__ __forceinline__ bf16x8 p_frag(const uint32_t (&pw)[8], int k2) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t x = {pw[4 * k2], pw[4 * k2 + 1], pw[4 * k2 + 2], pw[4 * k2 + 3]};
  return __builtin_bit_cast(bf16x8, x);
}

// Maximum of a lane's row over the 32 keys of a half, both lane halves; the
// mask drops keys past the row (key index within the block > rel).
template <bool MASK>
__device__ __forceinline__ float half_rowmax(f32x16& s, int kt, int half, int rel) {
  if (MASK) {
    // score e holds key kt*32 + (e/4)*8 + half*4 + e%4; compare its constant
    // part against the lane's bound so no per-score index stays live
    const int r2 = rel - kt * 32 - half * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((e / 4) * 8 + (e % 4) > r2) s[e] = -INFINITY;
  }
  float m = s[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) m = fmaxf(m, s[e]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---------------------------------------------------------------------------
// bf16 prefill, MFMA, 8 waves in two groups taking turns (ping-pong)
//
// Same tiles, fragments and MFMA shapes as attn_prefill_mfma (32 query rows
// per wave, S^T = K Q^T, O^T += V^T P^T), eight waves (four heads x two row
// halves), and each wave alternates two kinds of phase: a matrix phase (the
// S^T MFMAs of the next block and the PV MFMAs of the current one, with their
// LDS fragment reads) and a vector phase (row maximum, rescale,
// exponentials, bf16 packing of P^T).  Waves 0-3 run one phase ahead of
// waves 4-7, and wave w shares its SIMD with wave w+4, so in every phase each
// SIMD has one wave on the matrix core and one on the vector ALU: the two
// units overlap across waves, which they do better than inside one wave's
// instruction stream.  A barrier ends every phase.  Block y sits in tile slot
// y % 4 and is loaded four phases before its first use, when the slot's
// previous block is done.
// ---------------------------------------------------------------------------

// Matrix phase: S^T of a whole block (two 32-key M tiles, DO_S) from Kn and
// O^T += V^T P^T of a whole block (DO_PV) from Vx and p.  The MFMAs alternate
// between the two products and their LDS fragments are read kPpPF ahead.
#ifndef PYR_PP_PF
#define PYR_PP_PF 6
#endif
constexpr int kPpPF = PYR_PP_PF;

template <int D, bool DO_S, bool DO_PV>
struct PpSlot {
  static constexpr int NS = DO_S ? 2 * (D / 16) : 0;  // (half kt, step ks)
  static constexpr int NP = DO_PV ? 2 * (D / 16) : 0;  // (half kt, key group k2, dim tile dt)
  static constexpr int NM = NS + NP;
  __device__ static constexpr bool is_s(int t) { return DO_S && (!DO_PV || t % 2 == 0); }
  __device__ static constexpr int idx(int t) { return DO_S && DO_PV ? t / 2 : t; }
};

template <int D, bool DO_S, bool DO_PV, bool VT>
__device__ __forceinline__ bf16x8 pp_frag(int t, const lds_u8* Kn, const lds_u8* Vx,
                                          const FragOffsets<D>& fo) {
  using TG = TileGeom<D>;
  using SL = PpSlot<D, DO_S, DO_PV>;
  constexpr int HALF = 32 * TG::ROW;
  if (SL::is_s(t)) {
    const int u = SL::idx(t), kt = u % 2, ks = u / 2;
    const u32x4v x =
        *reinterpret_cast<const lds_u32x4*>(Kn + kt * HALF + fo.krow + ((32 * ks) ^ fo.kx));
    return __builtin_bit_cast(bf16x8, x);
  }
  const int u = SL::idx(t), kt = u / (D / 16), k2 = (u / (D / 32)) % 2, dt = u % (D / 32);
  if constexpr (VT) {  // one 16-byte read: the tile's keys are in the fragment's order
    const u32x4v x =
        *reinterpret_cast<const lds_u32x4*>(Vx + fo.vt[dt] + (((kt * 4 + 2 * k2) ^ fo.vx) << 4));
    return __builtin_bit_cast(bf16x8, x);
  }
  const lds_u8* p = Vx + kt * HALF + fo.v[dt] + 16 * k2 * TG::ROW;
  const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * TG::ROW));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D, bool DO_S, bool DO_PV, bool VT = false>
__device__ __forceinline__ void pp_matrix(const lds_u8* Kn, const lds_u8* Vx,
                                          const FragOffsets<D>& fo, const uint4 (&qb)[D / 16],
                                          f32x16 (&s)[2], const uint32_t (&p)[2][8],
                                          f32x16 (&oacc)[D / 32]) {
  using SL = PpSlot<D, DO_S, DO_PV>;
  constexpr int NM = SL::NM;
  FragOffsets<D> fl = fo;
  asm volatile("" : "+v"(fl.kx));
  if constexpr (DO_S) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
  }
  bf16x8 fr[NM];
#pragma unroll
  for (int t = 0; t < kPpPF && t < NM; ++t) fr[t] = pp_frag<D, DO_S, DO_PV, VT>(t, Kn, Vx, fl);
#pragma unroll
  for (int t = 0; t < NM; ++t) {
    if (t + kPpPF < NM) fr[t + kPpPF] = pp_frag<D, DO_S, DO_PV, VT>(t + kPpPF, Kn, Vx, fl);
    if (SL::is_s(t)) {
      const int u = SL::idx(t), kt = u % 2, ks = u / 2;
      s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[t], as_bf16x8(qb[ks]), s[kt], 0, 0, 0);
    } else {
      const int u = SL::idx(t), kt = u / (D / 16), k2 = (u / (D / 32)) % 2, dt = u % (D / 32);
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[t], p_frag(p[kt], k2), oacc[dt],
                                                         0, 0, 0);
    }
    // keep the order: the reads of fragment t + kPpPF go out before MFMA t
    __builtin_amdgcn_sched_barrier(0);
  }
}


// Vector phase: the block's scores in s -> P^T in p (packed bf16 pairs), with
// the running max, the rescale of O and l, and the row sum.
template <int D, bool MASK>
__device__ __forceinline__ void pp_vector(f32x16 (&s)[2], uint32_t (&p)[2][8],
                                          f32x16 (&oacc)[D / 32], float sl2, int half, int rel,
                                          float& m_run, float& l_run) {
  const float mraw =
      fmaxf(half_rowmax<MASK>(s[0], 0, half, rel), half_rowmax<MASK>(s[1], 1, half, rel));
  const float mx = mraw * sl2;
  const float m_new = mx > m_run + kRescaleLog2 ? mx : m_run;
  // a row that has seen no visible key yet keeps m = -inf: all its p are 0
  const float mneg = m_new == -INFINITY ? 0.f : -m_new;
  if (__any(m_new != m_run)) {
    const float alpha = m_new == m_run ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
  }
  m_run = m_new;
  // each exponential keeps its slot next to its fma, sum and conversion
  // (measured faster than leaving the order to the compiler)
  float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int e = 0; e < 16; ++e) exp_pair(e, s[kt], sl2, mneg, ps0, ps1, p[kt]);
  l_run += ps0 + ps1;
}

// Inputs of the ping-pong kernel's block loop (VT: vh is the transposed V).
template <int D, bool VT = false>
struct PpRun {
  const bf16_t* kh;
  const bf16_t* vh;
  const int* ord;
  int64_t Tk, row0;
  int nsel, w, l, grp;
  float sl2;
};

// Tile slots of the ping-pong kernel: block y in K slot y % 4 and V slot
// y % 4, each slot an LDS array of its own.  Inside the main loop every slot
// is named at compile time, so the compiler can tell the slots being read
// from the slots still loading and does not wait for those loads (with one
// array, or a slot chosen at run time, every LDS read waits for every tile
// load in flight, which undoes the prefetch).
constexpr int kPpSlots = 4;
constexpr int kPpTile = 64 * 2 * 128;  // bytes of a K or V tile at d = 128
__shared__ __align__(16) unsigned char pp_k0[kPpTile], pp_k1[kPpTile], pp_k2[kPpTile],
    pp_k3[kPpTile];
__shared__ __align__(16) unsigned char pp_v0[kPpTile], pp_v1[kPpTile], pp_v2[kPpTile],
    pp_v3[kPpTile];

template <int S>
__device__ __forceinline__ unsigned char* pp_kslot() {
  if constexpr (S == 0) return pp_k0;
  else if constexpr (S == 1) return pp_k1;
  else if constexpr (S == 2) return pp_k2;
  else return pp_k3;
}
template <int S>
__device__ __forceinline__ unsigned char* pp_vslot() {
  if constexpr (S == 0) return pp_v0;
  else if constexpr (S == 1) return pp_v1;
  else if constexpr (S == 2) return pp_v2;
  else return pp_v3;
}
// Slot S, or (S < 0) slot y % 4 chosen at run time.
template <int S>
__device__ __forceinline__ unsigned char* pp_k(int y) {
  if constexpr (S >= 0) return pp_kslot<S>();
  const int m = y % kPpSlots;
  return m == 0 ? pp_k0 : m == 1 ? pp_k1 : m == 2 ? pp_k2 : pp_k3;
}
template <int S>
__device__ __forceinline__ unsigned char* pp_v(int y) {
  if constexpr (S >= 0) return pp_vslot<S>();
  const int m = y % kPpSlots;
  return m == 0 ? pp_v0 : m == 1 ? pp_v1 : m == 2 ? pp_v2 : pp_v3;
}

// This wave's share of the loads of block y (if it exists) into slot S.
template <int D, int S, bool VT>
__device__ __forceinline__ void pp_issue(const PpRun<D, VT>& r, int y) {
  if (y < r.nsel)
    tile_loads8<D, VT>(r.kh, r.vh, r.Tk, r.ord[y], r.w, r.l, pp_k<S>(y), pp_v<S>(y));
}

// Wait for this wave's loads of block y: the loads of block y+1 (issued after
// them) may stay in flight.
template <int D, bool VT>
__device__ __forceinline__ void pp_wait(const PpRun<D, VT>& r, int y) {
  using TG = TileGeom<D>;
  constexpr int NLOAD = 2 * (TG::CPR / 8);  // tile-load instructions per block per wave
  if (y + 1 < r.nsel)
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NLOAD & 15) | ((NLOAD >> 4) << 14));
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Block x of a wave: the vector phase of block x, then the matrix phase with
// PV(x) and (DO_S) S(x+1).  The barrier before each phase ends a global
// phase; at the start of an even global phase 2x+2 the loads of block x+3 go
// out, and at the end of the odd one before it block x+1 must have landed.
// For group 0 the vector phase is the odd global phase 2x+1, for group 1 the
// even one 2x+2.
// J: the slot of block x (x % 4) when known at compile time, else -1.
template <int D, bool MASK, bool DO_S, int J, bool VT>
__device__ __forceinline__ void pp_block(const PpRun<D, VT>& r, int x, const FragOffsets<D>& fo,
                                         const uint4 (&qb)[D / 16], f32x16 (&s)[2],
                                         uint32_t (&p)[2][8], f32x16 (&oacc)[D / 32],
                                         float& m_run, float& l_run) {
  constexpr int JN = J < 0 ? -1 : (J + 1) % kPpSlots;  // slot of block x+1
  constexpr int JL = J < 0 ? -1 : (J + 3) % kPpSlots;  // slot of block x+3
  const int half = r.l / 32, lr = r.l % 32;
  if (r.grp) pp_wait(r, x + 1);
  lds_barrier();
  if (r.grp) pp_issue<D, JL>(r, x + 3);
  const int rel = MASK ? (int)(r.row0 - (int64_t)r.ord[x] * PYR_BLOCK) + lr : 0;
  pp_vector<D, MASK>(s, p, oacc, r.sl2, half, rel, m_run, l_run);
  if (!r.grp) pp_wait(r, x + 1);
  lds_barrier();
  if (!r.grp) pp_issue<D, JL>(r, x + 3);
  pp_matrix<D, DO_S, true, VT>((lds_u8*)pp_k<JN>(x + 1), (lds_u8*)pp_v<J>(x), fo, qb, s, p, oacc);
}

// Attention of one unit's four query heads sub*4 .. sub*4+3 of KV head hk by
// the eight waves of the workgroup.  s_sel holds the unit's route row (K+1
// entries, visible to every thread); s_ord and s_cnt are LDS scratch.  Must be
// called by every thread.  VT (dense batches): v is the transposed V of
// attn_vt_build instead of V.
template <int D, bool VT = false>
__device__ __forceinline__ void pp_unit(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                        const bf16_t* __restrict__ v, bf16_t* __restrict__ o,
                                        float* __restrict__ lse, const PyrGeom& g, int bi, int hk,
                                        int i, int sub, const PyrSeq& sq, const int* s_sel,
                                        int* s_ord, int* s_cnt) {
  using TG = TileGeom<D>;
  static_assert(TG::TILE <= kPpTile, "tile slots are sized for d <= 128");
  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int half = l / 32, lr = l % 32;
  // waves 2h and 2h+1 take the two 32-row halves of head sub*4 + h; waves
  // 0-3 form group 0, waves 4-7 group 1
  const int h = hk * g.G + sub * 4 + w / 2;
  const int grp = w >> 2;
  const int64_t row0 = (int64_t)i * PYR_BLOCK + (w % 2) * 32;
  const float sl2 = g.scale * PYR_LOG2E;

  // Q^T fragments (B operand): lane holds query row lr and d = ks*16 + 8*half .. +7.
  // Rows past the end of a ragged last block load the last row; they are never stored.
  // Issued first, so that they are in flight while the route is ordered.
  const bf16_t* qh = q + (sq.q0 + h * sq.qhs) * D;
  uint4 qb[D / 16];
  {
    const int64_t tok = min<int64_t>(row0 + lr, sq.Tq - 1);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qb[ks] = ld16(qh + tok * D + ks * 16 + 8 * half);
  }

  // route order: valid blocks before the unit's own block first (no mask
  // needed), then the rest (the diagonal block)
  // (entries outside [0, nb) and repeats of an earlier entry are skipped)
  if (w == 0) {
    const uint32_t used = route_used_mask(s_sel, g.K + 1, sq.nb);
    const int nun = route_compact_used(s_sel, g.K + 1, used, s_ord, 0,
                                       [i](int j) { return j < i; });
    const int n = route_compact_used(s_sel, g.K + 1, used, s_ord, nun,
                                     [i](int j) { return j >= i; });
    if (l == 0) {
      s_cnt[0] = n;
      s_cnt[1] = nun;
    }
  }
  lds_barrier();  // the order is in LDS; the Q loads stay in flight
  const int nsel = s_cnt[0], nun = s_cnt[1];
  const bf16_t* kh = k + (sq.k0 + hk * sq.khs) * D;
  const bf16_t* vh = VT ? v + ((int64_t)bi * g.Hk + hk) * g.nb * PYR_BLOCK * D
                        : v + (sq.k0 + hk * sq.khs) * D;

  const FragOffsets<D> fo(l);
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 s[2];
  uint32_t p[2][8];

  if (nsel > 0) {
    PpRun<D, VT> r;
    r.kh = kh;
    r.vh = vh;
    r.ord = s_ord;
    r.Tk = sq.Tk;
    r.row0 = row0;
    r.nsel = nsel;
    r.w = w;
    r.l = l;
    r.grp = grp;
    r.sl2 = sl2;
    pp_issue<D, 0>(r, 0);
    pp_issue<D, 1>(r, 1);
    // block 0 has landed once at most block 1's loads are outstanding
    pp_wait(r, 0);
    lds_barrier();
    // global phase 0 starts: block 2 loads; group 1 sits it out
    pp_issue<D, 2>(r, 2);
    if (grp) lds_barrier();
    pp_matrix<D, true, false, VT>((lds_u8*)pp_k0, (lds_u8*)pp_v0, fo, qb, s, p, oacc);  // S(0)
    // blocks before the last that need no mask, four at a time with every
    // slot named at compile time; then the others (masked blocks go last)
    const int last = nsel - 1;
    const int nu = nun < last ? nun : last;
    int x = 0;
#pragma unroll 1
    for (; x + 3 < nu; x += 4) {
      pp_block<D, false, true, 0>(r, x, fo, qb, s, p, oacc, m_run, l_run);
      pp_block<D, false, true, 1>(r, x + 1, fo, qb, s, p, oacc, m_run, l_run);
      pp_block<D, false, true, 2>(r, x + 2, fo, qb, s, p, oacc, m_run, l_run);
      pp_block<D, false, true, 3>(r, x + 3, fo, qb, s, p, oacc, m_run, l_run);
    }
#pragma unroll 1
    for (; x < nu; ++x) pp_block<D, false, true, -1>(r, x, fo, qb, s, p, oacc, m_run, l_run);
#pragma unroll 1
    for (; x < last; ++x) pp_block<D, true, true, -1>(r, x, fo, qb, s, p, oacc, m_run, l_run);
    if (last < nun)
      pp_block<D, false, false, -1>(r, last, fo, qb, s, p, oacc, m_run, l_run);
    else
      pp_block<D, true, false, -1>(r, last, fo, qb, s, p, oacc, m_run, l_run);
    lds_barrier();
    if (!grp) lds_barrier();  // group 0 sits out the last global phase
  }

  // finalize: row of this lane = lr; dims of oacc[dt][e] = dt*32 + (e/4)*8 + half*4 + e%4
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                  false, false);
  const float lt = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const int64_t tok = row0 + lr;
  if (tok >= sq.Tq) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  bf16_t* orow = o + (sq.q0 + h * sq.qhs + tok) * D;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(oacc[dt][g4 * 4 + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + dt * 32 + g4 * 8 + half * 4) = pk;
    }
  if (lse && half == 0)
    lse[sq.q0 + h * sq.qhs + tok] = lt > 0.f ? (m_run + log2f(lt)) * PYR_LN2 : -INFINITY;
}

template <int D, bool VT>
__global__ __launch_bounds__(512, 2) void attn_prefill_pp(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ sel, bf16_t* __restrict__ o, float* __restrict__ lse, PyrGeom g,
    int wg_per_unit) {
  __shared__ int s_sel[kMaxSel];
  __shared__ int s_ord[kMaxSel];
  __shared__ int s_cnt[2];
  const int sub = (int)(blockIdx.x % wg_per_unit);
  int bi, hk, i;
  int64_t unit;
  unit_of(g, blockIdx.x / wg_per_unit, bi, hk, i, unit);
  const PyrSeq sq = pyr_seq(g, bi);
  if (i >= sq.nqb) return;  // past the end of a shorter packed sequence
  for (int jj = threadIdx.x; jj <= g.K; jj += 512) s_sel[jj] = sel[unit * (g.K + 1) + jj];
  __syncthreads();
  pp_unit<D, VT>(q, k, v, o, lse, g, bi, hk, i, sub, sq, s_sel, s_ord, s_cnt);
}

// ---------------------------------------------------------------------------
// Fused selection and attention (bf16 prefill, four query heads per KV head):
// one workgroup of eight waves per unit finds the unit's route on the matrix
// cores (eight waves of two 16-row M tiles) and then attends over it with the
// ping-pong schedule, in one launch.  The selection's LDS lives in the
// attention's tile slots, free until the first tile load: its layout in V
// slot 0, its two candidate stages in K slots 0 and 1.  The route reaches the
// attention through LDS; it is also written to sel.  Units go in the
// attention's heavy-first order, which deals one (batch, KV head) slab to
// each XCD when there are eight of them, so an XCD's L2 holds one pyramid.
// ---------------------------------------------------------------------------
constexpr int kFusedWaves = 8;

template <int D>
__global__ __launch_bounds__(512, 2) void select_attend(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ pyr, int32_t* __restrict__ sel, int32_t* __restrict__ trace_ids,
    float* __restrict__ trace_scores, bf16_t* __restrict__ o, float* __restrict__ lse, PyrGeom g) {
  static_assert(kSelStages * kChunk * 4 * D <= 2 * kPpTile, "a candidate stage fits a K slot");
  __shared__ int s_sel[kMaxSel];
  __shared__ int s_ord[kMaxSel];
  __shared__ int s_cnt[2];
  int bi, hk, i;
  int64_t unit;
  unit_of(g, blockIdx.x, bi, hk, i, unit);
  select_mfma_unit<D, 2, kFusedWaves>(q, pyr, sel, trace_ids, trace_scores, g, unit, pp_v0, pp_k0,
                                      pp_k1);
  const PyrSeq sq = pyr_seq(g, bi);
  if (i >= sq.nqb) return;  // past the end of a shorter packed sequence (route blanked)
  // the route row, as the selection wrote it: kept blocks, the diagonal, -1
  const SelLayout lay(g.K, g.branching, D, true, kFusedWaves);
  const int* kept = reinterpret_cast<const int*>(pp_v0 + lay.off_kept);
  const int nk = reinterpret_cast<const int*>(pp_v0 + lay.off_misc)[PYR_MAX_LEVELS];
  for (int j = threadIdx.x; j <= g.K; j += 512) s_sel[j] = j < nk ? kept[j] : (j == nk ? i : -1);
  __syncthreads();
  pp_unit<D>(q, k, v, o, lse, g, bi, hk, i, 0, sq, s_sel, s_ord, s_cnt);
}

// ---------------------------------------------------------------------------
// fp32 prefill, MFMA (v_mfma_f32_32x32x2_f32)
//
// The layout of the bf16 kernels with fp32 tiles and fp32 products: S^T = K Q^T
// with keys on the M side and the lane's query row on N, and O^T += V^T P^T.
// One MFMA step covers two head dims (S^T) or two keys (O^T), one per lane
// half.  Step ks of S^T takes dim 8(ks/4) + 4*half + ks%4 in lane half `half`,
// so a lane reads the K values of four consecutive steps as one 16-byte chunk
// and holds the matching Q values in registers.  Step ks of O^T over a 32-key
// tile takes key 8(ks/4) + 4*half + ks%4 of the tile: exactly the key whose
// score element ks of the lane's S^T accumulator holds, so P^T feeds the MFMA
// as its B operand straight from registers, with no exchange between lanes.
// ---------------------------------------------------------------------------
template <int D>
struct TileGeomF32 {
  static constexpr int CPR = D / 4;      // 16-byte chunks per row
  static constexpr int ROW = 4 * D;      // bytes per row (a multiple of 256)
  static constexpr int TILE = 64 * ROW;  // bytes per K or V tile
  // K: the 16 lanes that read one chunk index from 16 consecutive rows find it
  // at 16 different positions (mod 16) of the row, i.e. in 16 distinct 4-bank groups
  __device__ static int swz_k(int r) { return r % 16; }
  // V: a lane half reads 32 consecutive floats of one key row (8 chunks) and
  // the other half those of a key 4 rows on; flipping chunk bit 3 every 4 rows
  // puts the two halves on different banks
  __device__ static int swz_v(int r) { return 8 * ((r / 4) % 2); }
};

// Issue the K and V tiles of block j: instruction t of a tile fills LDS chunks
// [64t, 64t+64); chunk p holds row p / CPR, logical chunk (p % CPR) ^ swz(row).
// Rows past the sequence end re-read its last row (the causal mask gives them
// zero weight).
template <int D, int NW>
__device__ __forceinline__ void issue_tiles_f32(const float* kh, const float* vh, int64_t Tk, int j,
                                                unsigned char* ktile, unsigned char* vtile, int w,
                                                int l) {
  using TG = TileGeomF32<D>;
  const int64_t key0 = (int64_t)__builtin_amdgcn_readfirstlane(j) * PYR_BLOCK;
  const float* kb = kh + key0 * D;
  const float* vb = vh + key0 * D;
  const int64_t lim = Tk - 1 - key0;
  const int last = lim < PYR_BLOCK - 1 ? (int)lim : PYR_BLOCK - 1;
#pragma unroll
  for (int tt = 0; tt < TG::CPR / NW; ++tt) {
    const int t = tt * NW + w;
    const int p = t * 64 + l, row = p / TG::CPR, sc = p % TG::CPR;
    const int rr = row < last ? row : last;
    const uint32_t ko = (uint32_t)(rr * D + (sc ^ TG::swz_k(row)) * 4) * 4;
    const uint32_t vo = (uint32_t)(rr * D + (sc ^ TG::swz_v(row)) * 4) * 4;
    lds_dma16(kb, TG::TILE, ko, (lds_dma_void*)(ktile + t * 1024));
    lds_dma16(vb, TG::TILE, vo, (lds_dma_void*)(vtile + t * 1024));
  }
}

// Per-wave state of the fp32 kernel: 32 query rows of one head.
template <int D>
struct F32Wave {
  float4 qf[D / 8];     // Q: row lr, dims 8c + 4*half .. +3
  f32x16 oacc[D / 32];  // O^T: dim dt*32 + (e/4)*8 + half*4 + e%4, row lr
  float m_run, l_run;   // running max (log2 domain) and the lane half's sum
  int64_t row0;         // first query position of the wave
  int kfrag[2];         // byte offset of the lane's K row in a tile, per 32-key tile
  int kswz;             // its swizzle (the same for both 32-key tiles)
  int voff[D / 32];     // byte offset of the lane's V value, key 4*half, per dim tile
};

// One selected block (key block j, tiles in rd): loads of the next selected
// block (jn >= 0) go to wr first.  rd and wr are distinct __shared__ arrays,
// so the compiler does not wait for those loads before reading rd.
template <int D, int NW>
__device__ __forceinline__ void f32_block(F32Wave<D>& s_, const unsigned char* rd, int j,
                                          unsigned char* wr, int jn, const float* kh,
                                          const float* vh, int64_t Tk, float sl2, int w, int l) {
  using TG = TileGeomF32<D>;
  const int half = l / 32, lr = l % 32;
  if (jn >= 0) issue_tiles_f32<D, NW>(kh, vh, Tk, jn, wr, wr + TG::TILE, w, l);
  const unsigned char* Kt = rd;
  const unsigned char* Vt = rd + TG::TILE;
  const int64_t key0 = (int64_t)j * PYR_BLOCK;
  f32x16 s[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
    for (int c4 = 0; c4 < D / 32; ++c4) {
      float4 a[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        a[c] = *reinterpret_cast<const float4*>(Kt + s_.kfrag[kt] +
                                                (((2 * (4 * c4 + c) + half) ^ s_.kswz) << 4));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 qv = s_.qf[4 * c4 + c];
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[c].x, qv.x, s[kt], 0, 0, 0);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[c].y, qv.y, s[kt], 0, 0, 0);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[c].z, qv.z, s[kt], 0, 0, 0);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[c].w, qv.w, s[kt], 0, 0, 0);
      }
      // keep the compiler from hoisting all reads of the block (register pressure)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // element e of tile kt is key kt*32 + (e/4)*8 + half*4 + e%4 of the block
  if (key0 + PYR_BLOCK - 1 > s_.row0) {  // the diagonal block (or a later one)
    const int rel = (int)(s_.row0 - key0) + lr;  // the lane row's position in the block
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (kt * 32 + (e / 4) * 8 + half * 4 + (e % 4) > rel) s[kt][e] = -INFINITY;
  }
  float mraw = fmaxf(s[0][0], s[1][0]);
#pragma unroll
  for (int e = 1; e < 16; ++e) mraw = fmaxf(mraw, fmaxf(s[0][e], s[1][e]));
  mraw = fmaxf(mraw, __shfl_xor(mraw, 32, 64));
  const float mx = mraw * sl2;
  const bool need = mx > s_.m_run + kRescaleLog2;
  if (__any(need)) {
    const float m_new = need ? mx : s_.m_run;
    const float alpha = m_new == s_.m_run ? 1.f : __builtin_amdgcn_exp2f(s_.m_run - m_new);
    s_.l_run *= alpha;
    s_.m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s_.oacc[dt][e] *= alpha;
  }
  // a row that has seen no visible key yet keeps m_run = -inf: all its p are 0
  const float mneg = s_.m_run == -INFINITY ? 0.f : -s_.m_run;
  float psum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][e], sl2, mneg));
      s[kt][e] = p;
      psum += p;
    }
  s_.l_run += psum;
  // O^T += V^T P^T: step ks of tile kt takes key kt*32 + 8(ks/4) + 4*half + ks%4
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      float a[4][D / 32];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          a[c][dt] = *reinterpret_cast<const float*>(Vt + (kt * 32 + 8 * k4 + c) * TG::ROW +
                                                     s_.voff[dt]);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          s_.oacc[dt] =
              __builtin_amdgcn_mfma_f32_32x32x2f32(a[c][dt], s[kt][4 * k4 + c], s_.oacc[dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_prefill_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ sel, float* __restrict__ o, float* __restrict__ lse, PyrGeom g,
    int wg_per_unit) {
  using TG = TileGeomF32<D>;
  constexpr int NT = NW * 64;
  // two stages [K tile, V tile], separate arrays used in a fixed rotation
  __shared__ __align__(16) unsigned char st0[2 * TG::TILE];
  __shared__ __align__(16) unsigned char st1[2 * TG::TILE];
  __shared__ int s_sel[kMaxSel];
  __shared__ int s_n;
  // the raw route row, in the second stage (free until the second block's loads)
  static_assert(kMaxSel * 4 <= TG::TILE, "route row fits a tile");
  int* s_raw = reinterpret_cast<int*>(st1);

  const int tid = threadIdx.x, w = tid / 64, l = tid % 64;
  const int half = l / 32, lr = l % 32;
  const int sub = (int)(blockIdx.x % wg_per_unit);
  int bi, hk, i;
  int64_t unit;
  unit_of(g, blockIdx.x / wg_per_unit, bi, hk, i, unit);
  const PyrSeq sq = pyr_seq(g, bi);
  if (i >= sq.nqb) return;  // past the end of a shorter packed sequence
  const int h = hk * g.G + sub * (NW / 2) + w / 2;  // two waves of 32 rows per head
  const float sl2 = g.scale * PYR_LOG2E;
  const float* kh = k + (sq.k0 + hk * sq.khs) * D;
  const float* vh = v + (sq.k0 + hk * sq.khs) * D;

  for (int jj = tid; jj <= g.K; jj += NT) s_raw[jj] = sel[unit * (g.K + 1) + jj];
  __syncthreads();  // s_raw visible
  if (w == 0) {     // compact the route row: entries outside [0, nb) and repeats are skipped
    const int n = route_compact_wave(s_raw, g.K + 1, sq.nb, s_sel, 0, [](int) { return true; });
    if (l == 0) s_n = n;
  }
  __syncthreads();
  const int nsel = s_n;
  if (nsel > 0) issue_tiles_f32<D, NW>(kh, vh, sq.Tk, s_sel[0], st0, st0 + TG::TILE, w, l);

  F32Wave<D> s_;
  s_.row0 = (int64_t)i * PYR_BLOCK + (w % 2) * 32;
  {
    // rows past the end of a ragged last block load the last row; they are never stored
    const float* qh = q + (sq.q0 + h * sq.qhs) * D;
    const int64_t tok = min<int64_t>(s_.row0 + lr, sq.Tq - 1);
#pragma unroll
    for (int c = 0; c < D / 8; ++c)
      s_.qf[c] = *reinterpret_cast<const float4*>(qh + tok * D + 8 * c + 4 * half);
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) s_.oacc[dt][e] = 0.f;
  s_.m_run = -INFINITY;
  s_.l_run = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) s_.kfrag[kt] = (kt * 32 + lr) * TG::ROW;
  s_.kswz = TG::swz_k(lr);  // rows lr and 32 + lr share it
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
    s_.voff[dt] = 4 * half * TG::ROW + (((dt * 8 + lr / 4) ^ TG::swz_v(4 * half)) << 4) +
                  (lr % 4) * 4;  // keys 8a + 4*half + c share swz_v(4*half)

  // block jj's tiles are in st0 (jj even) or st1 (jj odd)
  for (int jj = 0; jj < nsel; jj += 2) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block jj landed
    __syncthreads();                     // everyone's; the stage of block jj - 1 is free
    f32_block<D, NW>(s_, st0, s_sel[jj], st1, jj + 1 < nsel ? s_sel[jj + 1] : -1, kh, vh, sq.Tk,
                     sl2, w, l);
    if (jj + 1 < nsel) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      f32_block<D, NW>(s_, st1, s_sel[jj + 1], st0, jj + 2 < nsel ? s_sel[jj + 2] : -1, kh, vh,
                       sq.Tk, sl2, w, l);
    }
  }

  // finalize: the lane's row is row0 + lr; O^T element e of dim tile dt is dim
  // dt*32 + (e/4)*8 + half*4 + e%4
  const float lt = s_.l_run + __shfl_xor(s_.l_run, 32, 64);
  const int64_t tok = s_.row0 + lr;
  if (tok >= sq.Tq) return;
  float* orow = o + (sq.q0 + h * sq.qhs + tok) * D;
  const float inv = 1.f / lt;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float4 y;
      y.x = s_.oacc[dt][g4 * 4 + 0] * inv;
      y.y = s_.oacc[dt][g4 * 4 + 1] * inv;
      y.z = s_.oacc[dt][g4 * 4 + 2] * inv;
      y.w = s_.oacc[dt][g4 * 4 + 3] * inv;
      *reinterpret_cast<float4*>(orow + dt * 32 + g4 * 8 + half * 4) = y;
    }
  if (lse && half == 0) lse[sq.q0 + h * sq.qhs + tok] = (s_.m_run + log2f(lt)) * PYR_LN2;
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
  const T* kh = k + ((int64_t)bi * g.Hk + hk) * g.Tks * D;
  const T* vh = v + ((int64_t)bi * g.Hk + hk) * g.Tks * D;

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
  // entries outside [0, nb) and repeats of an earlier entry of the row are skipped
  int jj = jb0;
  while (jj < jb1 && !route_entry_used(srow, jj, srow[jj], g.nb)) ++jj;
  if (jj < jb1) fetch(srow[jj]);
  while (jj < jb1) {
    const int j = srow[jj];
    int nx = jj + 1;
    while (nx < jb1 && !route_entry_used(srow, nx, srow[nx], g.nb)) ++nx;
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

// ---------------------------------------------------------------------------
// Decode, bf16, on the matrix cores.  One workgroup (4 waves) per (unit,
// split); the workgroup walks the split's blocks one at a time and wave w
// takes keys [16w, 16w+16) of every block, keeping its own online softmax
// over them (the four partial states are merged at the end).  Per block and
// wave: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 keys x 16 query rows, the
// G real rows padded with zero rows), the K fragments loaded straight from
// global memory into registers; then O^T += V^T P^T on
// v_mfma_f32_16x16x16_bf16, the V tile staged in LDS by direct loads and its
// transposed fragments read with ds_read_b64_tr_b16, and P^T taken as is
// from the S^T accumulator layout.  Every byte of K and V is read from HBM
// once and from LDS at most once; the next block's K and V load while the
// current one is used.
// ---------------------------------------------------------------------------
typedef short s16x4v __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256, 4) void attn_decode_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ sel, float* __restrict__ ws, PyrGeom g, int nsplit) {
  using TG = TileGeom<D>;
  constexpr int KS = D / 32;       // k-steps of the S^T MFMA
  constexpr int DT = D / 16;       // d tiles of O^T
  constexpr int TL = TG::CPR / 4;  // V-tile load instructions per wave
  // two V slots, one array each, so that the LDS reads of one slot do not
  // wait for the loads into the other
  __shared__ __align__(16) unsigned char vt0[TG::TILE];
  __shared__ __align__(16) unsigned char vt1[TG::TILE];
  __shared__ float s_m[4][16], s_l[4][16];
  __shared__ int s_blk[kDecBlocksPerSplit];
  __shared__ int s_nb;

  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lr = l % 16, lg = l / 16;
  const int split = (int)(blockIdx.x % nsplit);
  const int64_t bhk = blockIdx.x / nsplit;  // unit (decode: one query block)
  const int bi = (int)(bhk / g.Hk), hk = (int)(bhk % g.Hk);
  const int G = g.G;
  const float sl2 = g.scale * PYR_LOG2E;
  const int64_t qpos = g.Tk - 1;
  const bf16_t* kh = k + ((int64_t)bi * g.Hk + hk) * g.Tks * D;
  const bf16_t* vh = v + ((int64_t)bi * g.Hk + hk) * g.Tks * D;

  // Q^T B fragments: lane holds query row lr (zero past G), d = 32*ks + 8*lg .. +7
  uint4 qb[KS];
  {
    const bf16_t* qrow = q + ((int64_t)bi * g.Hq + (int64_t)hk * G + (lr < G ? lr : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = lr < G ? ld16(qrow + ks * 32 + 8 * lg) : make_uint4(0u, 0u, 0u, 0u);
  }
  // this split's blocks: its entries of the route row that are used (block
  // ids in [0, nb) that no earlier entry of the whole row repeats)
  const int jb0 = split * kDecBlocksPerSplit;
  const int jb1 = min(g.K + 1, jb0 + kDecBlocksPerSplit);
  // the row's entries up to this split's last, in V slot 1 (free until block 1 loads)
  static_assert(kMaxSel * 4 <= TG::TILE, "route row fits a tile");
  int* s_row = reinterpret_cast<int*>(vt1);
  for (int jj = tid; jj < jb1; jj += 256) s_row[jj] = sel[bhk * (g.K + 1) + jj];
  __syncthreads();
  if (w == 0) {
    const int jj = jb0 + l;
    const bool ok = l < kDecBlocksPerSplit && jj < jb1 && route_entry_used(s_row, jj, s_row[jj], g.nb);
    const unsigned long long m = __ballot(ok);
    if (ok) s_blk[__popcll(m & ((1ull << l) - 1ull))] = s_row[jj];
    if (l == 0) s_nb = __popcll(m);
  }
  __syncthreads();
  const int nblk = s_nb;

  // loads of block b: this wave's K fragments into registers (key 16w + lr,
  // d = 32*ks + 8*lg), and a quarter of the V tile into vt (rows past the
  // sequence repeat its last row; the mask gives them no weight)
  auto load = [&](int b, uint4 (&kr)[KS], unsigned char* vt) {
    const int64_t key0 = (int64_t)__builtin_amdgcn_readfirstlane(s_blk[b]) * PYR_BLOCK;
    const int64_t lim = g.Tk - 1 - key0;
    const int last = lim < PYR_BLOCK - 1 ? (int)lim : PYR_BLOCK - 1;
    const int kk = 16 * w + lr;
    const bf16_t* krow = kh + (key0 + (kk < last ? kk : last)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kr[ks] = ld16_nt(krow + ks * 32 + 8 * lg);
    const bf16_t* vb = vh + key0 * D;
#pragma unroll
    for (int tt = 0; tt < TL; ++tt) {
      const int t = tt * 4 + w;
      const int p = t * 64 + l, row = p / TG::CPR, sc = p % TG::CPR;
      const int rr = row < last ? row : last;
      const uint32_t vo = (uint32_t)(rr * D + (sc ^ TG::swz_v(row)) * 8) * 2;
      lds_dma16(vb, TG::TILE, vo, (lds_dma_void*)(vt + t * 1024));
    }
  };
  // per-lane byte offset of the V^T fragment of d tile dt: row 16w + 4*lg +
  // lr / 4, columns 16*dt + 4*(lr % 4) .. +3 (the transposed read hands lane
  // lr of group lg the values V[16w + 4*lg + i][16*dt + lr], i = 0..3: the A
  // operand of the 16x16x16 MFMA)
  int voff[DT];
  {
    const int r = 16 * w + 4 * lg + lr / 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int c = 16 * dt + 4 * (lr % 4);
      voff[dt] = r * TG::ROW + (((c >> 3) ^ TG::swz_v(r)) << 4) + (c & 7) * 2;
    }
  }

  f32x4 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // block b from kc and vc; block b+1 starts loading into kn and vn
  auto step = [&](int b, const uint4 (&kc)[KS], uint4 (&kn)[KS], const unsigned char* vc,
                  unsigned char* vn) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block b
    lds_barrier();  // every wave's part of V(b) has landed; block b-1's slot is free
    if (b + 1 < nblk) load(b + 1, kn, vn);
    // S^T for this wave's 16 keys: lane column lr (query row), rows 4*lg + e (keys)
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[ks]), as_bf16x8(qb[ks]), s, 0, 0, 0);
    const int64_t kp0 = (int64_t)s_blk[b] * PYR_BLOCK + 16 * w + 4 * lg;
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (kp0 + e > qpos) s[e] = -INFINITY;
      mx = fmaxf(mx, s[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float mneg = m_new == -INFINITY ? 0.f : -m_new;
    const float alpha = m_run == m_new ? 1.f : __builtin_amdgcn_exp2f(m_run + mneg);
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t pb;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[e], sl2, mneg));
      ps += p;
      pb[e] = (__bf16)p;
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    const s16x4v pf = __builtin_bit_cast(s16x4v, pb);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const s16x4 vf =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((const lds_u8*)vc + voff[dt]));
      oacc[dt] *= alpha;
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4v, vf), pf,
                                                           oacc[dt], 0, 0, 0);
    }
  };
  uint4 k0[KS], k1[KS];
  if (nblk > 0) load(0, k0, vt0);
#pragma unroll 1
  for (int b = 0; b < nblk; b += 2) {
    step(b, k0, k1, vt0, vt1);
    if (b + 1 < nblk) step(b + 1, k1, k0, vt1, vt0);
  }

  // merge the four waves' states: lane holds row lr, d = 16*dt + 4*lg + e.
  // Row r's value of dim d sits at r*D + (d ^ dec_swz(r)): a row is a whole
  // number of 64-bank sweeps, so without the XOR the 16 rows of a store would
  // hit one bank; with it the 64 lanes of every store meet 64 distinct banks
  // (bits 0-1 of the column take r % 4, bits 4-5 take r / 4), and the merge's
  // reads of 64 consecutive dims of a row stay a permutation of 64 banks.
  auto dec_swz = [](int r) { return (r & 3) | ((r >> 2) << 4); };
  __syncthreads();  // the V slots are free: waves 0-1 park their sums in vt0, 2-3 in vt1
  float* s_o = reinterpret_cast<float*>(w < 2 ? vt0 : vt1) + (w % 2) * 16 * D;
  if (lg == 0) {
    s_m[w][lr] = m_run;
    s_l[w][lr] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[lr * D + ((16 * dt + 4 * lg + e) ^ dec_swz(lr))] = oacc[dt][e];
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int r = idx / D, d = idx % D;
    float m = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) m = fmaxf(m, s_m[ww][r]);
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[ww][r] - m);
      const float* so = reinterpret_cast<const float*>(ww < 2 ? vt0 : vt1) + (ww % 2) * 16 * D;
      lsum += a * s_l[ww][r];
      acc += a * so[r * D + (d ^ dec_swz(r))];
    }
    float* dst = ws + (((int64_t)bhk * G + r) * nsplit + split) * (D + 2);
    if (d == 0) {
      dst[0] = m;
      dst[1] = lsum;
    }
    dst[2 + d] = acc;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_decode_combine(const float* __restrict__ ws,
                                                          T* __restrict__ o,
                                                          float* __restrict__ lse, PyrGeom g,
                                                          int nsplit) {
  constexpr int DPL = D / 64;
  constexpr int U = 16;  // splits whose loads are in flight together
  const int64_t row = blockIdx.x;  // (bhk * G + r)
  const int l = threadIdx.x;
  const float* src = ws + row * nsplit * (D + 2);
  // the largest split maximum, then every split's sum and output weighted by
  // 2^(its maximum - that); loads of U splits are issued before their use
  // (indices past the last split are clamped to it, their values masked)
  float m = -INFINITY;
  for (int sp0 = 0; sp0 < nsplit; sp0 += U) {
    float mm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = sp0 + u < nsplit ? sp0 + u : nsplit - 1;
      mm[u] = src[sp * (D + 2)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) m = sp0 + u < nsplit ? fmaxf(m, mm[u]) : m;
  }
  float s = 0.f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  for (int sp0 = 0; sp0 < nsplit; sp0 += U) {
    float mm[U], ss[U], xx[U][DPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = sp0 + u < nsplit ? sp0 + u : nsplit - 1;
      mm[u] = src[sp * (D + 2)];
      ss[u] = src[sp * (D + 2) + 1];
#pragma unroll
      for (int e = 0; e < DPL; ++e) xx[u][e] = src[sp * (D + 2) + 2 + l * DPL + e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // an empty split (maximum -inf) adds nothing; so does every split of a
      // row with no visible key
      const float a = sp0 + u < nsplit && mm[u] != -INFINITY ? exp2f(mm[u] - m) : 0.f;
      s += ss[u] * a;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += xx[u][e] * a;
    }
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

// Block-transposed copy of V for attn_prefill_pp<D, true>: block j of
// (batch, KV head) bh becomes 64*D elements at vt + (bh*nb + j)*64*D, D rows
// of its 64 keys, so that a V^T fragment of the PV product (8 keys of one
// dim) is one 16-byte LDS read instead of two transposed 8-byte reads.
// Within every 16 keys the order is 0-3, 8-11, 4-7, 12-15: the order in which
// the fragment's two lane halves take the keys of P^T from the S^T
// accumulator.  Keys past the sequence end are zero (the causal mask gives
// them no weight).  Dense batches; one workgroup per block, grid-strided.
template <int D>
__global__ __launch_bounds__(256) void attn_vt_build(const bf16_t* __restrict__ v,
                                                bf16_t* __restrict__ vt, PyrGeom g) {
  __shared__ __align__(16) bf16_t tile[PYR_BLOCK][D + 8];
  const int64_t nblk = (int64_t)g.B * g.Hk * g.nb;
  for (int64_t x = blockIdx.x; x < nblk; x += gridDim.x) {
    const int64_t bh = x / g.nb;
    const int j = (int)(x % g.nb);
    const bf16_t* vb = v + (bh * g.Tks + (int64_t)j * PYR_BLOCK) * D;
    for (int idx = threadIdx.x; idx < PYR_BLOCK * D / 8; idx += 256) {
      const int r = idx / (D / 8), c = idx % (D / 8);
      const uint4 val = (int64_t)j * PYR_BLOCK + r < g.Tk ? ld16(vb + r * D + c * 8)
                                                          : make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&tile[r][c * 8]) = val;
    }
    __syncthreads();
    bf16_t* out = vt + x * PYR_BLOCK * D;
    for (int idx = threadIdx.x; idx < D * 8; idx += 256) {
      const int d = idx / 8, c8 = idx % 8;  // 16 bytes: positions 8*c8 .. +7 of row d
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint32_t pair = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int pos = c8 * 8 + e + h, p16 = pos % 16;
          const int key = pos - p16 + (p16 < 4 || p16 >= 12 ? p16 : (p16 < 8 ? p16 + 4 : p16 - 4));
          pair |= (uint32_t)tile[key][d] << (16 * h);
        }
        w[e / 2] = pair;
      }
      *reinterpret_cast<uint4*>(out + d * PYR_BLOCK + c8 * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __syncthreads();  // the tile is read before the next block overwrites it
  }
}

template <int D>
hipError_t launch_attn_d(const PyrGeom& g, int dtype, const void* q, const void* k,
                         const void* v, const int32_t* sel, void* o, float* lse, void* ws,
                         size_t ws_bytes, hipStream_t st) {
  const int64_t units = (int64_t)g.B * g.Hk * g.nqb;
  if (units == 0 || g.Tq == 0) return hipSuccess;
  if (g.decode) {
    const int ns = decode_splits(g.K);
    float* wsf = static_cast<float*>(ws);
    if (dtype == 1) {
      hipLaunchKernelGGL((attn_decode_mfma<D>), dim3((unsigned)(units * ns)), dim3(256), 0, st,
                         static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                         static_cast<const bf16_t*>(v), sel, wsf, g, ns);
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
    // heads per workgroup: 4, 2 or 1 (whichever divides G); 32 query rows per wave,
    // two waves per head
    const int nh = g.G % 4 == 0 ? 4 : (g.G % 2 == 0 ? 2 : 1);
    const int wpu = g.G / nh;
    const dim3 grid((unsigned)(units * wpu));
    const bf16_t* qq = static_cast<const bf16_t*>(q);
    const bf16_t* kk = static_cast<const bf16_t*>(k);
    const bf16_t* vv = static_cast<const bf16_t*>(v);
    bf16_t* oo = static_cast<bf16_t*>(o);
    const size_t vtb = pyr_attn_vt_bytes(g, dtype);
    if (nh == 4 && vtb > 0 && ws && ws_bytes >= vtb) {
      // V read through its block-transposed copy in the workspace
      bf16_t* vt = static_cast<bf16_t*>(ws);
      const int64_t nblk = (int64_t)g.B * g.Hk * g.nb;
      hipLaunchKernelGGL((attn_vt_build<D>), dim3((unsigned)(nblk < (1 << 20) ? nblk : (1 << 20))),
                         dim3(256), 0, st, vv, vt, g);
      hipLaunchKernelGGL((attn_prefill_pp<D, true>), grid, dim3(512), 0, st, qq, kk, vt, sel, oo, lse, g,
                         wpu);
    } else if (nh == 4)
      hipLaunchKernelGGL((attn_prefill_pp<D, false>), grid, dim3(512), 0, st, qq, kk, vv, sel, oo, lse, g,
                         wpu);
    else if (nh == 2)
      hipLaunchKernelGGL((attn_prefill_mfma<D, 4, 1>), grid, dim3(256), 0, st, qq, kk, vv, sel, oo, lse, g, wpu);
    else
      hipLaunchKernelGGL((attn_prefill_mfma<D, 2, 1>), grid, dim3(128), 0, st, qq, kk, vv, sel, oo, lse, g, wpu);
  } else {
    // two waves of 32 rows per head; at d = 128 the Q values, O accumulators
    // and scores of a wave need more than the 256 registers of two waves per
    // SIMD, so workgroups take at most two heads (four waves, one per SIMD)
    const int nh = D == 64 && g.G % 4 == 0 ? 4 : (g.G % 2 == 0 ? 2 : 1);
    const int wpu = g.G / nh;
    const dim3 grid((unsigned)(units * wpu));
    const float* qq = static_cast<const float*>(q);
    const float* kk = static_cast<const float*>(k);
    const float* vv = static_cast<const float*>(v);
    float* oo = static_cast<float*>(o);
    if (nh == 4)
      hipLaunchKernelGGL((attn_prefill_f32<D, D == 64 ? 8 : 4>), grid, dim3(D == 64 ? 512 : 256), 0, st,
                         qq, kk, vv, sel, oo, lse, g, wpu);
    else if (nh == 2)
      hipLaunchKernelGGL((attn_prefill_f32<D, 4>), grid, dim3(256), 0, st, qq, kk, vv, sel, oo, lse, g, wpu);
    else
      hipLaunchKernelGGL((attn_prefill_f32<D, 2>), grid, dim3(128), 0, st, qq, kk, vv, sel, oo, lse, g, wpu);
  }
  return hipGetLastError();
}

}  // namespace

bool pyr_select_attend_fused(const PyrGeom& g, int dtype) {
  return dtype == 1 && !g.decode && g.G == 4 && g.K + 1 <= kMaxSel &&
         SelLayout(g.K, g.branching, g.D, true, kFusedWaves).total <= kPpTile;
}

hipError_t pyr_launch_select_attend(const PyrGeom& g, int dtype, const void* q, const void* k,
                                    const void* v, const float* pyr, int32_t* sel,
                                    int32_t* trace_ids, float* trace_scores, void* o, float* lse,
                                    void* ws, size_t ws_bytes, hipStream_t st) {
  if (!pyr_select_attend_fused(g, dtype)) {
    const hipError_t e = pyr_launch_select(g, dtype, q, pyr, sel, trace_ids, trace_scores, st);
    if (e != hipSuccess) return e;
    return pyr_launch_attn(g, dtype, q, k, v, sel, o, lse, ws, ws_bytes, st);
  }
  const int64_t units = (int64_t)g.B * g.Hk * g.nqb;
  if (units == 0 || g.Tq == 0) return hipSuccess;
  const bf16_t* qq = static_cast<const bf16_t*>(q);
  const bf16_t* kk = static_cast<const bf16_t*>(k);
  const bf16_t* vv = static_cast<const bf16_t*>(v);
  bf16_t* oo = static_cast<bf16_t*>(o);
  if (g.D == 64)
    hipLaunchKernelGGL((select_attend<64>), dim3((unsigned)units), dim3(512), 0, st, qq, kk, vv,
                       pyr, sel, trace_ids, trace_scores, oo, lse, g);
  else
    hipLaunchKernelGGL((select_attend<128>), dim3((unsigned)units), dim3(512), 0, st, qq, kk, vv,
                       pyr, sel, trace_ids, trace_scores, oo, lse, g);
  return hipGetLastError();
}

// The transposed copy costs one HBM round trip of V and saves one LDS read
// per V^T fragment each time a workgroup attends a block: it pays when every
// tile of V is attended by enough workgroups, (K + 1) route slots x G/4
// workgroups per unit.  Measured on MI355X at d = 128 and 128K keys, the copy
// included: 9 visits (G = 4, K = 8) 1.9% slower, 17 and 18 visits 1% faster,
// 25 and 33 visits 1.8% faster; at 130 visits (G = 8, K = 64, 1M keys) 2-4%.
constexpr int kVtMinVisits = 16;

size_t pyr_attn_vt_bytes(const PyrGeom& g, int dtype) {
  if (dtype != 1 || g.decode || g.cu || g.G % 4 != 0) return 0;
  if ((int64_t)(g.K + 1) * (g.G / 4) < kVtMinVisits) return 0;
  return (size_t)g.B * g.Hk * g.nb * PYR_BLOCK * g.D * sizeof(bf16_t);
}

size_t pyr_attn_ws_bytes(const PyrGeom& g) {
  if (!g.decode) return 0;
  return (size_t)g.B * g.Hk * g.G * decode_splits(g.K) * (g.D + 2) * sizeof(float);
}

hipError_t pyr_launch_attn(const PyrGeom& g, int dtype, const void* q, const void* k,
                           const void* v, const int32_t* sel, void* o, float* lse, void* ws,
                           size_t ws_bytes, hipStream_t st) {
  return g.D == 64 ? launch_attn_d<64>(g, dtype, q, k, v, sel, o, lse, ws, ws_bytes, st)
                   : launch_attn_d<128>(g, dtype, q, k, v, sel, o, lse, ws, ws_bytes, st);
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free attention entry point
// (pyr_block_sparse_attn_noalloc): the decode partial states live in this
// fixed device array instead of a caller's workspace.  Every GPU the library
// runs on holds its own copy until the process ends; host code reaches a
// device's copy only through the address hipGetSymbolAddress returns for it
// (the array's name is a host-side stand-in, not a device address).
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[PYR_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, resolved on first use

// Device address of `scratch` on the device that runs stream st (the current
// device for the null stream), looked up once per device with that device
// current.
hipError_t scratch_of(hipStream_t st, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (st) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(st, &d);
    if (e != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t pyr_launch_attn_noalloc(const PyrGeom& g, int dtype, const void* q, const void* k,
                                   const void* v, const int32_t* sel, void* o, float* lse,
                                   hipStream_t st) {
  void* ws = nullptr;
  if (pyr_attn_ws_bytes(g) > 0) {
    const hipError_t e = scratch_of(st, &ws);
    if (e != hipSuccess) return e;
  }
  return pyr_launch_attn(g, dtype, q, k, v, sel, o, lse, ws, 0, st);  // (no transposed V)
}
