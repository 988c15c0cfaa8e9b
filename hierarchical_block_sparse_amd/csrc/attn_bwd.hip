// Backward of the block-sparse causal attention for a fixed route table, on
// gfx950.
//
// PHBA (Prefix-State Hybrid Block Attention) §A.1 and §A.1.4 describe the
// sparse backward; here it takes this form.  The key gradients walk, for each
// key block, the list of query blocks whose routes contain it, built from a
// per-slab bitmap with one bit per (key block, query block) pair.  P is
// rebuilt in registers from the stored log-sum-exp of every row, so no
// probability tensor ever reaches memory.  The route itself is a discrete
// choice and gets no gradient.  With P = exp(scale q k^T -
// lse) over the visible keys of the selected blocks:
//   dP = dO v^T,  D = rowsum(dO * O),  dS = P (dP - D),
//   dQ = scale dS k,  dK = scale dS^T q,  dV = P^T dO   (dK, dV summed over
//   the G query heads of the KV group).
//
// Kernels (bf16 tensors, fp32 accumulation):
//  * bwd_dsum: a record per (query head, query block) of the rows' log-sum-exp
//    (log2 domain) and D.
//  * bwd_route_clear + bwd_route_bits: the block-major route metadata, a bitmap
//    per (batch, KV head) slab with one row per key block and bit i of row j
//    set when query block i routes to key block j.  OR-ing bits does not depend
//    on the order of the writes, so the metadata, the order in which a key
//    block visits its query blocks, and the gradients are deterministic.
//  * bwd_dq: one workgroup per (unit, group of heads), 32 query rows per wave,
//    Q and dO of its rows held as MFMA B fragments in VGPRs.  For every
//    selected block the K and V tiles stream global -> LDS (direct loads, two
//    stages); S^T = K Q^T and dP^T = V dO^T read row fragments of the tiles,
//    and dQ^T += K^T dS^T reads K^T fragments with transposed LDS reads.
//  * bwd_dkdv: one workgroup per (slab, key block), four waves: wave w takes
//    the 32 keys (w & 1) of the block against the 32 query rows (w >> 1) of
//    each visiting (query block, head).  The wave keeps its keys' K and V as B
//    fragments in VGPRs and dK^T, dV^T accumulators, streams the Q and dO
//    tiles (and the rows' record) of each visitor, and computes S = Q K^T,
//    dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS with transposed reads
//    of the tiles.  The two row halves of a key tile are summed through LDS at
//    the end.
#include <math.h>

#include <algorithm>

#include "pyr_device.h"
#include "pyr_internal.h"

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kMaxSelB = PYR_BWD_MAX_SLOTS;  // route-row capacity staged in LDS
constexpr int kMaxItemQ = 256;               // query blocks per key-gradient work item

// A 64-row tile of bf16 rows of length D in LDS: row-major, the 16-byte chunks
// of row r XOR-swizzled by swz(r).  With u = r / RP the bank sweep of the row
// and n = CPR / 4, swz = 4 (u mod n) + (u / n) mod 4 takes every value over any
// 16 aligned rows (so a row-per-lane 16-byte read, 16 rows per pass, hits 16
// distinct 16-byte slots), and swz / 4 differs between the 4 rows of an
// aligned group (so a transposed 8-byte read, 4 rows x 2 chunk pairs per 32
// lanes, hits 8 distinct 32-byte slots): both are free of bank conflicts.
template <int D>
struct BTile {
  static constexpr int CPR = D / 8;      // 16-byte chunks per row
  static constexpr int ROW = 2 * D;      // bytes per row
  static constexpr int TILE = 64 * ROW;  // bytes per tile
  static constexpr int RP = 256 / ROW;   // rows per 256-byte bank sweep
  __device__ static int swz(int r) {
    const int u = r / RP;
    return 4 * (u % (CPR / 4)) + (u / (CPR / 4)) % 4;
  }
  // byte offset of logical 16-byte chunk c of row r
  __device__ static int off(int r, int c) { return r * ROW + ((c ^ swz(r)) << 4); }
};

// Load 64 rows (row0 .. row0 + 63, clamped to `last`) of a [rows, D] bf16
// matrix into a tile with direct 16-byte global->LDS loads.  Load t of a thread
// fills stored chunk p = t * NT + tid (a wave's 64 lanes fill 1 KiB in lane
// order): row p / CPR, stored chunk p % CPR, which holds logical chunk
// (p % CPR) ^ swz(row).
template <int D, int NT>
__device__ __forceinline__ void load_tile(const bf16_t* base, int64_t row0, int64_t last,
                                          unsigned char* tile, int w, int l) {
  using TG = BTile<D>;
  static_assert(64 * TG::CPR % NT == 0, "tile must split evenly");
  // row0 is uniform: from lane 0, so the tile base stays in scalar registers
  const int64_t r0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(row0 >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)row0));
  const int64_t rb = r0 < last ? r0 : last;
  const int lim = (int)min<int64_t>(last - rb, 63);
  const bf16_t* tb = base + rb * D;
#pragma unroll
  for (int t = 0; t < 64 * TG::CPR / NT; ++t) {
    const int p = t * NT + w * 64 + l;
    const int row = p / TG::CPR, sc = p % TG::CPR;
    const int rr = row < lim ? row : lim;
    // buffer form of the LDS DMA: the tile reads of other stages keep
    // per-read waits while these loads are in flight
    lds_dma16(tb, TG::TILE, (uint32_t)(rr * D + (sc ^ TG::swz(row)) * 8) * 2,
              (lds_dma_void*)(tile + (t * NT + w * 64) * 16));
  }
}

// A fragment of a 32x32x16 MFMA whose M index is a tile row (rows rb .. rb+31,
// lane's row rb + l%32) and whose K index is d (16 at ks*16): 8 consecutive d.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const unsigned char* tile, int rb, int ks, int l) {
  using TG = BTile<D>;
  return as_bf16x8(*reinterpret_cast<const uint4*>(tile + TG::off(rb + l % 32, 2 * ks + l / 32)));
}

// A fragment whose M index is d (32 at dt*32) and whose K index runs over 16
// tile rows starting at rb: two transposed reads.  MFMA k index 8*half + jj
// maps to tile row rb + 4*half + jj (jj < 4) or rb + 8 + 4*half + (jj - 4)
// (jj >= 4), the order in which a 32x32 C fragment holds its rows (per
// 16-lane group, lane i of a transposed read receives element i % 4 of the
// 8-byte chunk that lane 4j + i/4 addresses).
template <int D>
__device__ __forceinline__ bf16x8 trans_frag(const unsigned char* tile, int rb, int dt, int l) {
  using TG = BTile<D>;
  const int half = l / 32, g16 = l / 16, s16 = l % 16;
  const int r1 = rb + 4 * half + s16 / 4;
  const int c = dt * 32 + (g16 % 2) * 16 + 4 * (s16 % 4);  // first of the lane's 4 d
  const unsigned char* p1 = tile + TG::off(r1, c >> 3) + (c & 7) * 2;
  const unsigned char* p2 = tile + TG::off(r1 + 8, c >> 3) + (c & 7) * 2;
  const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  const s16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p2);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Pack the lane's 16 fp32 values of a 32x32 C fragment (column l%32, rows
// (e/4)*8 + half*4 + e%4) into the two bf16 B fragments (K index = those rows,
// in trans_frag's order) of the next product.
__device__ __forceinline__ void pack_b(const f32x16& x, bf16x8 (&b)[2]) {
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int e = 0; e < 8; ++e) b[k2][e] = (__bf16)x[k2 * 8 + e];
}

// Lane offsets into a tile for the reads of a wave whose rows start at a
// multiple of 16 (the swizzle repeats every 16 rows, so row shifts by 16 are
// plain additions):
//  * row reads: lane row l%32, chunk 2ks + l/32 lies at  r ^ (ks << 5);
//  * transposed reads (trans_frag's rows 4*half + (l%16)/4 and 8 further, the
//    lane's 4 d at dt*32 + (l/16 % 2)*16 + 4*(l%4)) lie at t ^ (dt << 6) and
//    t8 ^ (dt << 6).
// (XOR-ing the chunk index with 2ks or 4dt commutes with the swizzle XOR, and
// the row term has no bits in the chunk field.)
template <int D>
struct TileLanes {
  int r, t, t8;
  __device__ explicit TileLanes(int l) {
    using TG = BTile<D>;
    const int half = l / 32, s16 = l % 16, g16 = l / 16;
    r = TG::off(l % 32, half);
    const int y = (g16 % 2) * 2 + (s16 % 4) / 2;  // chunk of dt = 0
    const int b = (s16 % 2) * 8;                  // byte within the chunk
    t = TG::off(4 * half + s16 / 4, y) + b;
    t8 = TG::off(4 * half + s16 / 4 + 8, y) + b;
  }
};

// ---------------------------------------------------------------------------
// Per-row record of the backward: for every (batch, query head, query block) a
// 512-byte record of 64 log2-domain log-sum-exps (lse * log2 e) followed by 64
// values of D = rowsum(dO * O).  Rows past q_len, and rows whose log-sum-exp
// is not finite (they saw no key), get +inf and 0: their probabilities
// evaluate to exactly 0, so they contribute nothing and get zero gradients.
// ---------------------------------------------------------------------------
constexpr int kRec = 128;  // floats per record

template <int D>
__global__ __launch_bounds__(256) void bwd_dsum(const bf16_t* __restrict__ o,
                                                const bf16_t* __restrict__ dout,
                                                const float* __restrict__ lse,
                                                float* __restrict__ rec, PyrGeom g) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  const int64_t rows = (int64_t)g.B * g.Hq * g.nqb * PYR_BLOCK;  // padded rows
  const int64_t r = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 8;
  const int64_t padded = (int64_t)g.nqb * PYR_BLOCK;
  const int64_t bh = r / padded, t = r % padded;
  const bool live = r < rows && t < g.Tq;
  float s = 0.f;
  if (live) {
    const int64_t row = bh * g.Tq + t;
    const uint4 a = ld16(o + row * D + c), b = ld16(dout + row * D + c);
    float x[8], y[8];
    unpack16<bf16_t>(a, x);
    unpack16<bf16_t>(b, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(x[e], y[e], s);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (r < rows && threadIdx.x % TPR == 0) {
    float l2 = __builtin_inff(), dd = 0.f;
    if (live) {
      const float lv = lse[bh * g.Tq + t];
      if (__builtin_isfinite(lv)) {
        l2 = lv * PYR_LOG2E;
        dd = s;
      }
    }
    float* out = rec + (r / PYR_BLOCK) * kRec + r % PYR_BLOCK;
    out[0] = l2;
    out[PYR_BLOCK] = dd;
  }
}

// ---------------------------------------------------------------------------
// Block-major route metadata
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_route_clear(uint32_t* __restrict__ bits, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256)
    bits[x] = 0u;
}

__global__ __launch_bounds__(256) void bwd_route_bits(const int32_t* __restrict__ sel,
                                                      uint32_t* __restrict__ bits,
                                                      int32_t* __restrict__ cnt, PyrGeom g,
                                                      int words) {
  const int64_t n = (int64_t)g.B * g.Hk * g.nqb * (g.K + 1);
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n) return;
  const int64_t unit = x / (g.K + 1);
  const int j = sel[x];
  if (j < 0 || j >= g.nb) return;
  const int64_t slab = unit / g.nqb;
  const int i = (int)(unit % g.nqb);
  const int64_t row = slab * g.nb + j;
  const uint32_t bit = 1u << (i % 32);
  // count each (query block, key block) pair once, even if a row lists it twice
  if (!(atomicOr(bits + row * words + i / 32, bit) & bit)) atomicAdd(cnt + row, 1);
}

// Work list of the key-gradient kernel (count -> prefix sum -> scatter).  Key
// block row r with cnt[r] visiting query blocks is one item when cnt[r] <= chq
// ("light"), else ceil(cnt[r] / chq) items of chq query blocks each ("split"),
// whose fp32 partial sums go to partial slots pslot[r] .. + items - 1 and are
// added in slot order afterwards.  Split items are listed first, in row order
// (hitems, slot = position), then the light rows (litems); hdr = {number of
// split items, number of light rows}.  One workgroup scans all rows in tiles of
// 1024.
__global__ __launch_bounds__(1024) void bwd_route_plan(const int32_t* __restrict__ cnt,
                                                       int32_t* __restrict__ pslot,
                                                       int2* __restrict__ hitems,
                                                       int2* __restrict__ litems,
                                                       int32_t* __restrict__ hdr, int64_t rows,
                                                       int chq) {
  __shared__ int s_w[16][2];
  __shared__ int s_carry[2];
  const int tid = threadIdx.x, l = tid % 64, w = tid / 64;
  if (tid == 0) {
    s_carry[0] = 0;
    s_carry[1] = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < rows; base += 1024) {
    const int64_t r = base + tid;
    const int c = r < rows ? cnt[r] : 0;
    const bool split = r < rows && c > chq;
    const int hn = split ? (c + chq - 1) / chq : 0;
    const int ln = (r < rows && !split) ? 1 : 0;
    int hs = hn, ls = ln;  // inclusive scans within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int a = __shfl_up(hs, off, 64), b = __shfl_up(ls, off, 64);
      if (l >= off) {
        hs += a;
        ls += b;
      }
    }
    if (l == 63) {
      s_w[w][0] = hs;
      s_w[w][1] = ls;
    }
    __syncthreads();
    int hpre = s_carry[0] + hs - hn, lpre = s_carry[1] + ls - ln;
    for (int x = 0; x < w; ++x) {
      hpre += s_w[x][0];
      lpre += s_w[x][1];
    }
    if (split) {
      pslot[r] = hpre;
      for (int k2 = 0; k2 < hn; ++k2) hitems[hpre + k2] = make_int2((int)r, k2);
    } else if (r < rows) {
      pslot[r] = -1;
      litems[lpre] = make_int2((int)r, 0);
    }
    __syncthreads();  // s_w and s_carry are read
    if (tid == 1023) {
      s_carry[0] = hpre + hn;
      s_carry[1] = lpre + ln;
    }
    __syncthreads();
  }
  if (tid == 0) {
    hdr[0] = s_carry[0];
    hdr[1] = s_carry[1];
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (unit, group of NH heads); two waves per head.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4v lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

// Row fragment (see row_frag) read through an LDS-typed pointer, which the
// compiler does not order behind the global->LDS loads in flight.
template <int D>
__device__ __forceinline__ bf16x8 row_frag_l(const unsigned char* tile, int rb, int ks, int l) {
  using TG = BTile<D>;
  const lds_u8* p = (const lds_u8*)tile + TG::off(rb + l % 32, 2 * ks + l / 32);
  return __builtin_bit_cast(bf16x8, *(const lds_u32x4*)p);
}

// Per-wave state of the dQ kernel.
template <int D>
struct DqWave {
  uint4 qb[D / 16], ob[D / 16];  // Q^T, dO^T B fragments of the wave's 32 rows
  f32x16 acc[D / 32];            // dQ^T
  int r, t, t8;                  // TileLanes of the lane
  float lse2, dsr, sl2;
  int64_t row0;
};

// One selected block: K and V tiles in `rd` (key block starting at key0).
// First issues (if `wr`) the loads of block x+2 into `wr`: rd and wr are
// distinct __shared__ arrays, so the compiler does not wait for those loads.
template <int D, int NW>
__device__ __forceinline__ void dq_step(DqWave<D>& s_, const unsigned char* rd, int64_t key0,
                                        unsigned char* wr, int64_t key2, const bf16_t* kh,
                                        const bf16_t* vh, int64_t Tk, int w, int l) {
  using TG = BTile<D>;
  constexpr int NT = NW * 64;
  const int half = l / 32, lr = l % 32;
  if (wr) {
    load_tile<D, NT>(kh, key2, Tk - 1, wr, w, l);
    load_tile<D, NT>(vh, key2, Tk - 1, wr + TG::TILE, w, l);
  }
  __builtin_amdgcn_sched_barrier(0);
  // opaque copies of the lane offsets: the addresses are formed per step
  // instead of being kept live for all three stages
  int ro = s_.r, to = s_.t, to8 = s_.t8;
  asm volatile("" : "+v"(ro), "+v"(to), "+v"(to8));
  const lds_u8* Kt = (const lds_u8*)rd;
  const lds_u8* Vt = Kt + TG::TILE;
  // the block reaches past the wave's first row: the diagonal block (or a later one)
  const bool need_mask = key0 + PYR_BLOCK - 1 > s_.row0;
  const int rel = (int)(s_.row0 - key0) + lr;  // row position in the block's key coordinates
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    // row fragments of the K and V tiles, then S^T and dP^T, in PH phases
    // (two when two waves share a SIMD and registers are scarce)
    constexpr int PH = (D == 128 && NW == 8) ? 2 : 1;
    constexpr int KS = D / 16 / PH;
    f32x16 s, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s[e] = 0.f;
      dp[e] = 0.f;
    }
#pragma unroll
    for (int ph = 0; ph < PH; ++ph) {
      bf16x8 fk[KS], fv[KS];
#pragma unroll
      for (int x = 0; x < KS; ++x) {
        const int o = (ro ^ ((ph * KS + x) << 5)) + kt * 32 * TG::ROW;
        fk[x] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(Kt + o));
        fv[x] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(Vt + o));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int x = 0; x < KS; ++x) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[x], as_bf16x8(s_.qb[ph * KS + x]), s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[x], as_bf16x8(s_.ob[ph * KS + x]), dp, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // K^T fragments for dQ^T (independent of dS: in flight during the VALU
    // work); the second half is read after the first half's products
    auto tread = [&](int k2, int dt) {
      const int o = (kt * 32 + k2 * 16) * TG::ROW;
      const s16x4 t1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Kt + ((to ^ (dt << 6)) + o)));
      const s16x4 t2 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Kt + ((to8 ^ (dt << 6)) + o)));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 tk[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) tk[dt] = tread(0, dt);
    __builtin_amdgcn_sched_barrier(0);
    // S^T element e of the lane: key kt*32 + (e/4)*8 + half*4 + e%4, row lr
    f32x16 ds;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[e], s_.sl2, -s_.lse2));
      ds[e] = p * (dp[e] - s_.dsr);
    }
    if (need_mask) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kt * 32 + (e / 4) * 8 + half * 4 + (e % 4);
        if (key > rel) ds[e] = 0.f;
      }
    }
    bf16x8 dsb[2];
    pack_b(ds, dsb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      s_.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tk[dt], dsb[0], s_.acc[dt], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) tk[dt] = tread(1, dt);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      s_.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tk[dt], dsb[1], s_.acc[dt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ sel, const bf16_t* __restrict__ dout,
    const float* __restrict__ rec, bf16_t* __restrict__ dq, PyrGeom g, int wg_per_unit) {
  using TG = BTile<D>;
  constexpr int NT = NW * 64;
  constexpr int NH = NW / 2;  // heads per workgroup
  constexpr int PER = 2 * (64 * TG::CPR / NT);  // global->LDS loads per block per wave
  constexpr int WAIT_ONE = 0x0F70 | (PER & 15) | ((PER >> 4) << 14);  // vmcnt(PER)
  // Three stages of K and V tiles, each its own __shared__ array, used in a
  // fixed rotation (the loop is unrolled by three), so that the compiler can
  // tell the stage a step reads from the one being loaded.
  __shared__ __align__(16) unsigned char st0[2 * TG::TILE];
  __shared__ __align__(16) unsigned char st1[2 * TG::TILE];
  __shared__ __align__(16) unsigned char st2[2 * TG::TILE];
  __shared__ int s_sel[kMaxSelB + 1];
  // the raw route row, in stage 2 (free until its first tile load)
  static_assert(kMaxSelB * 4 <= 2 * TG::TILE, "route row fits a stage");
  int* s_raw = reinterpret_cast<int*>(st2);

  const int tid = threadIdx.x, l = tid % 64;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int half = l / 32, lr = l % 32;
  const int64_t ublk = blockIdx.x / wg_per_unit;
  const int sub = (int)(blockIdx.x % wg_per_unit);
  const int i = (int)(ublk % g.nqb);
  const int64_t slab = ublk / g.nqb;
  const int bi = (int)(slab / g.Hk), hk = (int)(slab % g.Hk);
  const int h = hk * g.G + sub * NH + w / 2;
  const bf16_t* kh = k + slab * g.Tk * D;
  const bf16_t* vh = v + slab * g.Tk * D;
  DqWave<D> s_;
  s_.row0 = (int64_t)i * PYR_BLOCK + (w % 2) * 32;  // first query token of the wave
  s_.sl2 = g.scale * PYR_LOG2E;
  {
    const TileLanes<D> tl(l);
    s_.r = tl.r;
    s_.t = tl.t;
    s_.t8 = tl.t8;
  }

  // compact the route row (entries outside [0, nb) and repeats of an earlier
  // entry are skipped, as the key gradients' bitmap counts a block once);
  // count in s_sel[kMaxSelB]
  for (int jj = tid; jj <= g.K; jj += NT) s_raw[jj] = sel[ublk * (g.K + 1) + jj];
  __syncthreads();
  if (w == 0) {
    const int n = route_compact_wave(s_raw, g.K + 1, g.nb, s_sel, 0, [](int) { return true; });
    if (l == 0) s_sel[kMaxSelB] = n;
  }
  __syncthreads();
  const int nsel = s_sel[kMaxSelB];
  if (nsel > 0) {
    load_tile<D, NT>(kh, (int64_t)s_sel[0] * PYR_BLOCK, g.Tk - 1, st0, w, l);
    load_tile<D, NT>(vh, (int64_t)s_sel[0] * PYR_BLOCK, g.Tk - 1, st0 + TG::TILE, w, l);
  }
  if (nsel > 1) {
    load_tile<D, NT>(kh, (int64_t)s_sel[1] * PYR_BLOCK, g.Tk - 1, st1, w, l);
    load_tile<D, NT>(vh, (int64_t)s_sel[1] * PYR_BLOCK, g.Tk - 1, st1 + TG::TILE, w, l);
  }

  // Q^T and dO^T B fragments: lane holds query row row0 + lr, d = ks*16 + 8*half .. +7;
  // rows past the end load the last row (never stored).
  const int64_t tok = min<int64_t>(s_.row0 + lr, g.Tq - 1);
  const int64_t qrow = ((int64_t)bi * g.Hq + h) * g.Tq + tok;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    s_.qb[ks] = ld16(q + qrow * D + ks * 16 + 8 * half);
    s_.ob[ks] = ld16(dout + qrow * D + ks * 16 + 8 * half);
  }
  const float* rrow = rec + (((int64_t)bi * g.Hq + h) * g.nqb + i) * kRec + (w % 2) * 32 + lr;
  s_.lse2 = rrow[0];
  s_.dsr = rrow[PYR_BLOCK];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) s_.acc[dt][e] = 0.f;

  // step x reads stage `rd` and issues block x+2 into `wr`
#define PYR_DQ_STEP(x, rd, wr)                                                                 \
  {                                                                                            \
    if ((x) + 1 < nsel)                                                                        \
      __builtin_amdgcn_s_waitcnt(WAIT_ONE); /* this wave's loads of block x are done */        \
    else                                                                                       \
      __builtin_amdgcn_s_waitcnt(0x0F70);                                                      \
    lds_barrier(); /* everyone's; the stage of block x-1 is free */                            \
    const bool more = (x) + 2 < nsel;                                                          \
    const int64_t key2 = more ? (int64_t)s_sel[(x) + 2] * PYR_BLOCK : 0;                        \
    dq_step<D, NW>(s_, rd, (int64_t)s_sel[x] * PYR_BLOCK, more ? (wr) : nullptr, key2, kh, vh, \
                   g.Tk, w, l);                                                                \
  }
  for (int x = 0; x < nsel; x += 3) {
    PYR_DQ_STEP(x, st0, st2);
    if (x + 1 < nsel) PYR_DQ_STEP(x + 1, st1, st0);
    if (x + 2 < nsel) PYR_DQ_STEP(x + 2, st2, st1);
  }
#undef PYR_DQ_STEP

  // dQ = scale * acc; lane's row = lr, dims of acc[dt][e] = dt*32 + (e/4)*8 + half*4 + e%4
  if (s_.row0 + lr >= g.Tq) return;
  bf16_t* out = dq + qrow * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4_t pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(s_.acc[dt][g4 * 4 + e] * g.scale);
      *reinterpret_cast<bf16x4_t*>(out + dt * 32 + g4 * 8 + half * 4) = pk;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (slab, key block), four waves.
// ---------------------------------------------------------------------------

// Walks the set bits of one bitmap row in ascending order.
struct BitWalk {
  const uint32_t* row;
  int words, wi;
  uint32_t cur;
  // start at the row's set bit number `skip` (0-based)
  __device__ void start(const uint32_t* r, int n, int skip) {
    row = r;
    words = n;
    wi = 0;
    cur = n > 0 ? __builtin_amdgcn_readfirstlane(r[0]) : 0u;
    while (skip > 0) {  // whole words first
      const int pc = __builtin_popcount(cur);
      if (pc > skip) break;
      skip -= pc;
      if (++wi >= words) {
        cur = 0u;
        break;
      }
      cur = __builtin_amdgcn_readfirstlane(row[wi]);
    }
    for (; skip > 0 && cur != 0u; --skip) cur &= cur - 1u;
  }
  // next query block, or -1 when none is left
  __device__ int next() {
    while (cur == 0u) {
      if (++wi >= words) return -1;
      cur = __builtin_amdgcn_readfirstlane(row[wi]);
    }
    const int b = __builtin_ctz(cur);
    cur &= cur - 1u;
    return wi * 32 + b;
  }
};

template <int D>
struct DkdvStage {
  static constexpr int TILE = BTile<D>::TILE;
  static constexpr int AUX = 512;  // the visitor's row record
  static constexpr int BYTES = 2 * TILE + AUX;
  // global->LDS loads per visitor per wave: Q and dO tiles, and one for the record
  static constexpr int PER = 2 * (64 * BTile<D>::CPR / 256) + 1;
};

// Stage the Q and dO tiles and the row record of visitor (query block i, head
// h).  The record's 32 16-byte chunks come from lanes 0..7 of each wave.
template <int D>
__device__ __forceinline__ void load_visitor(const bf16_t* q, const bf16_t* dout, const float* rec,
                                             const PyrGeom& g, int bi, int h, int i,
                                             unsigned char* st, int w, int l) {
  using TG = BTile<D>;
  const int64_t bh = (int64_t)bi * g.Hq + h;
  const int64_t r0 = (int64_t)i * PYR_BLOCK;
  load_tile<D, 256>(q + bh * g.Tq * D, r0, g.Tq - 1, st, w, l);
  load_tile<D, 256>(dout + bh * g.Tq * D, r0, g.Tq - 1, st + TG::TILE, w, l);
  if (l < 8)
    lds_dma16(rec + (bh * g.nqb + i) * kRec, kRec * 4, (uint32_t)(w * 8 + l) * 16,
              (lds_dma_void*)(st + 2 * TG::TILE + w * 128));
}

// Work-list metadata of the key-gradient kernel.
struct BwdList {
  const uint32_t* bits;  // route bitmap, `words` words per key block row
  const int32_t* cnt;    // visiting query blocks per row
  const int2* hitems;    // split items (row, chunk), slot = position
  const int2* litems;    // light rows (row, 0)
  const int32_t* hdr;    // {split items, light rows}
  float* part;           // [slot][dK, dV][64 keys][D] fp32 partial sums
  int words, chq;
};

// Per-wave state of the key-gradient kernel.
template <int D>
struct DkdvWave {
  uint4 kb[D / 16], vb[D / 16];  // K, V B fragments of the wave's 32 keys
  f32x16 dka[D / 32], dva[D / 32];  // dK^T, dV^T accumulators
  int r, t, t8;  // TileLanes of the lane (rows relative to rh*32)
  int kl, rh, half, l;  // kl: the lane's key within the block
  float sl2;
};

// Row fragments of a visitor's Q and dO rows rh*32 .. +31 in the tiles at Qt.
template <int D>
__device__ __forceinline__ void dkdv_row_frags(const lds_u8* Qt, int ro, int rh,
                                               bf16x8 (&fq)[D / 16], bf16x8 (&fo)[D / 16]) {
  using TG = BTile<D>;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int o = (ro ^ (ks << 5)) + rh * 32 * TG::ROW;
    fq[ks] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(Qt + o));
    fo[ks] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(Qt + TG::TILE + o));
  }
}

// Transposed fragments (see trans_frag) of the tile at t: rows rh*32 + 16 k2.
template <int D>
__device__ __forceinline__ bf16x8 dkdv_tread(const lds_u8* t, int to, int to8, int rh, int k2,
                                             int dt) {
  using TG = BTile<D>;
  const int o = (rh * 32 + k2 * 16) * TG::ROW;
  const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + ((to ^ (dt << 6)) + o)));
  const s16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + ((to8 ^ (dt << 6)) + o)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t1, t2, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S = Q K^T and dP = dO V^T of the first visitor (tiles in rd).
template <int D>
__device__ __forceinline__ void dkdv_first(const DkdvWave<D>& s_, const unsigned char* rd,
                                          f32x16& s, f32x16& dp) {
  bf16x8 fq[D / 16], fo[D / 16];
  dkdv_row_frags<D>((const lds_u8*)rd, s_.r, s_.rh, fq, fo);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    s[e] = 0.f;
    dp[e] = 0.f;
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[ks], as_bf16x8(s_.kb[ks]), s, 0, 0, 0);
    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fo[ks], as_bf16x8(s_.vb[ks]), dp, 0, 0, 0);
  }
}

// One pipelined step.  On entry s, dp hold S and dP of visitor n (tiles in
// rd, query block i); the tiles of visitor n+1 are in rdn.  Issues (if wr) the
// loads of visitor n+3, then computes S and dP of visitor n+1 on the matrix
// cores while the vector units form P of visitor n, then dV (with dS formed
// meanwhile) and dK of visitor n; leaves S, dP of visitor n+1 in s, dp.  rd,
// rdn and wr are distinct __shared__ arrays, so the compiler does not wait for
// the loads in flight before the step's LDS reads.  When visitor n+1 does not
// exist rdn holds stale tiles and its results are not used.
template <int D>
__device__ __forceinline__ void dkdv_pipe(DkdvWave<D>& s_, f32x16& s, f32x16& dp,
                                          const unsigned char* rd, const unsigned char* rdn,
                                          int i, int j, unsigned char* wr, int i3, int h3,
                                          const bf16_t* q, const bf16_t* dout, const float* rec,
                                          const PyrGeom& g, int bi, int w) {
  using TG = BTile<D>;
  const int l = s_.l, half = s_.half, rh = s_.rh;
  if (wr) load_visitor<D>(q, dout, rec, g, bi, h3, i3, wr, w, l);
  __builtin_amdgcn_sched_barrier(0);
  // opaque copies of the lane offsets: the addresses are formed per step
  // instead of being kept live for all four stages
  int ro = s_.r, to = s_.t, to8 = s_.t8;
  asm volatile("" : "+v"(ro), "+v"(to), "+v"(to8));
  const lds_u8* Qt = (const lds_u8*)rd;
  const lds_u8* Ot = Qt + TG::TILE;
  const lds_u8* aux = Qt + 2 * TG::TILE;
  const bool live = i >= j;  // a later key block has no visible pair
  // reads: the next visitor's row fragments, this visitor's dO^T fragments and record
  bf16x8 fq[D / 16], fo[D / 16];
  dkdv_row_frags<D>((const lds_u8*)rdn, ro, rh, fq, fo);
  bf16x8 tf[2][D / 32];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) tf[k2][dt] = dkdv_tread<D>(Ot, to, to8, rh, k2, dt);
  f32x4 ls4[4], dd4[4];
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    ls4[g4] = *(const lds_f32x4*)(aux + (rh * 32 + g4 * 8 + half * 4) * 4);
    dd4[g4] = *(const lds_f32x4*)(aux + (64 + rh * 32 + g4 * 8 + half * 4) * 4);
  }
  __builtin_amdgcn_sched_barrier(0);
  // S, dP of the next visitor on the matrix cores; P of this one meanwhile.
  // Element e of the lane: row rr(e) = rh*32 + (e/4)*8 + half*4 + e%4 of the
  // query block, key kl.
  constexpr int EPK = 16 / (D / 16);  // P elements per k step
  f32x16 s2, dp2, pf;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    s2[e] = 0.f;
    dp2[e] = 0.f;
  }
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[ks], as_bf16x8(s_.kb[ks]), s2, 0, 0, 0);
    dp2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fo[ks], as_bf16x8(s_.vb[ks]), dp2, 0, 0, 0);
#pragma unroll
    for (int e = ks * EPK; e < (ks + 1) * EPK; ++e)
      pf[e] = __builtin_amdgcn_exp2f(fmaf(s[e], s_.sl2, -ls4[e / 4][e % 4]));
  }
  // every pair is visible unless this is the diagonal block or the ragged
  // last query block; a later key block sees none
  const int64_t qpos0 = (int64_t)i * PYR_BLOCK;
  const bool full = i > j && qpos0 + PYR_BLOCK <= g.Tq;
  if (!full) {
    const int qoff = (i - j) * PYR_BLOCK;  // row position minus key position base
    const int64_t rows_left = g.Tq - qpos0;
    const int lim = !live ? 0 : (rows_left < PYR_BLOCK ? (int)rows_left : PYR_BLOCK);  // valid rows
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rr = rh * 32 + (e / 4) * 8 + half * 4 + e % 4;
      if (s_.kl > qoff + rr || rr >= lim) pf[e] = 0.f;
    }
  }
  bf16x8 pb[2];
  pack_b(pf, pb);
  __builtin_amdgcn_sched_barrier(0);
  // dV^T += dO^T P; the Q^T fragments are read and dS formed meanwhile
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      s_.dva[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[k2][dt], pb[k2], s_.dva[dt], 0, 0, 0);
  bf16x8 tq[2][D / 32];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) tq[k2][dt] = dkdv_tread<D>(Qt, to, to8, rh, k2, dt);
  f32x16 dsf;
#pragma unroll
  for (int e = 0; e < 16; ++e) dsf[e] = pf[e] * (dp[e] - dd4[e / 4][e % 4]);
  bf16x8 dsb[2];
  pack_b(dsf, dsb);
  __builtin_amdgcn_sched_barrier(0);
  // dK^T += Q^T dS
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      s_.dka[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[k2][dt], dsb[k2], s_.dka[dt], 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  s = s2;
  dp = dp2;
}

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ rec, BwdList wl,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, PyrGeom g) {
  using SG = DkdvStage<D>;
  // Four visitor stages, each its own __shared__ array, used in a fixed
  // rotation (the loop is unrolled by four): step n reads the stages of
  // visitors n and n+1 while the loads of visitors n+2 and n+3 fill the
  // others, and the compiler can tell the arrays apart, so it does not wait for
  // those loads before the step's LDS reads.
  __shared__ __align__(16) unsigned char st0[SG::BYTES];
  __shared__ __align__(16) unsigned char st1[SG::BYTES];
  __shared__ __align__(16) unsigned char st2[SG::BYTES];
  __shared__ __align__(16) unsigned char st3[SG::BYTES];
  __shared__ int s_ids[kMaxItemQ];  // the item's query blocks, ascending

  const int nsplit = wl.hdr[0], nlight = wl.hdr[1];
  const int item = blockIdx.x;
  if (item >= nsplit + nlight) return;
  const int2 it = item < nsplit ? wl.hitems[item] : wl.litems[item - nsplit];
  const int64_t krow = it.x;
  const int ncnt = wl.cnt[krow];
  const bool split = item < nsplit;
  const int first = split ? it.y * wl.chq : 0;
  const int nq = split ? min(wl.chq, ncnt - first) : ncnt;  // query blocks of this item

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / 64);
  const int kt = w & 1;  // key tile of this wave; w >> 1 is its row half
  const int64_t slab = krow / g.nb;
  const int j = (int)(krow % g.nb);
  const int bi = (int)(slab / g.Hk), hk = (int)(slab % g.Hk);
  const int64_t kbase = slab * g.Tk;
  DkdvWave<D> s_;
  s_.l = tid % 64;
  s_.half = s_.l / 32;
  s_.rh = w >> 1;
  s_.sl2 = g.scale * PYR_LOG2E;
  s_.kl = kt * 32 + s_.l % 32;  // the lane's key in the block (B fragment column)
  const int l = s_.l, half = s_.half;
  {
    const TileLanes<D> tl(l);
    s_.r = tl.r;
    s_.t = tl.t;
    s_.t8 = tl.t8;
  }
  const int kposl = j * PYR_BLOCK + s_.kl;  // the lane's key position

  // K and V B fragments: lane key kpos, d = ks*16 + 8*half .. +7
  {
    const int64_t kr = kbase + min<int64_t>(kposl, g.Tk - 1);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      s_.kb[ks] = ld16(k + kr * D + ks * 16 + 8 * half);
      s_.vb[ks] = ld16(v + kr * D + ks * 16 + 8 * half);
    }
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s_.dka[dt][e] = 0.f;
      s_.dva[dt][e] = 0.f;
    }

  // list the item's query blocks: set bits first .. first + nq - 1 of the row
  if (w == 0) {
    BitWalk bw;
    bw.start(wl.bits + krow * wl.words, wl.words, first);
    for (int x = 0; x < nq; ++x) {
      const int ib = bw.next();
      if (l == 0) s_ids[x] = ib;
    }
  }
  __syncthreads();

  const int G = g.G;
  const int hk0 = hk * G;
  const int nvis = nq * G;  // visitors: (query block, head), heads fastest
  // cursor of the visitor whose loads are issued next
  int ci = 0, ch = 0;
  auto issue_next = [&](unsigned char* dst) {
    load_visitor<D>(q, dout, rec, g, bi, hk0 + ch, s_ids[ci], dst, w, l);
    if (++ch == G) {
      ch = 0;
      ++ci;
    }
  };
  if (nvis > 0) issue_next(st0);
  if (nvis > 1) issue_next(st1);
  if (nvis > 2) issue_next(st2);
  int vi = 0, vh = 0;  // the visitor of the current step
  constexpr int PER = SG::PER;
  f32x16 s, dp;  // S and dP of the current visitor
  if (nvis > 0) {
    // this wave's loads of visitor 0 are done when at most those of visitors
    // 1 and 2 are in flight
    if (nvis > 2)
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * PER) & 15) | (((2 * PER) >> 4) << 14));
    else if (nvis > 1)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (PER & 15) | ((PER >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();
    dkdv_first<D>(s_, st0, s, dp);
  }
  // step n: visitor n's tiles in rd, visitor n+1's in rdn; issues visitor n+3 into wr
#define PYR_DKDV_STEP(n, rd, rdn, wr)                                                       \
  {                                                                                         \
    if ((n) + 2 < nvis) /* visitor n+1 done; n+2 may be in flight */                        \
      __builtin_amdgcn_s_waitcnt(0x0F70 | (PER & 15) | ((PER >> 4) << 14));                 \
    else                                                                                    \
      __builtin_amdgcn_s_waitcnt(0x0F70);                                                   \
    lds_barrier(); /* everyone's; the stage of visitor n-1 is free */                       \
    const bool more = (n) + 3 < nvis;                                                       \
    const int i3 = more ? s_ids[ci] : 0, h3 = hk0 + ch;                                     \
    dkdv_pipe<D>(s_, s, dp, rd, rdn, s_ids[vi], j, more ? (wr) : nullptr, i3, h3, q, dout,  \
                 rec, g, bi, w);                                                            \
    if (more && ++ch == G) {                                                                \
      ch = 0;                                                                               \
      ++ci;                                                                                 \
    }                                                                                       \
    if (++vh == G) {                                                                        \
      vh = 0;                                                                               \
      ++vi;                                                                                 \
    }                                                                                       \
  }
  // (guarded steps, not breaks: an exit in mid-body makes the register
  // allocator copy the accumulators around the loop)
  for (int n = 0; n < nvis; n += 4) {
    PYR_DKDV_STEP(n, st0, st1, st3);
    if (n + 1 < nvis) PYR_DKDV_STEP(n + 1, st1, st2, st0);
    if (n + 2 < nvis) PYR_DKDV_STEP(n + 2, st2, st3, st1);
    if (n + 3 < nvis) PYR_DKDV_STEP(n + 3, st3, st0, st2);
  }
#undef PYR_DKDV_STEP

  // the two row halves of a key tile add up: waves with rh = 1 hand their sums
  // to the waves with rh = 0 through LDS (key tile 0 in st0, 1 in st1)
  __syncthreads();
  float* red = reinterpret_cast<float*>(kt == 0 ? st0 : st1);  // [dt][k or v][e][lane]
  static_assert((D / 32) * 2 * 16 * 64 * 4 <= SG::BYTES, "reduction must fit a stage");
  if (s_.rh == 1) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red[((dt * 2 + 0) * 16 + e) * 64 + l] = s_.dka[dt][e];
        red[((dt * 2 + 1) * 16 + e) * 64 + l] = s_.dva[dt][e];
      }
  }
  __syncthreads();
  if (s_.rh == 1) return;
  const int kpos = kposl;
  const int lr = l % 32;
  if (split) {  // unscaled fp32 sums into the item's slot
    float* pk = wl.part + (int64_t)item * 2 * PYR_BLOCK * D + (kt * 32 + lr) * D;
    float* pv = pk + PYR_BLOCK * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 a, b;
        float* av = reinterpret_cast<float*>(&a);
        float* bv = reinterpret_cast<float*>(&b);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int e = g4 * 4 + e4;
          av[e4] = s_.dka[dt][e] + red[((dt * 2 + 0) * 16 + e) * 64 + l];
          bv[e4] = s_.dva[dt][e] + red[((dt * 2 + 1) * 16 + e) * 64 + l];
        }
        *reinterpret_cast<float4*>(pk + dt * 32 + g4 * 8 + half * 4) = a;
        *reinterpret_cast<float4*>(pv + dt * 32 + g4 * 8 + half * 4) = b;
      }
    return;
  }
  if (kpos >= g.Tk) return;
  bf16_t* dko = dk + (kbase + kpos) * D;
  bf16_t* dvo = dv + (kbase + kpos) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4_t pk, pv;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int e = g4 * 4 + e4;
        const float sk = s_.dka[dt][e] + red[((dt * 2 + 0) * 16 + e) * 64 + l];
        const float sv = s_.dva[dt][e] + red[((dt * 2 + 1) * 16 + e) * 64 + l];
        pk[e4] = (__bf16)(sk * g.scale);
        pv[e4] = (__bf16)sv;
      }
      *reinterpret_cast<bf16x4_t*>(dko + dt * 32 + g4 * 8 + half * 4) = pk;
      *reinterpret_cast<bf16x4_t*>(dvo + dt * 32 + g4 * 8 + half * 4) = pv;
    }
}

// Sum the partial slots of every split key block row in slot order, then
// scale dK and round both to bfloat16.  One workgroup per row; light rows exit.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce(const int32_t* __restrict__ cnt,
                                                       const int32_t* __restrict__ pslot,
                                                       const float* __restrict__ part,
                                                       bf16_t* __restrict__ dk,
                                                       bf16_t* __restrict__ dv, PyrGeom g,
                                                       int chq) {
  const int64_t krow = blockIdx.x;
  const int ps = pslot[krow];
  if (ps < 0) return;
  const int nch = (cnt[krow] + chq - 1) / chq;
  const int64_t slab = krow / g.nb;
  const int j = (int)(krow % g.nb);
  constexpr int N4 = PYR_BLOCK * D / 4;  // float4 per slot half
  for (int x = threadIdx.x; x < 2 * N4; x += 256) {
    const int kv = x / N4, rem = x % N4;
    const int key = rem / (D / 4), d4 = rem % (D / 4);
    const int64_t kpos = (int64_t)j * PYR_BLOCK + key;
    if (kpos >= g.Tk) continue;
    const float4* src = reinterpret_cast<const float4*>(part) + ((int64_t)ps * 2 + kv) * N4 + rem;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < nch; ++c) {
      const float4 b = src[(int64_t)c * 2 * N4];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    const float sc = kv == 0 ? g.scale : 1.f;
    bf16x4_t o4;
    o4[0] = (__bf16)(a.x * sc);
    o4[1] = (__bf16)(a.y * sc);
    o4[2] = (__bf16)(a.z * sc);
    o4[3] = (__bf16)(a.w * sc);
    *reinterpret_cast<bf16x4_t*>((kv == 0 ? dk : dv) + (slab * g.Tk + kpos) * D + d4 * 4) = o4;
  }
}

// Workspace plan: row records, route bitmap + counts (cleared together), then
// the work list and the partial slots.
struct BwdPlan {
  int words, chq;
  int64_t rows, slots;
  size_t off_bits, off_cnt, off_pslot, off_hitems, off_litems, off_hdr, off_part, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

BwdPlan bwd_plan(const PyrGeom& g) {
  BwdPlan p;
  p.words = (g.nqb + 31) / 32;
  p.rows = (int64_t)g.B * g.Hk * g.nb;
  // visitors (query block, head) per item: about 1/4096 of the route's upper
  // bound, between G and 256, so large problems get >= ~4096 items of at most
  // 256 visitors and small ones split rows finely
  const int64_t entries = (int64_t)g.B * g.Hk * g.nqb * (g.K + 1);
  const int64_t budget = std::min<int64_t>(std::max<int64_t>(entries * g.G / 4096, g.G),
                                           std::max(256, g.G));
  p.chq = (int)std::max<int64_t>(1, budget / g.G);  // <= 256 = kMaxItemQ
  // a split row with c > chq visitors has ceil(c / chq) < 2c / chq items
  p.slots = (2 * entries + p.chq - 1) / p.chq;
  size_t off = align256((size_t)g.B * g.Hq * g.nqb * kRec * 4);
  p.off_bits = off;
  p.off_cnt = off + (size_t)p.rows * p.words * 4;
  off = align256(p.off_cnt + (size_t)p.rows * 4);
  p.off_pslot = off;
  off = align256(off + (size_t)p.rows * 4);
  p.off_hitems = off;
  off = align256(off + (size_t)p.slots * 8);
  p.off_litems = off;
  off = align256(off + (size_t)p.rows * 8);
  p.off_hdr = off;
  off = align256(off + 16);
  p.off_part = off;
  p.total = off + (size_t)p.slots * 2 * PYR_BLOCK * g.D * 4;
  return p;
}

template <int D>
hipError_t launch_bwd_d(const PyrGeom& g, const bf16_t* q, const bf16_t* k, const bf16_t* v,
                        const int32_t* sel, const bf16_t* o, const float* lse,
                        const bf16_t* dout, bf16_t* dq, bf16_t* dk, bf16_t* dv, void* ws,
                        hipStream_t st) {
  const BwdPlan pl = bwd_plan(g);
  unsigned char* base = static_cast<unsigned char*>(ws);
  float* rec = reinterpret_cast<float*>(base);
  uint32_t* bits = reinterpret_cast<uint32_t*>(base + pl.off_bits);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + pl.off_cnt);
  int32_t* pslot = reinterpret_cast<int32_t*>(base + pl.off_pslot);
  int2* hitems = reinterpret_cast<int2*>(base + pl.off_hitems);
  int2* litems = reinterpret_cast<int2*>(base + pl.off_litems);
  int32_t* hdr = reinterpret_cast<int32_t*>(base + pl.off_hdr);
  float* part = reinterpret_cast<float*>(base + pl.off_part);

  const int64_t rows = (int64_t)g.B * g.Hq * g.nqb * PYR_BLOCK;
  constexpr int TPR = D / 8;
  hipLaunchKernelGGL((bwd_dsum<D>), dim3((unsigned)((rows + 256 / TPR - 1) / (256 / TPR))), dim3(256),
                     0, st, o, dout, lse, rec, g);
  const int64_t nclear = pl.rows * pl.words + pl.rows;  // bitmap and counts
  const int64_t clear_wgs = std::min<int64_t>((nclear + 255) / 256, 4096);
  hipLaunchKernelGGL(bwd_route_clear, dim3((unsigned)clear_wgs), dim3(256), 0, st, bits, nclear);
  const int64_t nent = (int64_t)g.B * g.Hk * g.nqb * (g.K + 1);
  hipLaunchKernelGGL(bwd_route_bits, dim3((unsigned)((nent + 255) / 256)), dim3(256), 0, st, sel,
                     bits, cnt, g, pl.words);
  hipLaunchKernelGGL(bwd_route_plan, dim3(1), dim3(1024), 0, st, cnt, pslot, hitems, litems, hdr,
                     pl.rows, pl.chq);
  const int nh = g.G % 4 == 0 ? 4 : (g.G % 2 == 0 ? 2 : 1);
  const int wpu = g.G / nh;
  const dim3 grid((unsigned)((int64_t)g.B * g.Hk * g.nqb * wpu));
  if (nh == 4)
    hipLaunchKernelGGL((bwd_dq<D, 8>), grid, dim3(512), 0, st, q, k, v, sel, dout, rec, dq, g, wpu);
  else if (nh == 2)
    hipLaunchKernelGGL((bwd_dq<D, 4>), grid, dim3(256), 0, st, q, k, v, sel, dout, rec, dq, g, wpu);
  else
    hipLaunchKernelGGL((bwd_dq<D, 2>), grid, dim3(128), 0, st, q, k, v, sel, dout, rec, dq, g, wpu);
  BwdList wl;
  wl.bits = bits;
  wl.cnt = cnt;
  wl.hitems = hitems;
  wl.litems = litems;
  wl.hdr = hdr;
  wl.part = part;
  wl.words = pl.words;
  wl.chq = pl.chq;
  hipLaunchKernelGGL((bwd_dkdv<D>), dim3((unsigned)(pl.rows + pl.slots)), dim3(256), 0, st, q, k,
                     v, dout, rec, wl, dk, dv, g);
  hipLaunchKernelGGL((bwd_dkdv_reduce<D>), dim3((unsigned)pl.rows), dim3(256), 0, st, cnt, pslot,
                     part, dk, dv, g, pl.chq);
  return hipGetLastError();
}

}  // namespace

size_t pyr_attn_bwd_ws_bytes(const PyrGeom& g) { return bwd_plan(g).total; }

int64_t pyr_attn_bwd_items_bound(const PyrGeom& g) {
  const BwdPlan p = bwd_plan(g);
  return p.rows + p.slots;
}

hipError_t pyr_launch_attn_bwd(const PyrGeom& g, const void* q, const void* k, const void* v,
                               const int32_t* sel, const void* o, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, void* ws,
                               hipStream_t st) {
  const bf16_t* qq = static_cast<const bf16_t*>(q);
  const bf16_t* kk = static_cast<const bf16_t*>(k);
  const bf16_t* vv = static_cast<const bf16_t*>(v);
  const bf16_t* oo = static_cast<const bf16_t*>(o);
  const bf16_t* dd = static_cast<const bf16_t*>(dout);
  bf16_t* dqq = static_cast<bf16_t*>(dq);
  bf16_t* dkk = static_cast<bf16_t*>(dk);
  bf16_t* dvv = static_cast<bf16_t*>(dv);
  return g.D == 64 ? launch_bwd_d<64>(g, qq, kk, vv, sel, oo, lse, dd, dqq, dkk, dvv, ws, st)
                   : launch_bwd_d<128>(g, qq, kk, vv, sel, oo, lse, dd, dqq, dkk, dvv, ws, st);
}
