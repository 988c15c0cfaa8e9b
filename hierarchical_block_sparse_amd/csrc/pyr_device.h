// Device-side helpers for the gfx950 kernels of libpyr: bf16 conversion,
// 16-byte loads, MFMA operand types and LogSumExp pair merging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // storage type of bfloat16 tensors
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define PYR_LOG2E 1.4426950408889634f
#define PYR_LN2 0.6931471805599453f

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 values -> one packed pair of bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Unpack 8 elements of a 16-byte chunk to fp32.
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& r, float* out);

template <>
__device__ __forceinline__ void unpack16<float>(const uint4& r, float* out) {
  out[0] = __uint_as_float(r.x);
  out[1] = __uint_as_float(r.y);
  out[2] = __uint_as_float(r.z);
  out[3] = __uint_as_float(r.w);
}

template <>
__device__ __forceinline__ void unpack16<bf16_t>(const uint4& r, float* out) {
  out[0] = bf16_to_f32(r.x & 0xffffu);
  out[1] = bf16_to_f32(r.x >> 16);
  out[2] = bf16_to_f32(r.y & 0xffffu);
  out[3] = bf16_to_f32(r.y >> 16);
  out[4] = bf16_to_f32(r.z & 0xffffu);
  out[5] = bf16_to_f32(r.z >> 16);
  out[6] = bf16_to_f32(r.w & 0xffffu);
  out[7] = bf16_to_f32(r.w >> 16);
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load (non-temporal: data read once, keep it out of the way).
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& r) {
  return __builtin_bit_cast(bf16x8, r);
}

// Merge two LogSumExp partials (m, s) meaning m + log2(s) in the log2 domain.
// An empty partial has m = -inf and s = 0.
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  float mx = fmaxf(m, m2);
  if (mx == -INFINITY) {
    m = mx;
    s = 0.f;
    return;
  }
  s = s * exp2f(m - mx) + s2 * exp2f(m2 - mx);
  m = mx;
}

// Workgroup barrier that orders LDS only.  __syncthreads() carries a
// workgroup fence, and a fence waits for every direct global-to-LDS load in
// flight (the compiler counts them as pending LDS writes), which would undo a
// prefetch; code that waits for its own loads explicitly uses this instead.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier; lgkmcnt(0) completes this wave's LDS accesses first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Combine a value with that of the lane's partner in the other 16-lane row
// (xor 16) or the other 32-lane half (xor 32).  A swap hands each lane the
// pair (even, odd) of the two lanes, so a symmetric combine needs no select.
__device__ __forceinline__ float max16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Full-wavefront reductions (64 lanes).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// A route row is a set of key blocks (PHBA §A.1.2 routes to distinct strictly
// preceding blocks; its block-major metadata lists each (query, block) pair
// once): entry jj of a row, holding block j, is used only when j is a block
// id in [0, nb) and no earlier entry of the row holds j.  The loop reads every
// earlier entry without an early exit, so the reads can be issued together.
__device__ __forceinline__ bool route_entry_used(const int* row, int jj, int j, int nb) {
  if (j < 0 || j >= nb) return false;
  bool first = true;
  for (int x = 0; x < jj; ++x) first = first && row[x] != j;
  return first;
}

// Whole-wave form of route_entry_used for the entries c*64 + lane of a row
// raw[0..cnt) (in LDS, visible to the wave): bit c of the result is set when
// entry c*64 + lane is used.  Each lane holds its entry in a register; for
// every earlier entry x, taken with readlane (one uniform lane index per
// step), the compare j == x is itself the 64-lane mask of the lanes holding
// the same block, so a step is one readlane, one compare and a few scalar
// mask operations, with no per-lane branch.  At most 32 chunks (cnt <= 2048).
__device__ __forceinline__ uint32_t route_used_mask(const int* raw, int cnt, int nb) {
  const int l = threadIdx.x % 64;
  uint32_t used = 0;
  for (int c = 0; c * 64 < cnt; ++c) {
    const int jj = c * 64 + l;
    const int j = jj < cnt ? raw[jj] : -1;
    unsigned long long dup = 0;  // bit l: an earlier entry holds lane l's block
    // every entry of the earlier chunks (all earlier than this chunk's)
    for (int b = 0; b < c; ++b) {
      const int e = raw[b * 64 + l];
#pragma unroll 8
      for (int x = 0; x < 64; ++x) dup |= __ballot(j == __builtin_amdgcn_readlane(e, x));
    }
    // the entries of this chunk before the lane's: lanes above x
    const int nx = cnt - c * 64 < 64 ? cnt - c * 64 : 64;
    const int nx8 = (nx + 7) & ~7;  // lanes past cnt hold -1, which no block equals
    for (int x0 = 0; x0 < nx8; x0 += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int x = x0 + u;
        const unsigned long long above = x == 63 ? 0ull : ~((2ull << x) - 1ull);
        dup |= __ballot(j == __builtin_amdgcn_readlane(j, x)) & above;
      }
    }
    if (j >= 0 && j < nb && !((dup >> l) & 1ull)) used |= 1u << c;
  }
  return used;
}

// One whole wave appends to out[n0..) the entries of the route row raw[0..cnt)
// marked in `used` (route_used_mask) that also satisfy keep(j), in row order;
// returns the new count, uniform across the wave.
template <typename Keep>
__device__ __forceinline__ int route_compact_used(const int* raw, int cnt, uint32_t used, int* out,
                                                  int n0, Keep keep) {
  const int l = threadIdx.x % 64;
  int n = n0;
  for (int c = 0; c * 64 < cnt; ++c) {
    const int jj = c * 64 + l;
    const int j = jj < cnt ? raw[jj] : -1;
    const bool ok = (used >> c & 1u) && keep(j);
    const unsigned long long m = __ballot(ok);
    if (ok) out[n + __popcll(m & ((1ull << l) - 1ull))] = j;
    n += __popcll(m);
  }
  return n;
}

// One whole wave appends to out[n0..) the used entries of the route row
// raw[0..cnt) (both in LDS, raw visible to the wave) that also satisfy
// keep(j), in row order; returns the new count, uniform across the wave.
template <typename Keep>
__device__ __forceinline__ int route_compact_wave(const int* raw, int cnt, int nb, int* out,
                                                  int n0, Keep keep) {
  return route_compact_used(raw, cnt, route_used_mask(raw, cnt, nb), out, n0, keep);
}

// Direct 16-byte global -> LDS load through a buffer resource (the MUBUF form
// of the LDS DMA).  Lane i's 16 bytes at base + voffset land at
// lds + 16 * i; base and lds must be wave-uniform, and byte offsets at or past
// `bytes` read as zero instead of touching memory.  Like the global form, it
// is counted by the vector-memory counter only.  It replaces
// __builtin_amdgcn_global_load_lds where a kernel reads LDS while such loads
// are in flight: the compiler treats the global form as a flat access that may
// also be counted by the LDS counter, and then every wait for an LDS read
// becomes a wait for all of them; with the buffer form it keeps counting the
// reads one by one.
typedef __attribute__((address_space(3))) void lds_dma_void;
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t bytes, uint32_t voffset,
                                          lds_dma_void* lds) {
  // word 3 of a raw gfx9 buffer resource: 32-bit data format, no stride, no swizzle
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voffset, 0, 0, 0);
}
