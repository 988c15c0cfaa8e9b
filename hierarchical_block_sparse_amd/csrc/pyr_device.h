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
