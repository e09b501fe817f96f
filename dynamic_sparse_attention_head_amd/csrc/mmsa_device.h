// Device helpers for the gfx950 kernels of libmmsa.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mmsa_internal.h"

namespace mmsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;   // raw bfloat16 bits in memory

template <class T>
__device__ __forceinline__ T* wsp(char* ws, int64_t off) { return reinterpret_cast<T*>(ws + off); }
template <class T>
__device__ __forceinline__ const T* wsp(const char* ws, int64_t off) { return reinterpret_cast<const T*>(ws + off); }

// Read-only tables through the constant address space: with a uniform address
// these become scalar loads, and the values stay in scalar registers.
#define MMSA_CONST __attribute__((address_space(4)))
template <class T>
__device__ __forceinline__ const MMSA_CONST T* cptr(const char* ws, int64_t off) {
  return (const MMSA_CONST T*)(ws + off);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l: A row l%16, k-slots
// 8*(l/16)..+8; B column l%16, same k-slots; D column l%16, rows 4*(l/16)+i.
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }
// round to nearest even (inputs here are finite)
__device__ __forceinline__ uint32_t f2bf_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf_bits(lo) | (f2bf_bits(hi) << 16);
}

// two floats -> packed bf16 pair with the hardware round-to-nearest-even convert
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2_hw(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Merge two (max, sum-of-exp2) pairs of the same row.
__device__ __forceinline__ float2 lse2_merge(float2 a, float2 b) {
  if (a.x == -INFINITY) return b;
  if (b.x == -INFINITY) return a;
  float m = fmaxf(a.x, b.x);
  return make_float2(m, a.y * exp2f(a.x - m) + b.y * exp2f(b.x - m));
}

// Orderable key of a float32: larger value -> larger key; -0 equals +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ----- exact comparison of grid line scores sgn(X) X^2 / cnt ---------------
struct U128 { uint64_t hi, lo; };
__device__ __forceinline__ U128 mul64x64(uint64_t a, uint64_t b) { return U128{__umul64hi(a, b), a * b}; }
__device__ __forceinline__ U128 mul128x64(U128 a, uint64_t b) {
  U128 r = mul64x64(a.lo, b);
  r.hi += a.hi * b;
  return r;
}
__device__ __forceinline__ int cmp128(U128 a, U128 b) {
  if (a.hi != b.hi) return a.hi > b.hi ? 1 : -1;
  if (a.lo != b.lo) return a.lo > b.lo ? 1 : -1;
  return 0;
}
// +1 if (X1,c1) scores higher than (X2,c2), -1 if lower, 0 if equal.
__device__ __forceinline__ int grid_cmp(int64_t X1, int64_t c1, int64_t X2, int64_t c2) {
  int s1 = (X1 > 0) - (X1 < 0), s2 = (X2 > 0) - (X2 < 0);
  if (s1 != s2) return s1 > s2 ? 1 : -1;
  if (s1 == 0) return 0;
  uint64_t a1 = (uint64_t)(X1 < 0 ? -X1 : X1), a2 = (uint64_t)(X2 < 0 ? -X2 : X2);
  int c = cmp128(mul128x64(mul64x64(a1, a1), (uint64_t)c2), mul128x64(mul64x64(a2, a2), (uint64_t)c1));
  return s1 > 0 ? c : -c;
}

// Workgroup-wide exclusive prefix count of a predicate, in thread order.
// `red` must hold blockDim/64 + 1 ints of LDS.  Returns the thread's rank and
// sets *total.  Contains two barriers.
__device__ __forceinline__ int block_excl_count(bool pred, int* red, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  uint64_t bal = __ballot(pred);
  int in_wave = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) red[wv] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    int c = red[i];
    before += (i < wv) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + in_wave;
}

}  // namespace mmsa
