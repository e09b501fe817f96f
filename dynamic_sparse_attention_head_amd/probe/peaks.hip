// Microbenchmarks for the roofline peaks measured on the box (not part of the
// sparse-attention path, and not in libmmsa): a loop of bf16 32x32x16 MFMAs,
// the instruction the attention kernel runs on, and a 16-bytes-per-lane
// streaming copy.  Built into libmmsa_probe.so; timed by bench.py --peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Every wave issues `iters` x 4 independent MFMAs (four accumulators, so
// back-to-back issue never waits on a result).  FLOPs per launch:
// blocks * (256 / 64) waves * iters * 4 * 32 * 32 * 16 * 2.
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float acc = 0.f;
  for (int i = 0; i < 16; ++i) acc += c0[i] + c1[i] + c2[i] + c3[i];
  // one store per thread keeps the results alive (the values do not matter)
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// dst[i] = src[i] over n16 16-byte words: each thread moves 4 words, a
// block's 1024 consecutive words per pass (four loads in flight per lane).
__global__ __launch_bounds__(256) void k_copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024; base < n16; base += stride) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = base + j * 256 + threadIdx.x;
      if (i < n16) v[j] = src[i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = base + j * 256 + threadIdx.x;
      if (i < n16) dst[i] = v[j];
    }
  }
}

// Read-only stream: each thread sums the 16-byte words it reads (four in
// flight per pass) and writes one word, so the bytes moved are the reads.
__global__ __launch_bounds__(256) void k_read16(const uint4* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 1024;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * 1024; base < n16; base += stride) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = base + j * 256 + threadIdx.x;
      v[j] = i < n16 ? src[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

extern "C" {

// sink: device float[blocks * 256]
int probe_mfma(int blocks, int iters, float* sink, void* stream) {
  k_mfma_loop<<<blocks, 256, 0, (hipStream_t)stream>>>(iters, sink);
  return (int)hipGetLastError();
}

// src, dst: device buffers of `bytes` (a multiple of 16, 16-byte aligned)
int probe_copy(const void* src, void* dst, int64_t bytes, int blocks, void* stream) {
  k_copy16<<<blocks, 256, 0, (hipStream_t)stream>>>((const uint4*)src, (uint4*)dst, bytes / 16);
  return (int)hipGetLastError();
}

// sink: device uint32[blocks * 256]
int probe_read(const void* src, int64_t bytes, int blocks, void* sink, void* stream) {
  k_read16<<<blocks, 256, 0, (hipStream_t)stream>>>((const uint4*)src, bytes / 16, (uint32_t*)sink);
  return (int)hipGetLastError();
}

}  // extern "C"
