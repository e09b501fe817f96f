// Workgroup-wide scans shared by the selection kernels (top-k of scores,
// top-k of pooled block logits).
#pragma once
#include "mmsa_device.h"

namespace mmsa {

// Workgroup-wide exclusive prefix sum of v in thread order; sets *total.
// red: 17 ints of LDS.  Two barriers.
__device__ __forceinline__ int block_excl_sum(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(inc, m, 64);
    if (lane >= m) inc += o;
  }
  if (lane == 63) red[wv] = inc;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const int c = red[i];
    before += (i < wv) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

}  // namespace mmsa
