// Workgroup-wide scans and wave histograms shared by the selection kernels
// (top-k of scores, top-k of pooled block logits).
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

// Adds one to bin `bin` of a per-wave LDS histogram for every lane with
// `valid`.  Lanes adding to one LDS word are serialised, so the lanes sharing
// the bin of the first valid lane, then of the next one left, are counted
// with one add each; the remaining lanes add one by one.  Any subset of the
// wave's lanes may call it together.  It pays where keys crowd into few bins
// (score top-k: 1M layer estimation 8.44 -> 8.28 ms) and costs where they
// spread (pooled block logits: 256K block estimation 2.54 -> 2.68 ms, so the
// block top-k adds directly).
__device__ __forceinline__ void wave_hist_add(uint32_t* hist, uint32_t bin, bool valid) {
  const int lane = threadIdx.x & 63;
  uint64_t todo = __ballot(valid);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (todo == 0ull) return;
    const int ld = __builtin_ctzll(todo);
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, ld);
    const uint64_t same = __ballot(valid && bin == lb) & todo;
    if (lane == ld) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
    todo &= ~same;
  }
  if ((todo >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
}

}  // namespace mmsa
