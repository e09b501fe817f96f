// Block-sparse index estimation (MInference 1.0 summary page, "Approach":
// mean-pooled 64-token block attention).  Q and K are mean-pooled per 64-row
// block in fp32, the pooled logits z[b][c] = scale * Qp[b] . Kp[c] are formed
// for c <= b, and each query block keeps its top-k key blocks (ties to the
// lower block index, output ascending).  Ranking uses the pre-softmax logits:
// a softmax is monotone within a row, so the selected set is the same.
#include "block_scan.h"

namespace mmsa {

// grid (blocks, pool tasks), block 256.
template <int D>
__global__ __launch_bounds__(256) void k_pool(Dims dm, Tables tb, char* ws, const bf16_t* __restrict__ q,
                                              const bf16_t* __restrict__ k) {
  const PoolTask T = wsp<const PoolTask>(ws, tb.off_pool)[blockIdx.y];
  const bf16_t* src = (T.is_k ? k : q) + T.src_off;
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int RG = 256 / CH;         // row groups
  constexpr int RPT = 64 / RG;         // rows per thread
  __shared__ float part[RG][D];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int rq = tid / CH, dc = tid % CH;
  const int r_begin = b * 64, n = min(64, dm.L - r_begin);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int r = rq + RG * rr;
    if (r < n) {
      uint4 u = ld16(src + (int64_t)(r_begin + r) * T.row_stride + 8 * dc);
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(w4[e] << 16);
        acc[2 * e + 1] += __uint_as_float(w4[e] & 0xffff0000u);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rq][8 * dc + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int g = 0; g < RG; ++g) s += part[g][tid];
    wsp<float>(ws, T.ws_dst)[(int64_t)b * D + tid] = s / (float)n;
  }
}

// Lower-triangle 64x64 tiles of z.  grid (tiles, block heads), block 256.
// The pooled rows pass through LDS 32 dims at a time, stored d-major, so for
// each d a thread reads its 4 query values and its 4 key values as one
// 16-byte read each (2 LDS reads per 16 FMAs) and 16 KB of LDS lets many
// workgroups share a CU; every output still sums over d in order.
template <int D>
__global__ __launch_bounds__(256) void k_block_logits(Dims dm, Tables tb, char* ws, int nB) {
  constexpr int DC = 32;   // dims staged at a time
  const BlockTask T = wsp<const BlockTask>(ws, tb.off_block)[blockIdx.y];
  const int r = blockIdx.x;
  int bt = (int)((sqrtf(8.f * r + 1.f) - 1.f) * 0.5f);
  while ((bt + 1) * (bt + 2) / 2 <= r) ++bt;
  while (bt * (bt + 1) / 2 > r) --bt;
  const int ct = r - bt * (bt + 1) / 2;
  __shared__ float4 Qs[DC][16];   // Qs[d][i] = pooled Q of rows 4i..4i+3 at dim d0 + d
  __shared__ float4 Ks[DC][16];
  const float* qp = wsp<const float>(ws, T.ws_qp);
  const float* kp = wsp<const float>(ws, T.ws_kp);
  const int tid = threadIdx.x;
  // this thread's staging element: row rr, dims cc..cc+3 of each 32-dim chunk
  const int rr = tid % 64, cc = 4 * (tid / 64);   // 64 rows x 4 groups of 4 dims: 16 dims a pass
  const int bq = 64 * bt + rr, bk = 64 * ct + rr;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  float* qs = reinterpret_cast<float*>(&Qs[0][0]);
  float* ks = reinterpret_cast<float*>(&Ks[0][0]);
  for (int d0 = 0; d0 < D; d0 += DC) {
#pragma unroll
    for (int h = 0; h < DC / 16; ++h) {   // 256 threads x 4 dims = 16 dims of 64 rows per pass
      const int c = cc + 16 * h;
      const float4 a = bq < nB ? *reinterpret_cast<const float4*>(qp + (int64_t)bq * D + d0 + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 e = bk < nB ? *reinterpret_cast<const float4*>(kp + (int64_t)bk * D + d0 + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      qs[(c + 0) * 64 + rr] = a.x, qs[(c + 1) * 64 + rr] = a.y, qs[(c + 2) * 64 + rr] = a.z, qs[(c + 3) * 64 + rr] = a.w;
      ks[(c + 0) * 64 + rr] = e.x, ks[(c + 1) * 64 + rr] = e.y, ks[(c + 2) * 64 + rr] = e.z, ks[(c + 3) * 64 + rr] = e.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int d = 0; d < DC; ++d) {
      const float4 a4 = Qs[d][ty], b4 = Ks[d][tx];
      const float a[4] = {a4.x, a4.y, a4.z, a4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* z = wsp<float>(ws, T.ws_z);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 64 * bt + 4 * ty + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 64 * ct + 4 * tx + j;
      if (b < nB && c <= b) z[(int64_t)b * nB + c] = acc[i][j] * dm.scale;
    }
  }
}

// Top-k key blocks of one query block from its LDS-resident logit row.
// Radix select on the orderable key, 8 bits a round from the top: one
// histogram per wave (logits cluster in few bins), then the threshold bin by a
// suffix sum over the bins across the workgroup.
// grid (query blocks, block heads), block 256, dynamic LDS nB floats.
__global__ __launch_bounds__(256) void k_block_topk(Tables tb, char* ws, int nB) {
  const BlockTask T = wsp<const BlockTask>(ws, tb.off_block)[blockIdx.y];
  extern __shared__ float zs[];
  __shared__ uint32_t hist[4][256];
  __shared__ uint32_t sh_pref, sh_krem, sh_all;
  __shared__ int red[17];
  const int b = blockIdx.x, tid = threadIdx.x, wv = tid >> 6;
  const int n = b + 1;
  const int k = min(T.kb, n);
  const float* zrow = wsp<const float>(ws, T.ws_z) + (int64_t)b * nB;
  for (int i = tid; i < n; i += 256) zs[i] = zrow[i];
  int32_t* out = wsp<int32_t>(ws, T.ws_idx) + (int64_t)b * T.kb;
  for (int i = k + tid; i < T.kb; i += 256) out[i] = -1;
  __syncthreads();
  uint32_t pref = 0, pmask = 0, krem = (uint32_t)k;
  if (k < n) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += 256) {
        const uint32_t key = order_key(zs[i]);
        if ((key & pmask) == pref) atomicAdd(&hist[wv][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // thread t holds bin 255 - t: a prefix sum in thread order is a suffix sum over bins
      const uint32_t c = hist[0][255 - tid] + hist[1][255 - tid] + hist[2][255 - tid] + hist[3][255 - tid];
      int tot;
      const uint32_t above = (uint32_t)block_excl_sum((int)c, red, &tot);
      if (above < krem && above + c >= krem) {
        sh_pref = pref | ((uint32_t)(255 - tid) << shift);
        sh_krem = krem - above;
        sh_all = (above + c == krem) ? 1u : 0u;   // the whole bin is taken
      }
      __syncthreads();
      pref = sh_pref;
      krem = sh_krem;
      pmask |= 255u << shift;
      const bool done = sh_all != 0u;
      __syncthreads();
      // every key of the threshold bin is selected: the lower bits decide nothing
      if (done) break;
    }
  } else {
    pref = 0;
    krem = (uint32_t)n;
  }
  // Emit: every key above the threshold, and the first `need` keys equal to
  // it in index order, comparing the bits the rounds decided (all of them
  // unless a round took its whole threshold bin).  Each thread takes a
  // contiguous run of the row, so thread order is index order and two scans
  // place every output.
  const uint32_t thr = pref;
  const int need = (int)krem;
  const int per = (n + 255) / 256;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  int n_eq = 0, n_gt = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = order_key(zs[i]) & pmask;
    n_eq += key == thr ? 1 : 0;
    n_gt += key > thr ? 1 : 0;
  }
  int eq_tot, sel_tot;
  const int eq_before = block_excl_sum(n_eq, red, &eq_tot);
  const int take_eq = max(0, min(n_eq, need - eq_before));
  int pos = block_excl_sum(n_gt + take_eq, red, &sel_tot);
  int eq_seen = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = order_key(zs[i]) & pmask;
    bool sel = key > thr;
    if (key == thr) sel = eq_seen++ < take_eq;
    if (sel) out[pos++] = i;
  }
}

hipError_t launch_block_estimate(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k, int nB,
                                 hipStream_t s) {
  if (tb.n_block == 0) return hipSuccess;
  const bf16_t* qq = (const bf16_t*)q;
  const bf16_t* kk = (const bf16_t*)k;
  const int nBt = (nB + 63) / 64;
  const int ntri = nBt * (nBt + 1) / 2;
  if (dm.d == 128) {
    k_pool<128><<<dim3(nB, (unsigned)tb.n_pool), 256, 0, s>>>(dm, tb, ws, qq, kk);
    k_block_logits<128><<<dim3(ntri, (unsigned)tb.n_block), 256, 0, s>>>(dm, tb, ws, nB);
  } else {
    k_pool<64><<<dim3(nB, (unsigned)tb.n_pool), 256, 0, s>>>(dm, tb, ws, qq, kk);
    k_block_logits<64><<<dim3(ntri, (unsigned)tb.n_block), 256, 0, s>>>(dm, tb, ws, nB);
  }
  k_block_topk<<<dim3(nB, (unsigned)tb.n_block), 256, (size_t)nB * sizeof(float), s>>>(tb, ws, nB);
  return hipGetLastError();
}

}  // namespace mmsa
