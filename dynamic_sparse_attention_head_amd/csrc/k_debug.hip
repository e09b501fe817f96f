// Debug support (MMSA_FLAG_DEBUG): a scan of Q, K and V that records whether
// any element is a NaN or an infinity.  A bf16 value is non-finite exactly
// when its 8 exponent bits are all ones.  One pass over the three tensors,
// 16 bytes per lane, bound by HBM bandwidth; one atomic OR per wave that saw
// a non-finite value.
#include "mmsa_device.h"

namespace mmsa {

__device__ __forceinline__ bool any_nonfinite_bf16x8(uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) bad |= ((w[i] & 0x7f80u) == 0x7f80u) | ((w[i] & 0x7f800000u) == 0x7f800000u);
  return bad;
}

// blockIdx.y: one (batch, head) slice of Q (first B*Hq), then of K, then of V.
__global__ __launch_bounds__(256) void k_nonfinite_scan(Dims dm, const bf16_t* __restrict__ q,
                                                        const bf16_t* __restrict__ k,
                                                        const bf16_t* __restrict__ v, uint32_t* __restrict__ flag) {
  const int nq = dm.B * dm.Hq, nkv = dm.B * dm.Hkv;
  int sl = blockIdx.y, which;
  const bf16_t* base;
  int64_t rs;
  if (sl < nq) {
    which = 0;
    base = q + (sl / dm.Hq) * dm.q_sb + (sl % dm.Hq) * dm.q_sh;
    rs = dm.q_sl;
  } else if (sl < nq + nkv) {
    sl -= nq;
    which = 1;
    base = k + (sl / dm.Hkv) * dm.k_sb + (sl % dm.Hkv) * dm.k_sh;
    rs = dm.k_sl;
  } else {
    sl -= nq + nkv;
    which = 2;
    base = v + (sl / dm.Hkv) * dm.v_sb + (sl % dm.Hkv) * dm.v_sh;
    rs = dm.v_sl;
  }
  const int cpr = dm.d / 8;                       // 16-byte chunks per row
  const int64_t n = (int64_t)dm.L * cpr;
  bool bad = false;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = c / cpr, ch = c - row * cpr;
    bad |= any_nonfinite_bf16x8(ld16(base + row * rs + 8 * ch));
  }
  if (__ballot(bad) != 0ull && (threadIdx.x & 63) == 0) atomicOr(flag, 1u << which);
}

hipError_t launch_nonfinite_scan(const Dims& dm, char* ws, const void* q, const void* k, const void* v,
                                 hipStream_t s) {
  const int slices = dm.B * dm.Hq + 2 * dm.B * dm.Hkv;
  if (slices <= 0 || dm.L <= 0) return hipSuccess;
  const int64_t chunks = (int64_t)dm.L * (dm.d / 8);
  const int64_t want = (chunks + 255) / 256;
  const int gx = (int)(want < 32 ? want : 32);
  k_nonfinite_scan<<<dim3(gx, slices), 256, 0, s>>>(dm, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                                                    reinterpret_cast<uint32_t*>(ws + dm.ws_flag));
  return hipGetLastError();
}

}  // namespace mmsa
