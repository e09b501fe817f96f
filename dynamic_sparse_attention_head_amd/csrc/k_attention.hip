// Block-sparse causal prefill over the planned key tiles and gathered columns
// (MMInference verdict page, key_machinery: FlashAttention-style kernels that
// load only the permuted blocks and keep matrix-core compute dense; the online
// softmax is the FlashAttention-2 recurrence those kernels build on).
//
// One workgroup = one 64-row query tile of one head, 4 waves x 16 rows.  Key
// chunks of 64 (a whole view tile, or 64 gathered columns) are staged in LDS:
// K row-major, V transposed (d-major, keys in MFMA k-slot order), so both
// products run as bf16 16x16x32 MFMA with fp32 accumulation:
//   S^T (keys x queries) = K . Q^T     -> each lane holds one query's 16 logits
//   O^T (d x queries)   += V^T . P^T   -> each lane holds one query's outputs
// With these transposed layouts a lane owns one query row throughout, so the
// online-softmax row max needs only two cross-lane shuffles per chunk and the
// running rescale is a per-lane scalar.  Staging is double-buffered: the next
// chunk's global loads are in flight while the current chunk is computed.
// Masking is element-wise on original positions (causal, A-shape window).
#include "mmsa_device.h"

namespace mmsa {

template <int D>
struct AttnSmem {
  static constexpr int KS = D + 8;    // K row stride (elements)
  static constexpr int VS = 64 + 8;   // V^T row stride (elements)
  bf16_t K[2][64 * KS];
  bf16_t Vt[2][D * VS];
  int kp[2][64];
};

// k-slot of the first key of key-quad kq (4 consecutive keys) inside V^T rows
__device__ __forceinline__ int vt_slot(int kq) {
  const int c = kq >> 3, q = kq & 7;
  return 32 * c + (q < 4 ? 8 * q : 8 * (q - 4) + 4);
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn(Dims dm, Tables tb, char* ws, const bf16_t* __restrict__ q,
                                                 const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                 bf16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int KS = AttnSmem<D>::KS, VS = AttnSmem<D>::VS, NC = D / 32, ND = D / 16;
  __shared__ AttnSmem<D> sm;
  const int n_items = wsp<const int32_t>(ws, dm.ws_qhist)[QUEUE_BINS];
  if ((int)blockIdx.x >= n_items) return;
  const uint32_t item = wsp<const uint32_t>(ws, dm.ws_queue)[blockIdx.x];
  const int bh = (int)(item >> 16), t = (int)(item & 0xffff);
  const HeadDev& H = wsp<const HeadDev>(ws, tb.off_heads)[bh];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 15, g4 = lane >> 4;

  // ---- query rows of this wave (B operand of S^T) ----
  const int slot = 64 * t + 16 * w + qc;
  int qpos;
  if (H.row_kind == ROW_IDENTITY) qpos = slot < dm.L ? slot : -1;
  else qpos = wsp<const int32_t>(ws, H.ws_row_order)[slot];
  bf16x8 qf[NC];
  {
    const bf16_t* qrow = (H.ws_qperm >= 0) ? wsp<const bf16_t>(ws, H.ws_qperm) + (int64_t)slot * D
                                           : q + H.q_off + (int64_t)(qpos < 0 ? 0 : qpos) * dm.q_sl;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qpos >= 0) u = ld16(qrow + 32 * c + 8 * g4);
      qf[c] = as_bf16x8(u);
    }
  }

  // ---- plan of this tile ----
  const int4 info = wsp<const int4>(ws, H.ws_info)[t];
  const int W = H.bm_words;
  // clamped to the buffers' capacities (a plan that was never built stays in bounds)
  const int n_tiles = min(max(info.x, 0), 64 * W);
  const int g_cap = (H.pattern == MMSA_GRID) ? dm.L : H.gcap;
  const int g_cnt = min(max(info.y, 0), g_cap);
  const uint64_t* bmrow = wsp<const uint64_t>(ws, H.ws_bm) + (int64_t)t * W;
  const int32_t* glist = nullptr;
  if (H.pattern == MMSA_GRID) glist = wsp<const int32_t>(ws, H.ws_row_order);
  else if (H.gcap > 0) glist = wsp<const int32_t>(ws, H.ws_gather) + (int64_t)t * H.gcap;
  const bool grouped_view = H.view_kind == VIEW_GROUPED;
  const bf16_t* kview = grouped_view ? wsp<const bf16_t>(ws, H.ws_kgrp) : k + H.k_off;
  const bf16_t* vview = grouped_view ? wsp<const bf16_t>(ws, H.ws_vgrp) : v + H.v_off;
  const int64_t kv_sl = grouped_view ? D : dm.k_sl;
  const int64_t vv_sl = grouped_view ? D : dm.v_sl;
  const int32_t* pgrp = wsp<const int32_t>(ws, dm.ws_pgrp);
  const bf16_t* kg = k + H.k_off;
  const bf16_t* vg = v + H.v_off;
  const bool ashape = H.pattern == MMSA_ASHAPE;
  const int sink = H.sink, window = H.window;
  const int n_chunks = n_tiles + (g_cnt + 63) / 64;

  // chunk descriptor -> (source row, key position) of staged row r
  // kind 0: view tile `idx`; kind 1: gathered chunk `idx`
  auto row_src = [&](int kind, int idx, int r, const bf16_t*& kb, const bf16_t*& vb, int64_t& krow,
                     int64_t& vrow) -> int {
    if (kind == 0) {
      const int vr = idx < 0 ? 0 : 64 * idx + r;
      int pos;
      if (idx < 0 || vr >= 64 * H.nT_view) pos = -1;
      else if (grouped_view) pos = pgrp[vr];
      else pos = vr < dm.L ? vr : -1;
      kb = kview;
      vb = vview;
      krow = (int64_t)vr * kv_sl;
      vrow = (int64_t)vr * vv_sl;
      return pos;
    }
    const int e = 64 * idx + r;
    const int pos = e < g_cnt ? glist[e] : -1;
    kb = kg;
    vb = vg;
    krow = (int64_t)(pos < 0 ? 0 : pos) * dm.k_sl;
    vrow = (int64_t)(pos < 0 ? 0 : pos) * dm.v_sl;
    return pos;
  };

  // ---- staging registers ----
  constexpr int KCH = D / 32;           // 16-byte K chunks per thread (row r = tid/4)
  uint4 kreg[KCH];
  uint4 vreg[4];
  int kpreg = -1;
  const int kr = tid >> 2, kpart = tid & 3;
  constexpr int VDC = D / 8;            // d-chunks of 8
  constexpr int VUNITS = 16 * VDC;      // key-quads x d-chunks
  const bool v_active = tid < VUNITS;
  const int vkq = tid / VDC, vdc = tid % VDC;

  auto load_chunk = [&](int kind, int idx) {
    const bf16_t *kb, *vb;
    int64_t krow, vrow;
    const int pos = row_src(kind, idx, kr, kb, vb, krow, vrow);
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      kreg[j] = make_uint4(0, 0, 0, 0);
      if (pos >= 0) kreg[j] = ld16(kb + krow + kpart * (D / 4) + 8 * j);
    }
    if (v_active) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int p2 = row_src(kind, idx, 4 * vkq + rr, kb, vb, krow, vrow);
        vreg[rr] = make_uint4(0, 0, 0, 0);
        if (p2 >= 0) vreg[rr] = ld16(vb + vrow + 8 * vdc);
      }
    }
    if (tid < 64) {
      const int p3 = row_src(kind, idx, tid, kb, vb, krow, vrow);
      kpreg = p3 >= 0 ? p3 : KPOS_NONE;
    }
  };
  auto store_chunk = [&](int buf) {
    bf16_t* kd = sm.K[buf] + kr * KS + kpart * (D / 4);
#pragma unroll
    for (int j = 0; j < KCH; ++j) st16(kd + 8 * j, kreg[j]);
    if (v_active) {
      const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
      bf16_t* vd = sm.Vt[buf] + (8 * vdc) * VS + vt_slot(vkq);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint2 lo, hi;
        lo.x = (w0[m] & 0xffffu) | (w1[m] << 16);
        lo.y = (w2[m] & 0xffffu) | (w3[m] << 16);
        hi.x = (w0[m] >> 16) | (w1[m] & 0xffff0000u);
        hi.y = (w2[m] >> 16) | (w3[m] & 0xffff0000u);
        *reinterpret_cast<uint2*>(vd + (2 * m) * VS) = lo;
        *reinterpret_cast<uint2*>(vd + (2 * m + 1) * VS) = hi;
      }
    }
    if (tid < 64) sm.kp[buf][tid] = kpreg;
  };

  // tile iteration over the bitmap (uniform across the workgroup)
  int wi = 0;
  uint64_t bits = W > 0 ? bmrow[0] : 0ull;
  auto next_desc = [&](int ci, int& kind, int& idx) {
    if (ci < n_tiles) {
      while (bits == 0ull && wi + 1 < W) bits = bmrow[++wi];
      const int b = __ffsll((unsigned long long)bits) - 1;
      bits &= bits - 1;
      kind = 0;
      idx = b < 0 ? -1 : 64 * wi + b;
    } else {
      kind = 1;
      idx = ci - n_tiles;
    }
  };

  floatx4 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = dm.scale_log2;

  if (n_chunks > 0) {
    int kind, idx;
    next_desc(0, kind, idx);
    load_chunk(kind, idx);
    store_chunk(0);
    __syncthreads();
  }
  for (int ci = 0; ci < n_chunks; ++ci) {
    const int buf = ci & 1;
    const bool has_next = ci + 1 < n_chunks;
    if (has_next) {
      int kind, idx;
      next_desc(ci + 1, kind, idx);
      load_chunk(kind, idx);
    }
    // ---- S^T = K . Q^T ----
    const bf16_t* Kb = sm.K[buf];
    floatx4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 a = as_bf16x8(ld16(Kb + (16 * kb + qc) * KS + 32 * c + 8 * g4));
        sacc[kb] = mfma16(a, qf[c], sacc[kb]);
      }
    }
    // ---- mask, online softmax ----
    float s[16];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int4 kk = *reinterpret_cast<const int4*>(&sm.kp[buf][16 * kb + 4 * g4]);
      const int kpv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bool ok = kpv[i] <= qpos;
        if (ashape) ok = ok && (kpv[i] < sink || qpos - kpv[i] < window);
        const float x = ok ? sacc[kb][i] * sl2 : -INFINITY;
        s[4 * kb + i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float corr = exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = exp2f(s[e] - m_use), p1 = exp2f(s[e + 1] - m_use);
      psum += p0 + p1;
      pk[e >> 1] = pack_bf2(p0, p1);
    }
    l_run = l_run * corr + psum;
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] *= corr;
    // ---- O^T += V^T . P^T ----
    const bf16_t* Vb = sm.Vt[buf];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const bf16x8 pb = as_bf16x8(make_uint4(pk[4 * cc], pk[4 * cc + 1], pk[4 * cc + 2], pk[4 * cc + 3]));
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16x8 a = as_bf16x8(ld16(Vb + (16 * db + qc) * VS + 32 * cc + 8 * g4));
        oacc[db] = mfma16(a, pb, oacc[db]);
      }
    }
    if (has_next) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  float l_tot = l_run + shfl_xor_f(l_run, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  if (qpos >= 0) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    bf16_t* orow = (H.ws_operm >= 0) ? wsp<bf16_t>(ws, H.ws_operm) + (int64_t)slot * D
                                     : o + H.o_off + (int64_t)qpos * dm.o_sl;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      uint2 pkd;
      pkd.x = pack_bf2(oacc[db][0] * inv, oacc[db][1] * inv);
      pkd.y = pack_bf2(oacc[db][2] * inv, oacc[db][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * db + 4 * g4) = pkd;
    }
    if (lse != nullptr && g4 == 0) {
      const float val = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      lse[((int64_t)H.b * dm.Hq + H.h) * dm.L + qpos] = val;
    }
  }
}

hipError_t launch_attention(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k, const void* v,
                            void* o, float* lse, int64_t max_items, hipStream_t s) {
  if (max_items <= 0) return hipSuccess;
  if (dm.d == 128)
    k_attn<128><<<(unsigned)max_items, 256, 0, s>>>(dm, tb, ws, (const bf16_t*)q, (const bf16_t*)k,
                                                     (const bf16_t*)v, (bf16_t*)o, lse);
  else
    k_attn<64><<<(unsigned)max_items, 256, 0, s>>>(dm, tb, ws, (const bf16_t*)q, (const bf16_t*)k,
                                                    (const bf16_t*)v, (bf16_t*)o, lse);
  return hipGetLastError();
}

}  // namespace mmsa
