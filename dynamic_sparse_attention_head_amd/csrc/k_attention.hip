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
struct AttnSmem {  // 2 stages of K (row-major), V^T (d-major) and key positions
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

// One (head, query tile) work item.  Ends with a workgroup barrier, so the
// next item may reuse the LDS at once.
template <int D>
__device__ __forceinline__ void attn_item(AttnSmem<D>& sm, const Dims& dm, const Tables& tb, char* ws,
                                          const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                          const bf16_t* __restrict__ v, bf16_t* __restrict__ o,
                                          float* __restrict__ lse, uint32_t item) {
  constexpr int KS = AttnSmem<D>::KS, VS = AttnSmem<D>::VS, NC = D / 32, ND = D / 16;
  const int bh = (int)(item >> 16), t = (int)(item & 0xffff);
  const HeadDev& H = wsp<const HeadDev>(ws, tb.off_heads)[bh];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 15, g4 = lane >> 4;
  if (wsp<const int4>(ws, H.ws_info)[t].w <= 0) return;   // a tile of padding rows only (uniform)

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
  const int view_rows = 64 * H.nT_view;
  const int32_t* pgrp = wsp<const int32_t>(ws, dm.ws_pgrp);
  const bf16_t* kg = k + H.k_off;
  const bf16_t* vg = v + H.v_off;
  const bool ashape = H.pattern == MMSA_ASHAPE;
  const int sink = H.sink, window = H.window;
  const int n_chunks = n_tiles + (g_cnt + 63) / 64;
  const int last_row = dm.L - 1;

  // ---- staging registers ----
  // K: a thread moves 16-byte chunk kc of rows kr0 + j*KRP (coalesced row reads,
  //    bank-conflict-free row-major LDS stores).
  // V: a thread moves d-chunk vdc of key quad vkq (4 rows), transposes the 4x8
  //    block in registers and stores 8-byte runs of 4 keys; lanes of one store
  //    instruction vary over 16 key quads x 2 d-rows, which hit distinct banks.
  // Loads are unconditional: a row without a token reads a real (finite) row
  // through a clamped address and is masked by its key position.
  constexpr int VDC = D / 8;            // 16-byte d-chunks per row
  constexpr int KRP = 256 / VDC;        // rows per K pass
  constexpr int KCH = 64 / KRP;         // K passes (rows per thread)
  uint4 kreg[KCH];
  uint4 vreg[4];
  int kpreg = KPOS_NONE;
  const int kc = tid % VDC, kr0 = tid / VDC;
  const int vkq = lane & 15, vdc = 4 * w + (lane >> 4);
  const bool v_active = (D == 128) || w < 2;   // wave-uniform

  auto load_tile = [&](int c) {          // key tile c of the head's key view
    const int r0 = 64 * c;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      int vr = r0 + kr0 + KRP * j;
      vr = grouped_view ? vr : min(vr, last_row);
      kreg[j] = ld16(kview + (int64_t)vr * kv_sl + 8 * kc);
    }
    if (v_active) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int vr = r0 + 4 * vkq + rr;
        vr = grouped_view ? vr : min(vr, last_row);
        vreg[rr] = ld16(vview + (int64_t)vr * vv_sl + 8 * vdc);
      }
    }
    if (w == 0) {
      const int vr = r0 + lane;
      int pos;
      if (grouped_view) pos = pgrp[min(vr, view_rows - 1)];
      else pos = vr < dm.L ? vr : -1;
      kpreg = pos >= 0 ? pos : KPOS_NONE;
    }
  };
  auto load_gather = [&](int n) {        // gathered key columns 64n .. 64n+63
    const int e0 = 64 * n, el = g_cnt - 1;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      const int p = glist[min(e0 + kr0 + KRP * j, el)];
      kreg[j] = ld16(kg + (int64_t)p * dm.k_sl + 8 * kc);
    }
    if (v_active) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int p = glist[min(e0 + 4 * vkq + rr, el)];
        vreg[rr] = ld16(vg + (int64_t)p * dm.v_sl + 8 * vdc);
      }
    }
    if (w == 0) kpreg = (e0 + lane <= el) ? glist[e0 + lane] : KPOS_NONE;
  };
  auto load_chunk = [&](int kind, int idx) {
    if (kind == 0) load_tile(idx);
    else load_gather(idx);
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) st16(sm.K[buf] + (kr0 + KRP * j) * KS + 8 * kc, kreg[j]);
    if (v_active) {
      const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
      bf16_t* vd = sm.Vt[buf] + (8 * vdc) * VS + vt_slot(vkq);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint2 lo, hi;
        lo.x = __builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(w3[m], w2[m], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(w3[m], w2[m], 0x07060302u);
        *reinterpret_cast<uint2*>(vd + (2 * m) * VS) = lo;
        *reinterpret_cast<uint2*>(vd + (2 * m + 1) * VS) = hi;
      }
    }
    if (w == 0) sm.kp[buf][lane] = kpreg;
  };

  // tile iteration over the bitmap (uniform across the workgroup)
  auto uload64 = [&](int i) -> uint64_t {   // a bitmap word, known uniform
    const uint64_t x = bmrow[i];
    return ((uint64_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  };
  int wi = 0;
  uint64_t bits = W > 0 ? uload64(0) : 0ull;
  auto next_desc = [&](int ci, int& kind, int& idx) {
    if (ci < n_tiles) {
      while (bits == 0ull && wi + 1 < W) bits = uload64(++wi);
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
      pk[e >> 1] = pack_bf2_hw(p0, p1);
    }
    l_run = l_run * corr + psum;
    if (__builtin_amdgcn_read_exec() & __ballot(corr != 1.0f)) {   // some row's max moved (wave-uniform test)
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db] *= corr;
    }
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
      pkd.x = pack_bf2_hw(oacc[db][0] * inv, oacc[db][1] * inv);
      pkd.y = pack_bf2_hw(oacc[db][2] * inv, oacc[db][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * db + 4 * g4) = pkd;
    }
    if (lse != nullptr && g4 == 0) {
      const float val = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      lse[((int64_t)H.b * dm.Hq + H.h) * dm.L + qpos] = val;
    }
  }
}

// Persistent workgroups: workgroup i drains the queue segment of XCD i % 8
// (items popped with an atomic counter), then helps the other segments.
// Every workgroup exits once all segments are empty.
template <int D>
__global__ __launch_bounds__(256, 2) void k_attn(Dims dm, Tables tb, char* ws, const bf16_t* __restrict__ q,
                                                 const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                 bf16_t* __restrict__ o, float* __restrict__ lse) {
  __shared__ AttnSmem<D> sm;
  __shared__ int sh_j;
  const int64_t* seg = wsp<const int64_t>(ws, dm.ws_seg);
  int32_t* ctr = reinterpret_cast<int32_t*>(wsp<int64_t>(ws, dm.ws_seg) + N_XCD + 1);
  const int32_t* items = wsp<const int32_t>(ws, dm.ws_enum_item);
  const int x0 = blockIdx.x % N_XCD;
  for (int s = 0; s < N_XCD; ++s) {
    const int x = (x0 + s) % N_XCD;
    const int64_t beg = seg[x], end = seg[x + 1];
    while (true) {
      if (threadIdx.x == 0) sh_j = atomicAdd(&ctr[x], 1);
      __syncthreads();
      // the popped index is the same in every lane; saying so keeps the item's
      // descriptors in scalar registers and its control flow uniform
      const int64_t e = beg + __builtin_amdgcn_readfirstlane(sh_j);
      __syncthreads();
      if (e >= end) break;
      const uint32_t item = (uint32_t)__builtin_amdgcn_readfirstlane(items[e]);
      attn_item<D>(sm, dm, tb, ws, q, k, v, o, lse, item);
    }
  }
}

hipError_t launch_attention(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k, const void* v,
                            void* o, float* lse, int n_workgroups, hipStream_t s) {
  if (dm.n_items <= 0 || n_workgroups <= 0) return hipSuccess;
  if (dm.d == 128)
    k_attn<128><<<(unsigned)n_workgroups, 256, 0, s>>>(dm, tb, ws, (const bf16_t*)q, (const bf16_t*)k,
                                                        (const bf16_t*)v, (bf16_t*)o, lse);
  else
    k_attn<64><<<(unsigned)n_workgroups, 256, 0, s>>>(dm, tb, ws, (const bf16_t*)q, (const bf16_t*)k,
                                                       (const bf16_t*)v, (bf16_t*)o, lse);
  return hipGetLastError();
}

}  // namespace mmsa
