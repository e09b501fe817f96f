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
struct AttnSmem {  // 2 stages of K (row-major), V^T (d-major), key positions and their max
  static constexpr int KS = D + 8;    // K row stride (elements)
  static constexpr int VS = 64 + 8;   // V^T row stride (elements)
  bf16_t K[2][64 * KS];
  bf16_t Vt[2][D * VS];
  int kp[2][64];
  int kmax[2];
};

// k-slot of the first key of key-quad kq (4 consecutive keys) inside V^T rows
__device__ __forceinline__ int vt_slot(int kq) {
  const int c = kq >> 3, q = kq & 7;
  return 32 * c + (q < 4 ? 8 * q : 8 * (q - 4) + 4);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

constexpr uint32_t OOB = 0x80000000u;   // a buffer offset past every tensor slice

// One (head, query tile) work item.  Ends with a workgroup barrier, so the
// next item may reuse the LDS at once.
template <int D>
__device__ __forceinline__ void attn_item(AttnSmem<D>& sm, const Dims& dm, const Tables& tb, char* ws,
                                          const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                          const bf16_t* __restrict__ v, bf16_t* __restrict__ o,
                                          float* __restrict__ lse, uint32_t item) {
  constexpr int KS = AttnSmem<D>::KS, VS = AttnSmem<D>::VS, NC = D / 32, ND = D / 16;
  const int bh = (int)(item >> 16), t = (int)(item & 0xffff);
  const MMSA_CONST HeadDev& H = cptr<HeadDev>(ws, tb.off_heads)[bh];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 15, g4 = lane >> 4;
  const MMSA_CONST int32_t* info = cptr<int32_t>(ws, H.ws_info) + 4 * t;   // tiles, gathered, cost, rows
  if (info[3] <= 0) return;   // a tile of padding rows only

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
  // smallest valid query position of the wave: chunks whose keys all precede it need no mask
  int wq = qpos >= 0 ? qpos : 0x7fffffff;
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) wq = min(wq, __shfl_xor(wq, m, 64));
  const int wave_qmin = uniform(wq);

  // ---- plan of this tile ----
  const int W = H.bm_words;
  // clamped to the buffers' capacities (a plan that was never built stays in bounds)
  const int n_tiles = min(max(info[0], 0), 64 * W);
  const int g_cap = (H.pattern == MMSA_GRID) ? dm.L : H.gcap;
  const int g_cnt = min(max(info[1], 0), g_cap);
  const MMSA_CONST uint64_t* bmrow = cptr<uint64_t>(ws, H.ws_bm) + (int64_t)t * W;
  const int32_t* glist = nullptr;
  if (H.pattern == MMSA_GRID) glist = wsp<const int32_t>(ws, H.ws_row_order);
  else if (H.gcap > 0) glist = wsp<const int32_t>(ws, H.ws_gather) + (int64_t)t * H.gcap;
  const bool grouped_view = H.view_kind == VIEW_GROUPED;
  const int32_t* pgrp = wsp<const int32_t>(ws, dm.ws_pgrp);
  const bool ashape = H.pattern == MMSA_ASHAPE;
  const int sink = H.sink, window = H.window;
  const int n_chunks = n_tiles + (g_cnt + 63) / 64;

  // buffer views: the head's key view (tiles) and its original K/V (gathered columns)
  const uint32_t rb_view = grouped_view ? 2u * D : 2u * (uint32_t)dm.k_sl;
  const uint32_t rbv_view = grouped_view ? 2u * D : 2u * (uint32_t)dm.v_sl;
  const uint32_t rbk = 2u * (uint32_t)dm.k_sl, rbv = 2u * (uint32_t)dm.v_sl;
  const int view_rows = grouped_view ? dm.L_grp : dm.L;
  const __amdgpu_buffer_rsrc_t rk_view =
      make_rsrc(grouped_view ? (const void*)wsp<const bf16_t>(ws, H.ws_kgrp) : (const void*)(k + H.k_off),
                (uint32_t)(view_rows - 1) * rb_view + 2u * D);
  const __amdgpu_buffer_rsrc_t rv_view =
      make_rsrc(grouped_view ? (const void*)wsp<const bf16_t>(ws, H.ws_vgrp) : (const void*)(v + H.v_off),
                (uint32_t)(view_rows - 1) * rbv_view + 2u * D);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + H.k_off, (uint32_t)(dm.L - 1) * rbk + 2u * D);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + H.v_off, (uint32_t)(dm.L - 1) * rbv + 2u * D);

  // ---- staging ----
  // K: a thread moves 16-byte chunk kc of rows kr0 + j*KRP (coalesced row reads,
  //    bank-conflict-free row-major LDS stores).
  // V: a thread moves d-chunk vdc of key quad vkq (4 rows), transposes the 4x8
  //    block in registers and stores 8-byte runs of 4 keys; lanes of one store
  //    instruction vary over 16 key quads x 2 d-rows, which hit distinct banks.
  // Rows past the end of a view read zeros (buffer bounds) and carry no position.
  constexpr int VDC = D / 8;            // 16-byte d-chunks per row
  constexpr int KRP = 256 / VDC;        // rows per K pass
  constexpr int KCH = 64 / KRP;         // K passes (rows per thread)
  uint4 kreg[KCH];
  uint4 vreg[4];
  int kpreg = KPOS_NONE;
  const int kc = tid % VDC, kr0 = tid / VDC;
  const int vkq = lane & 15, vdc = 4 * w + (lane >> 4);
  const bool v_active = (D == 128) || w < 2;   // wave-uniform
  uint32_t kvoff[KCH], vvoff[4];
#pragma unroll
  for (int j = 0; j < KCH; ++j) kvoff[j] = (uint32_t)(kr0 + KRP * j) * rb_view + 16u * kc;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) vvoff[rr] = (uint32_t)(4 * vkq + rr) * rbv_view + 16u * vdc;

  auto load_tile = [&](int c) {          // key tile c of the head's key view
    const uint32_t sk = (uint32_t)(64 * c) * rb_view, sv = (uint32_t)(64 * c) * rbv_view;
#pragma unroll
    for (int j = 0; j < KCH; ++j) kreg[j] = bload16(rk_view, kvoff[j], sk);
    if (v_active) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) vreg[rr] = bload16(rv_view, vvoff[rr], sv);
    }
    if (w == 0) {
      const int vr = 64 * c + lane;
      int pos;
      if (grouped_view) pos = vr < view_rows ? pgrp[vr] : -1;
      else pos = vr < dm.L ? vr : -1;
      kpreg = pos >= 0 ? pos : KPOS_NONE;
    }
  };
  auto load_gather = [&](int n) {        // gathered key columns 64n .. 64n+63
    // indices first (clamped, unconditional, so they issue back to back), then rows
    const int e0 = 64 * n, el = g_cnt - 1;
    int pk[KCH], pv[4];
#pragma unroll
    for (int j = 0; j < KCH; ++j) pk[j] = glist[min(e0 + kr0 + KRP * j, el)];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) pv[rr] = glist[min(e0 + 4 * vkq + rr, el)];
    const int p3 = glist[min(e0 + lane, el)];
#pragma unroll
    for (int j = 0; j < KCH; ++j)
      kreg[j] = bload16(rk, e0 + kr0 + KRP * j <= el ? (uint32_t)pk[j] * rbk + 16u * kc : OOB, 0);
    if (v_active) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        vreg[rr] = bload16(rv, e0 + 4 * vkq + rr <= el ? (uint32_t)pv[rr] * rbv + 16u * vdc : OOB, 0);
    }
    if (w == 0) kpreg = (e0 + lane <= el) ? p3 : KPOS_NONE;
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
    if (w == 0) {
      sm.kp[buf][lane] = kpreg;
      int mx = kpreg;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) mx = max(mx, __shfl_xor(mx, m, 64));
      if (lane == 0) sm.kmax[buf] = mx;
    }
  };

  // tile iteration over the bitmap (uniform across the workgroup)
  auto uload64 = [&](int i) -> uint64_t { return bmrow[i]; };
  int wi = 0;
  uint64_t bits = W > 0 ? uload64(0) : 0ull;
  auto load_next = [&](int ci) {
    if (ci < n_tiles) {
      while (bits == 0ull && wi + 1 < W) bits = uload64(++wi);
      const int b = __ffsll((unsigned long long)bits) - 1;
      bits &= bits - 1;
      load_tile(b < 0 ? (view_rows + 63) / 64 : 64 * wi + b);   // (b < 0 only for a corrupt plan)
    } else {
      load_gather(ci - n_tiles);
    }
  };

  floatx4 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = dm.scale_log2;

  if (n_chunks > 0) {
    load_next(0);
    store_chunk(0);
    __syncthreads();
  }
  for (int ci = 0; ci < n_chunks; ++ci) {
    const int buf = ci & 1;
    const bool has_next = ci + 1 < n_chunks;
    if (has_next) load_next(ci + 1);
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
    // ---- mask (only chunks crossing the causal edge, or A-shape), online softmax ----
    const bool full = !ashape && uniform(sm.kmax[buf]) <= wave_qmin;
    if (!full) {
      // branch-free selects (bitwise boolean ops, no short-circuit evaluation)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int4 kk = *reinterpret_cast<const int4*>(&sm.kp[buf][16 * kb + 4 * g4]);
        const int kpv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bool ok = kpv[i] <= qpos;
          if (ashape) ok = ok & ((kpv[i] < sink) | (qpos - kpv[i] < window));
          sacc[kb][i] = ok ? sacc[kb][i] : -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      mx = fmaxf(fmaxf(fmaxf(mx, sacc[kb][0]), fmaxf(sacc[kb][1], sacc[kb][2])), sacc[kb][3]);
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 2][e & 3], sl2, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[(e + 1) >> 2][(e + 1) & 3], sl2, -m_use));
      psum += p0 + p1;
      pk[e >> 1] = pack_bf2_hw(p0, p1);
    }
    l_run = l_run * corr + psum;
    if (__ballot(corr != 1.0f)) {   // some row's max moved (wave-uniform test)
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
  const MMSA_CONST int64_t* seg = cptr<int64_t>(ws, dm.ws_seg);
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
