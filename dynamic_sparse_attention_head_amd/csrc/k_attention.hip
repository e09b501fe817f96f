// Block-sparse causal prefill over the planned key tiles and gathered columns
// (MMInference verdict page, key_machinery: FlashAttention-style kernels that
// load only the permuted blocks and keep matrix-core compute dense; the online
// softmax is the FlashAttention-2 recurrence those kernels build on).
//
// One workgroup = one pair of adjacent 64-row query tiles of one head (128
// rows), 4 waves x 32 rows.  Key chunks of 64 (a whole view tile, or 64
// gathered columns) are staged once in LDS for both tiles: K row-major, V
// transposed (d-major, keys in MFMA k-slot order).  The staged chunks are the
// union of the two tiles' plans; a wave computes only the chunks its own tile
// selected.  Both products run as bf16 32x32x16 MFMA with fp32 accumulation:
//   S^T (keys x queries) = K . Q^T     -> each lane holds one query's 32 logits
//   O^T (d x queries)   += V^T . P^T   -> each lane holds one query's outputs
// With these layouts a lane owns one query row throughout, so the online
// softmax needs one cross-lane exchange per chunk and its rescale is a per-lane
// scalar.  32 query rows per wave make every LDS fragment feed two 16-row
// blocks' worth of MFMA work, and 128 rows per workgroup halve the K/V bytes
// staged per FLOP.  Staging is double-buffered: the next chunk's global loads
// are in flight while the current chunk is computed.  Masking is element-wise
// on original positions (causal, A-shape window) and is skipped for chunks
// whose keys all precede the wave's first row.
#include "mmsa_device.h"

namespace mmsa {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).  Lane l: A row l%32, k-slots
// 8*(l/32)..+8; B column l%32, same k-slots; D column l%32, rows 8i+4(l/32)+j
// held at index 4i+j.
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct AttnSmem {  // 2 stages of K (row-major), V^T (d-major), key positions and their max
  static constexpr int KS = D + 8;    // K row stride (elements)
  static constexpr int VS = 64 + 8;   // V^T row stride (elements)
  bf16_t K[2][64 * KS];
  bf16_t Vt[2][D * VS];
  int kp[2][64];
  int kmax[2];
};

// V^T slot of the first key of key quad kq (keys 4kq..4kq+3).  Within each
// 16-key MFMA step, k-slots 8h..8h+7 of lane half h hold keys {4h..4h+3,
// 8+4h..8+4h+3}, the keys that half holds in the S^T accumulator.
__device__ __forceinline__ int vt_slot(int kq) { return 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq >> 1) & 1); }

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

constexpr uint32_t OOB = 0x80000000u;   // a buffer offset past every tensor slice
constexpr float LAZY_LOG2 = 8.0f;       // stale-max slack of the online softmax (log2 units)
__device__ constexpr bf16x2_t ONES_BF2 = {(__bf16)1.0f, (__bf16)1.0f};

// One (head, query-tile pair) work item.  Ends with a workgroup barrier, so the
// next item may reuse the LDS at once.
template <int D>
__device__ __forceinline__ void attn_pair(AttnSmem<D>& sm, const Dims& dm, const Tables& tb, char* ws,
                                          const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                          const bf16_t* __restrict__ v, bf16_t* __restrict__ o,
                                          float* __restrict__ lse, uint32_t item) {
  constexpr int KS = AttnSmem<D>::KS, VS = AttnSmem<D>::VS, NS = D / 16, ND = D / 32;
  const int bh = (int)(item >> 16), pr = (int)(item & 0xffff);
  const MMSA_CONST HeadDev& H = cptr<HeadDev>(ws, tb.off_heads)[bh];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, qc = lane & 31, hh = lane >> 5;
  const int t0 = 2 * pr, t1 = 2 * pr + 1;
  const bool has1 = t1 < H.nT_rows;
  const MMSA_CONST int32_t* inf0 = cptr<int32_t>(ws, H.ws_info) + 4 * t0;   // tiles, gathered, cost, rows
  const MMSA_CONST int32_t* inf1 = cptr<int32_t>(ws, H.ws_info) + 4 * (has1 ? t1 : t0);
  const int rows0 = inf0[3], rows1 = has1 ? inf1[3] : 0;
  if (rows0 <= 0 && rows1 <= 0) return;   // padding tiles only

  // ---- query rows of this wave (B operand of S^T) ----
  const int myt = w < 2 ? t0 : t1;
  const bool wave_has = (w < 2) ? rows0 > 0 : rows1 > 0;   // wave-uniform
  const int slot = 64 * myt + 32 * (w & 1) + qc;
  int qpos = -1;
  if (wave_has) {
    if (H.row_kind == ROW_IDENTITY) qpos = slot < dm.L ? slot : -1;
    else qpos = wsp<const int32_t>(ws, H.ws_row_order)[slot];
  }
  bf16x8 qf[NS];
  {
    const bf16_t* qrow = (H.ws_qperm >= 0) ? wsp<const bf16_t>(ws, H.ws_qperm) + (int64_t)slot * D
                                           : q + H.q_off + (int64_t)(qpos < 0 ? 0 : qpos) * dm.q_sl;
    uint4 u[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u[s] = make_uint4(0, 0, 0, 0);
      if (qpos >= 0) u[s] = ld16(qrow + 16 * s + 8 * hh);
    }
    // Consume the fragments here, once: afterwards they are plain register values,
    // not loads in flight, so the chunk loop never has to wait for them (a wait
    // there would also wait for the next chunk's prefetch and serialise it).
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      asm volatile("" : "+v"(u[s].x), "+v"(u[s].y), "+v"(u[s].z), "+v"(u[s].w));
      qf[s] = as_bf16x8(u[s]);
    }
  }
  // smallest valid query position of the wave: chunks whose keys all precede it need no mask
  int wq = qpos >= 0 ? qpos : 0x7fffffff;
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) wq = min(wq, __shfl_xor(wq, m, 64));
  const int wave_qmin = uniform(wq);

  // ---- plan of the pair ----
  const int W = H.bm_words;
  const bool grid = H.pattern == MMSA_GRID;
  const int g_cap = grid ? dm.L : H.gcap;
  // clamped to the buffers' capacities (a plan that was never built stays in bounds)
  const int g0 = rows0 > 0 ? min(max(inf0[1], 0), g_cap) : 0;
  const int g1 = rows1 > 0 ? min(max(inf1[1], 0), g_cap) : 0;
  const MMSA_CONST uint64_t* bm0 = cptr<uint64_t>(ws, H.ws_bm) + (int64_t)t0 * W;
  const MMSA_CONST uint64_t* bm1 = cptr<uint64_t>(ws, H.ws_bm) + (int64_t)(has1 ? t1 : t0) * W;
  const bool use0 = rows0 > 0, use1 = rows1 > 0;
  int n_union = 0;
  for (int i = 0; i < W; ++i) n_union += __popcll((use0 ? bm0[i] : 0ull) | (use1 ? bm1[i] : 0ull));
  // gathered columns: grid tiles share one ascending list (prefixes of it);
  // vertical-slash tiles each have their own list
  const int32_t* gl0 = nullptr;
  const int32_t* gl1 = nullptr;
  if (grid) {
    gl0 = gl1 = wsp<const int32_t>(ws, H.ws_row_order);
  } else if (H.gcap > 0) {
    gl0 = wsp<const int32_t>(ws, H.ws_gather) + (int64_t)t0 * H.gcap;
    gl1 = wsp<const int32_t>(ws, H.ws_gather) + (int64_t)(has1 ? t1 : t0) * H.gcap;
  }
  const int nch0 = (g0 + 63) / 64, nch1 = (g1 + 63) / 64;
  const int n_gath = grid ? max(nch0, nch1) : nch0 + nch1;
  const int n_chunks = n_union + n_gath;
  const bool grouped_view = H.view_kind == VIEW_GROUPED;
  const int32_t* pgrp = wsp<const int32_t>(ws, dm.ws_pgrp);
  const bool ashape = H.pattern == MMSA_ASHAPE;
  const int sink = H.sink, window = H.window;

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
  int kpreg = -1;
  const int kc = tid % VDC, kr0 = tid / VDC;
  const int vkq = lane & 15, vdc = 4 * w + (lane >> 4);
  const bool v_active = (D == 128) || w < 2;   // wave-uniform
  uint32_t kvoff[KCH], vvoff[4];
#pragma unroll
  for (int j = 0; j < KCH; ++j) kvoff[j] = (uint32_t)(kr0 + KRP * j) * rb_view + 16u * kc;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) vvoff[rr] = (uint32_t)(4 * vkq + rr) * rbv_view + 16u * vdc;

  // A chunk is staged in two halves so that only one half's registers are live
  // at a time: V (and the key positions) are loaded when the chunk is chosen and
  // stored at the end of the iteration; K is loaded after the current chunk's
  // S^T products and stored right after them.
  auto loadv_tile = [&](int c) {         // key tile c of the head's key view
    const uint32_t sv = (uint32_t)(64 * c) * rbv_view;
    if (v_active) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) vreg[rr] = bload16(rv_view, vvoff[rr], sv);
    }
    if (w == 0) {   // raw position; -1 (no token) becomes KPOS_NONE at store time
      const int vr = 64 * c + lane;
      if (grouped_view) kpreg = pgrp[min(vr, view_rows - 1)];
      else kpreg = vr < dm.L ? vr : -1;
    }
  };
  auto loadk_tile = [&](int c) {
    const uint32_t sk = (uint32_t)(64 * c) * rb_view;
#pragma unroll
    for (int j = 0; j < KCH; ++j) kreg[j] = bload16(rk_view, kvoff[j], sk);
  };
  // gathered columns 64n .. 64n+63 of a list: indices first (clamped,
  // unconditional, so they issue back to back), then rows
  auto loadv_gather = [&](const int32_t* glist, int cnt, int n) {
    const int e0 = 64 * n, el = cnt - 1;
    int pv[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) pv[rr] = glist[min(e0 + 4 * vkq + rr, el)];
    const int p3 = glist[min(e0 + lane, el)];
    if (v_active) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        vreg[rr] = bload16(rv, e0 + 4 * vkq + rr <= el ? (uint32_t)pv[rr] * rbv + 16u * vdc : OOB, 0);
    }
    if (w == 0) kpreg = (e0 + lane <= el) ? p3 : -1;
  };
  auto loadk_gather = [&](const int32_t* glist, int cnt, int n) {
    const int e0 = 64 * n, el = cnt - 1;
    int pk[KCH];
#pragma unroll
    for (int j = 0; j < KCH; ++j) pk[j] = glist[min(e0 + kr0 + KRP * j, el)];
#pragma unroll
    for (int j = 0; j < KCH; ++j)
      kreg[j] = bload16(rk, e0 + kr0 + KRP * j <= el ? (uint32_t)pk[j] * rbk + 16u * kc : OOB, 0);
  };
  auto storek = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KCH; ++j) st16(sm.K[buf] + (kr0 + KRP * j) * KS + 8 * kc, kreg[j]);
  };
  auto storev = [&](int buf) {
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
      const int kpos = kpreg >= 0 ? kpreg : KPOS_NONE;
      sm.kp[buf][lane] = kpos;
      int mx = kpos;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) mx = max(mx, __shfl_xor(mx, m, 64));
      if (lane == 0) sm.kmax[buf] = mx;
    }
  };

  // Chunk sequence (uniform across the workgroup): the union of both tiles'
  // key tiles, highest first -- workgroups on neighbouring query tiles then
  // stream the same key tiles at about the same time and share them in L2, and
  // the diagonal (the only chunk a causal tile needs masked) comes first -- then
  // the gathered columns.  The returned bits say which tiles (bit 0: first,
  // bit 1: second) selected the chunk.
  int wi = W;
  uint64_t bits = 0, wb0 = 0, wb1 = 0;
  // chunk ci -> (source: -1 tile / 0 first list / 1 second list, index, membership bits)
  auto next_chunk = [&](int ci, int& src, int& idx) -> int {
    if (ci < n_union) {
      while (bits == 0ull && wi > 0) {
        --wi;
        wb0 = use0 ? bm0[wi] : 0ull;
        wb1 = use1 ? bm1[wi] : 0ull;
        bits = wb0 | wb1;
      }
      const int b = bits ? 63 - __clzll((long long)bits) : -1;
      bits &= ~(1ull << (b & 63));
      src = -1;
      idx = b < 0 ? (view_rows + 63) / 64 : 64 * wi + b;   // (b < 0 only for a corrupt plan)
      return b < 0 ? 0 : (int)(((wb0 >> b) & 1ull) | (((wb1 >> b) & 1ull) << 1));
    }
    const int n = ci - n_union;
    if (grid) {
      src = 0;
      idx = n;
      return (64 * n < g0 ? 1 : 0) | (64 * n < g1 ? 2 : 0);
    }
    if (n < nch0) {
      src = 0;
      idx = n;
      return 1;
    }
    src = 1;
    idx = n - nch0;
    return 2;
  };
  const int gcnt0 = grid ? max(g0, g1) : g0;
  auto loadv = [&](int src, int idx) {
    if (src < 0) loadv_tile(idx);
    else if (src == 0) loadv_gather(gl0, gcnt0, idx);
    else loadv_gather(gl1, g1, idx);
  };
  auto loadk = [&](int src, int idx) {
    if (src < 0) loadk_tile(idx);
    else if (src == 0) loadk_gather(gl0, gcnt0, idx);
    else loadk_gather(gl1, g1, idx);
  };

  floatx16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = dm.scale_log2;
  const int wbit = w < 2 ? 1 : 2;

  int memb_cur = 0;
  if (n_chunks > 0) {
    int src, idx;
    memb_cur = next_chunk(0, src, idx);
    loadv(src, idx);
    loadk(src, idx);
    storek(0);
    storev(0);
    __syncthreads();
  }
  // LDS fragment reads are software-pipelined PF ahead of the MFMAs that use
  // them; scheduling barriers pin that order (the scheduler would otherwise
  // pair each read with its MFMA and expose every read's latency).
  constexpr int PF = 4, NK = 2 * NS, NV = 4 * ND;
  for (int ci = 0; ci < n_chunks; ++ci) {
    const int buf = ci & 1;
    const bool has_next = ci + 1 < n_chunks;
    int memb_next = 0;
    if (has_next) {
      int nsrc, nidx;
      memb_next = next_chunk(ci + 1, nsrc, nidx);
      loadv(nsrc, nidx);
      loadk(nsrc, nidx);
    }
    const bool mine = wave_has && (memb_cur & wbit);
    floatx16 sacc[2];
    if (mine) {
      // ---- S^T = K . Q^T (fragment i: key block i&1, d-step i>>1) ----
      const bf16_t* Kb = sm.K[buf] + qc * KS + 8 * hh;
      auto kfrag = [&](int i) { return as_bf16x8(ld16(Kb + 32 * (i & 1) * KS + 16 * (i >> 1))); };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
      bf16x8 af[NK];
#pragma unroll
      for (int i = 0; i < PF; ++i) af[i] = kfrag(i);
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + PF < NK) af[i + PF] = kfrag(i + PF);
        sacc[i & 1] = mfma32(af[i], qf[i >> 1], sacc[i & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (has_next) storek(buf ^ 1);
    if (mine) {
      // first V^T fragments in flight during the softmax (fragment i: d-block i%ND, key step i/ND)
      const bf16_t* Vb = sm.Vt[buf] + qc * VS + 8 * hh;
      auto vfrag = [&](int i) { return as_bf16x8(ld16(Vb + 32 * (i % ND) * VS + 16 * (i / ND))); };
      bf16x8 vf[NV];
#pragma unroll
      for (int i = 0; i < PF; ++i) vf[i] = vfrag(i);
      __builtin_amdgcn_sched_barrier(0);
      // ---- mask (only chunks crossing the causal edge, or A-shape), online softmax ----
      const bool full = !ashape && uniform(sm.kmax[buf]) <= wave_qmin;
      if (!full) {
        // branch-free selects (bitwise boolean ops, no short-circuit evaluation)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int4 kk = *reinterpret_cast<const int4*>(&sm.kp[buf][32 * kb + 8 * i + 4 * hh]);
            const int kpv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              bool ok = kpv[j] <= qpos;
              if (ashape) ok = ok & ((kpv[j] < sink) | (qpos - kpv[j] < window));
              sacc[kb][4 * i + j] = ok ? sacc[kb][4 * i + j] : -INFINITY;
            }
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(sacc[kb][e], sacc[kb][e + 1]));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      // Lazy rescale: the running max moves (and O, l are rescaled) only when
      // some row's max grows by more than 2^LAZY; otherwise probabilities are
      // taken against the stale max and stay below 2^LAZY.
      const float m_cand = fmaxf(m_run, mx * sl2);
      if (__ballot(m_cand > m_run + LAZY_LOG2)) {
        const float m_use = (m_cand == -INFINITY) ? 0.f : m_cand;
        const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_cand;
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db] *= corr;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      uint32_t pk[16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e], sl2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e + 1], sl2, -m_use));
          pk[8 * kb + (e >> 1)] = pack_bf2_hw(p0, p1);
        }
      }
      // row sum of the bf16-rounded probabilities, the values the MFMA consumes
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[e]), ONES_BF2, psum, false);
      l_run += psum;
      __builtin_amdgcn_sched_barrier(0);
      // ---- O^T += V^T . P^T ----
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + PF < NV) vf[i + PF] = vfrag(i + PF);
        const int st = i / ND;   // 16-key step: accumulator values 8(st&1).. of key block st>>1
        const bf16x8 pb = as_bf16x8(make_uint4(pk[4 * st], pk[4 * st + 1], pk[4 * st + 2], pk[4 * st + 3]));
        oacc[i % ND] = mfma32(vf[i], pb, oacc[i % ND]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (has_next) storev(buf ^ 1);
    memb_cur = memb_next;
    __syncthreads();
  }

  // ---- epilogue ----
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if (qpos >= 0) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    bf16_t* orow = (H.ws_operm >= 0) ? wsp<bf16_t>(ws, H.ws_operm) + (int64_t)slot * D
                                     : o + H.o_off + (int64_t)qpos * dm.o_sl;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 pkd;
        pkd.x = pack_bf2_hw(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv);
        pkd.y = pack_bf2_hw(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * db + 8 * i + 4 * hh) = pkd;
      }
    }
    if (lse != nullptr && hh == 0) {
      const float val = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      lse[((int64_t)H.b * dm.Hq + H.h) * dm.L + qpos] = val;
    }
  }
}

// Persistent workgroups: a workgroup drains the queue segment of its own XCD
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
  // this workgroup's XCD (hardware XCC id), so its L2 serves its segment
  const int x0 = (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (N_XCD - 1));
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
      attn_pair<D>(sm, dm, tb, ws, q, k, v, o, lse, item);
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
