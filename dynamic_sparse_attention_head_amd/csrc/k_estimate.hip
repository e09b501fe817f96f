// Online index estimation for vertical-slash, boundary and grid heads.
//
// Pages: MInference 1.0 summary page, "Approach" (vertical and slash lines
// from the attention of the last 64 queries); MMInference verdict page,
// key_machinery (grid stride and phase found by scanning an approximate
// attention matrix of the last 64 queries) and pith_summary (index from the
// last 64 queries of each modality segment).
//
// The attention of the estimation rows is exact: pass 1 streams K once for the
// row max and the sum of exponentials, pass 2 streams K again and forms the
// normalised probabilities, their column sums (vertical scores) and their
// diagonal sums (slash scores).  Pass 1 workgroups stream key chunks of one
// KV head against up to four regions whose rows sit in LDS; a pass 2
// workgroup takes 256 keys and every region of its KV head.  Either way K is
// read about twice in total.  QK^T uses bf16 MFMA with fp32 accumulation.
// Diagonal sums cross workgroups; they are added as 2^-40 fixed-point
// integers, so the result does not depend on the order in which workgroups
// finish.
#include <type_traits>

#include "block_scan.h"

namespace mmsa {

// Merge two (max, sum of 2^(x - max)) pairs of one row (hardware exp2).
__device__ __forceinline__ float2 lse2_merge_hw(float2 a, float2 b) {
  if (a.x == -INFINITY) return b;
  if (b.x == -INFINITY) return a;
  const float m = fmaxf(a.x, b.x);
  return make_float2(m, a.y * __builtin_amdgcn_exp2f(a.x - m) + b.y * __builtin_amdgcn_exp2f(b.x - m));
}

// Max and sum over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48), in registers: v_permlane16_swap pairs rows 0-1 and 2-3, then
// v_permlane32_swap pairs the halves.  Every lane receives the result, and
// the pairs are combined symmetrically, so all four lanes agree bit for bit.
__device__ __forceinline__ float max_rows4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_rows4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The batch of a workgroup of a 1-D estimation launch: groups hold
// consecutive workgroup ranges [wg0, wg0 + nwg).  Returns the group's index
// and sets x to this workgroup's index within it.
__device__ __forceinline__ int est_group(const MMSA_CONST EstGroup* gs, int64_t n, int& x) {
  int lo = 0, hi = (int)n - 1;
  const int b = (int)blockIdx.x;
  while (lo < hi) {   // last group with wg0 <= b
    const int mid = (lo + hi + 1) >> 1;
    if (gs[mid].wg0 <= b) lo = mid;
    else hi = mid - 1;
  }
  x = b - gs[lo].wg0;
  return lo;
}

// Swizzle of the LDS copy of the estimation rows: physical 16-byte chunk =
// logical ^ swz1(row), so the 16 rows one B-fragment read touches fall in 16
// different bank groups (d = 128: 256-byte rows; d = 64: two 128-byte rows per
// 256 bytes).
template <int D>
__device__ __forceinline__ int swz1(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// ---------------------------------------------------------------------------
// Pass 1: (max, sum of exp2) of each estimation row over its causal keys.
// 1-D grid: each batch (at most EST1_JB jobs of one (b, KV head)) owns a range
// of workgroups, block 256 = 4 waves.  The batch's Q rows are copied into
// LDS once, straight from memory (16 bytes a lane).  Workgroup x of a batch's
// nwg takes the 256-key chunks x, x + nwg, ...: each wave owns 64
// keys of a chunk, held in registers while the next chunk's keys load into a
// second register set, and keeps a running (max, sum) per row in LDS.  At the
// end the workgroup merges its four waves into one partial per row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void k_est_pass1(Dims dm, Tables tb, char* ws, const bf16_t* __restrict__ q,
                                                      const bf16_t* __restrict__ k) {
  constexpr int NC = D / 32, CPR = D / 8, RPI = 64 / CPR, IPW = EST_ROWS / RPI / 4;
  constexpr int QJ = EST_ROWS * D * 2;   // bytes of one job's rows of Q
  __shared__ __attribute__((aligned(16))) char Qs[EST1_JB * QJ];
  __shared__ int pos_s[EST1_JB][EST_ROWS];
  __shared__ int minpos_s[EST1_JB];
  __shared__ float2 st_s[EST1_JB][4][EST_ROWS];
  int xw;
  const MMSA_CONST EstGroup* gs = cptr<EstGroup>(ws, tb.off_groups1);
  const MMSA_CONST EstGroup& G = gs[est_group(gs, tb.n_groups1, xw)];
  const MMSA_CONST EstJob* jobs = cptr<EstJob>(ws, tb.off_jobs) + G.job_begin;
  const int nj = min(G.job_end - G.job_begin, EST1_JB);
  const int tid = threadIdx.x, lane = tid & 63, qc = lane & 15, g4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int gimax = -1;
  for (int jj = 0; jj < nj; ++jj) gimax = max(gimax, jobs[jj].imax);
  const int n_ck = min((dm.L + EST_CK - 1) / EST_CK, gimax / EST_CK + 1);

  // ---- the batch's rows of Q into LDS; row positions; running stats ----
  // Copy instruction i of a job fills rows i*RPI .. +RPI-1; lane l writes row
  // i*RPI + l/CPR, physical chunk l%CPR, so it reads logical chunk
  // (l%CPR) ^ swz1(row).  Rows past n_rows repeat the last row (never used).
  for (int jj = 0; jj < nj; ++jj) {
    const MMSA_CONST EstJob& J = jobs[jj];
    if (tid < EST_ROWS) pos_s[jj][tid] = tid < J.n_rows ? J.rows[tid] : -1;
    st_s[jj][w][lane] = make_float2(-INFINITY, 0.f);
    const bf16_t* qh = q + J.q_off;
#pragma unroll
    for (int p = 0; p < IPW; ++p) {
      const int ins = w * IPW + p;
      const int row = ins * RPI + lane / CPR;
      const int lch = (lane % CPR) ^ swz1<D>(row);
      const int pos = J.n_rows > 0 ? J.rows[min(row, J.n_rows - 1)] : 0;
      __builtin_amdgcn_global_load_lds(qh + (int64_t)pos * dm.q_sl + 8 * lch,
                                       (__attribute__((address_space(3))) void*)(Qs + jj * QJ + ins * 1024), 16, 0,
                                       0);
    }
  }
  __syncthreads();
  // smallest row position of each job (-1 if it has padding rows): a wave's
  // 64 keys all at or before it need no causal mask
  if (tid < nj) {
    int mn = pos_s[tid][0];
    for (int r = 1; r < EST_ROWS; ++r) mn = min(mn, pos_s[tid][r]);
    minpos_s[tid] = mn;
  }

  // Keys past the end read the last row: they are masked, so their values never
  // count, and the loads stay unconditional (the compiler then waits for the
  // current chunk's loads only, not for the prefetch of the next).
  const bf16_t* kh = k + G.k_off;
  auto load_k = [&](bf16x8 (&kf)[4][NC], int c) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = min(c * EST_CK + 64 * w + 16 * kb + qc, dm.L - 1);
      const bf16_t* kr = kh + (int64_t)key * dm.k_sl + 8 * g4;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) kf[kb][cc] = as_bf16x8(ld16(kr + 32 * cc));
    }
  };
  const float sl2 = dm.scale_log2;
  // the 64 rows of one job against the wave's 64 keys (masked: causal mask on)
  auto job = [&](const bf16x8 (&kf)[4][NC], int jj, int kbase, auto masked) {
    const char* qt = Qs + jj * QJ;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int row = 16 * qb + qc;
      bf16x8 qf[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        qf[cc] = *reinterpret_cast<const bf16x8*>(qt + row * (2 * D) + 16 * ((4 * cc + g4) ^ swz1<D>(row)));
      const float2 o = st_s[jj][w][row];
      floatx4 acc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        acc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) acc[kb] = mfma16(kf[kb][cc], qf[cc], acc[kb]);
      }
      if constexpr (decltype(masked)::value) {
        const int pos = pos_s[jj][row];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[kb][i] = (kbase + 16 * kb + 4 * g4 + i <= pos) ? acc[kb][i] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mx = fmaxf(mx, fmaxf(fmaxf(acc[kb][0], acc[kb][1]), fmaxf(acc[kb][2], acc[kb][3])));
      mx = max_rows4(mx);
      const float m_new = fmaxf(o.x, mx * sl2);
      const float mu = m_new == -INFINITY ? 0.f : m_new;
      float sm = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm += __builtin_amdgcn_exp2f(fmaf(acc[kb][i], sl2, -mu));
      sm = sum_rows4(sm);
      const float s_new = o.y * __builtin_amdgcn_exp2f(o.x - mu) + sm;
      // the four lanes of a row hold the same values: all of them store (no branch)
      st_s[jj][w][row] = make_float2(m_new, s_new);
    }
  };
  // one chunk: every job of the batch whose rows see some of the wave's keys
  auto body = [&](const bf16x8 (&kf)[4][NC], int c) {
    const int kbase = c * EST_CK + 64 * w;
    for (int jj = 0; jj < nj; ++jj) {
      if (kbase > jobs[jj].imax) continue;   // uniform
      if (kbase + 63 <= __builtin_amdgcn_readfirstlane(minpos_s[jj]))
        job(kf, jj, kbase, std::false_type{});
      else
        job(kf, jj, kbase, std::true_type{});
    }
  };

  // The next chunk's keys are loaded unconditionally (past the end: the last
  // row again), so every path through the loop has the same loads in flight
  // and the compiler's waits cover only the chunk being computed.
  bf16x8 kA[4][NC], kB[4][NC];
  const int gx = G.nwg;
  int c = xw;
  load_k(kA, c);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the copies of Q and the first keys
  __syncthreads();
  while (c < n_ck) {
    load_k(kB, c + gx);
    body(kA, c);
    c += gx;
    if (c >= n_ck) break;
    load_k(kA, c + gx);
    body(kB, c);
    c += gx;
  }
  __syncthreads();
  for (int t = tid; t < nj * EST_ROWS; t += 256) {
    const int jj = t / EST_ROWS, r = t % EST_ROWS;
    float2 st = st_s[jj][0][r];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) st = lse2_merge_hw(st, st_s[jj][ww][r]);
    wsp<float2>(ws, jobs[jj].ws_part)[(int64_t)xw * EST_ROWS + r] = st;
  }
}

// Final (max, sum) per estimation row from the partials of its job (one per
// pass-1 workgroup of its batch): 16 waves each merge a contiguous range
// (lane = row), then the 16 results are merged.
__global__ __launch_bounds__(1024) void k_est_combine(Tables tb, char* ws) {
  const EstJob& J = wsp<const EstJob>(ws, tb.off_jobs)[blockIdx.x];
  const int n_part = J.n_part1;
  const int r = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float2* part = wsp<const float2>(ws, J.ws_part);
  const int per = (n_part + 15) / 16, c0 = wv * per, c1 = min(n_part, c0 + per);
  float2 st = make_float2(-INFINITY, 0.f);
  for (int c = c0; c < c1; ++c) st = lse2_merge_hw(st, part[(int64_t)c * 64 + r]);
  __shared__ float2 red[16][64];
  red[wv][r] = st;
  __syncthreads();
  if (wv == 0) {
    for (int w2 = 1; w2 < 16; ++w2) st = lse2_merge_hw(st, red[w2][r]);
    wsp<float2>(ws, J.ws_stats)[r] = st;
  }
}

// ---------------------------------------------------------------------------
// Pass 2: probabilities, column sums (v) and diagonal sums (s).
// 1-D grid: each batch (at most EST2_JB jobs sharing (b, KV head, key view))
// owns a range of workgroups, block 256 = 4 waves.  Like pass 1, workgroup x
// of a batch's nwg takes the 256-slot chunks x, x + nwg, ... with the rows of Q
// in LDS and the next chunk's keys loading into a second register set; the
// key positions are read into registers two chunks ahead.
// Per job, the normalised probabilities of 32 rows at a time go to an LDS
// tile whose rows carry 32 zero columns on either side: a diagonal then reads
// one entry per row at a constant stride, with no bounds test (a diagonal
// through 32 rows leaves the 256 keys by at most 31 columns).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void k_est_pass2(Dims dm, Tables tb, char* ws, const bf16_t* __restrict__ q,
                                                      const bf16_t* __restrict__ k) {
  constexpr int NC = D / 32, CPR = D / 8, RPI = 64 / CPR, IPW = EST_ROWS / RPI / 4;
  constexpr int QJ = EST_ROWS * D * 2;
  constexpr int HR = EST_ROWS / 2;          // rows of the probability tile
  constexpr int ZP = 32;                    // zero columns on either side
  constexpr int PW = EST_CK + 2 * ZP + 4;   // row pitch in floats (the 4 spread the rows over the banks)
  __shared__ __attribute__((aligned(16))) char Qs[EST2_JB * QJ];
  __shared__ __attribute__((aligned(16))) float P[HR][PW];
  __shared__ __attribute__((aligned(16))) int kp_s[2][EST_CK];   // key positions of the chunk (-1: no token)
  __shared__ int pos_s[EST2_JB][EST_ROWS];
  __shared__ float2 st_s[EST2_JB][EST_ROWS];   // (max, 1 / sum) of each row
  int xw;
  const MMSA_CONST EstGroup* gs = cptr<EstGroup>(ws, tb.off_groups2);
  const MMSA_CONST EstGroup& G = gs[est_group(gs, tb.n_groups2, xw)];
  const MMSA_CONST EstJob* jobs = cptr<EstJob>(ws, tb.off_jobs) + G.job_begin;
  const int nj = min(G.job_end - G.job_begin, EST2_JB);
  const int tid = threadIdx.x, lane = tid & 63, qc = lane & 15, g4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grouped = G.view == VIEW_GROUPED;
  // identity views: no chunk past the batch's last estimation row holds a
  // key any of its rows sees (grouped views order keys by modality first)
  int gimax = -1;
  for (int jj = 0; jj < nj; ++jj) gimax = max(gimax, jobs[jj].imax);
  const int n_ck = grouped ? (G.n_keys + EST_CK - 1) / EST_CK
                           : min((G.n_keys + EST_CK - 1) / EST_CK, gimax / EST_CK + 1);
  const int32_t* pgrp = wsp<const int32_t>(ws, dm.ws_pgrp);

  // ---- rows of Q into LDS (as in pass 1), row positions and statistics ----
  for (int jj = 0; jj < nj; ++jj) {
    const MMSA_CONST EstJob& J = jobs[jj];
    if (tid < EST_ROWS) {
      pos_s[jj][tid] = tid < J.n_rows ? J.rows[tid] : -1;
      const float2 st = wsp<const float2>(ws, J.ws_stats)[tid];
      st_s[jj][tid] = make_float2(st.x, st.y > 0.f ? 1.0f / st.y : 0.f);
    }
    const bf16_t* qh = q + J.q_off;
#pragma unroll
    for (int p = 0; p < IPW; ++p) {
      const int ins = w * IPW + p;
      const int row = ins * RPI + lane / CPR;
      const int lch = (lane % CPR) ^ swz1<D>(row);
      const int pos = J.n_rows > 0 ? J.rows[min(row, J.n_rows - 1)] : 0;
      __builtin_amdgcn_global_load_lds(qh + (int64_t)pos * dm.q_sl + 8 * lch,
                                       (__attribute__((address_space(3))) void*)(Qs + jj * QJ + ins * 1024), 16, 0,
                                       0);
    }
  }
  for (int i = tid; i < HR * 2 * ZP; i += 256) {   // the zero columns, never written again
    const int r = i / (2 * ZP), cz = i % (2 * ZP);
    P[r][cz < ZP ? cz : EST_CK + cz] = 0.f;
  }
  // Key positions of chunk c: those of the rows this lane loads (slots
  // 64w + 16kb + qc) and of this thread's own slot (-1: no token).  Identity
  // views compute them; grouped views read the slot map.
  struct Pos {
    int kb[4], own;
  };
  auto load_pos = [&](Pos& P, int c) {
    const int x0 = c * EST_CK, lim = min(G.n_keys, dm.L);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int slot = x0 + 64 * w + 16 * kb + qc;
      P.kb[kb] = grouped ? pgrp[min(slot, G.n_keys - 1)] : (slot < lim ? slot : -1);
    }
    const int slot = x0 + tid;
    P.own = grouped ? (slot < G.n_keys ? pgrp[slot] : -1) : (slot < lim ? slot : -1);
  };
  const bf16_t* kh = k + G.k_off;
  // keys of a chunk; slots without a token read row 0 (masked)
  auto load_k = [&](bf16x8 (&kf)[4][NC], const Pos& P) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bf16_t* kr = kh + (int64_t)max(P.kb[kb], 0) * dm.k_sl + 8 * g4;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) kf[kb][cc] = as_bf16x8(ld16(kr + 32 * cc));
    }
  };

  const float sl2 = dm.scale_log2;
  // one chunk (positions in kp_s[sl])
  auto body = [&](const bf16x8 (&kf)[4][NC], int c, int sl) {
    const int x0 = c * EST_CK;
    const int kmin = __builtin_amdgcn_readfirstlane(kp_s[sl][0]);   // smallest position (ascending; -1: empty)
    const int kpos_mine = kp_s[sl][tid];
    const int m_chunk = (grouped && x0 >= dm.video_base) ? MMSA_VIDEO : MMSA_TEXT;
    const int chunk_base = (m_chunk == MMSA_VIDEO) ? dm.video_base : dm.text_base;
    for (int jj = 0; jj < nj; ++jj) {
      const MMSA_CONST EstJob& J = jobs[jj];
      if (kmin < 0 || J.imax < kmin) continue;   // uniform
      const char* qt = Qs + jj * QJ;
      const bool slash = J.kind == JOB_VS_ORIG || J.kind == JOB_VS_2D;
      float colsum = 0.f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int h0 = HR * half;
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          const int row = h0 + 16 * qh + qc;
          bf16x8 qf[NC];
#pragma unroll
          for (int cc = 0; cc < NC; ++cc)
            qf[cc] = *reinterpret_cast<const bf16x8*>(qt + row * (2 * D) + 16 * ((4 * cc + g4) ^ swz1<D>(row)));
          const int pos = pos_s[jj][row];
          const float2 st = st_s[jj][row];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) acc = mfma16(kf[kb][cc], qf[cc], acc);
            const int4 kq = *reinterpret_cast<const int4*>(&kp_s[sl][64 * w + 16 * kb + 4 * g4]);
            const int kk[4] = {kq.x, kq.y, kq.z, kq.w};
            float4 pv;
            float* pp = reinterpret_cast<float*>(&pv);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool valid = kk[i] >= 0 && kk[i] <= pos;   // pos = -1 for padding rows
              pp[i] = valid ? __builtin_amdgcn_exp2f(fmaf(acc[i], sl2, -st.x)) * st.y : 0.f;
            }
            *reinterpret_cast<float4*>(&P[16 * qh + qc][ZP + 64 * w + 16 * kb + 4 * g4]) = pv;
          }
        }
        __syncthreads();

        // column sums of this half (rows past n_rows hold zeros)
        {
          float part[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < HR; ++r) part[r & 7] += P[r][ZP + tid];
          colsum += ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
        }
        // diagonal sums of this half -> slash accumulators (fixed point, so the
        // result does not depend on the order of the additions)
        if (slash) {
          const int pi = (J.kind == JOB_VS_2D && J.pair[0].m_k != m_chunk) ? 1 : 0;
          const MMSA_CONST PairDev& Pd = J.pair[pi];
          unsigned long long* sacc = wsp<unsigned long long>(ws, Pd.ws_sacc);
          const int n_runs = (J.kind == JOB_VS_2D) ? 1 : J.n_runs;
          for (int ru = 0; ru < n_runs; ++ru) {
            int r0, len, A;
            if (J.kind == JOB_VS_2D) {
              r0 = 0;
              len = J.n_rows;
              A = J.rho0 + Pd.n_k - 1 - (x0 - chunk_base);
            } else {
              r0 = J.run_r0[ru];
              len = J.run_len[ru];
              A = J.rows[r0] - r0 - x0;
            }
            // rows [ra, rb) of this run in this half; diagonal idx holds the
            // entries (r, A + r - idx), whose columns stay within 31 of the keys
            const int ra = max(r0, h0), rb = min(r0 + len, h0 + HR);
            if (ra >= rb) continue;   // uniform
            const int idx_lo = A + ra - (EST_CK - 1), span = rb - ra + EST_CK - 1;
            const bool whole = ra == h0 && rb == h0 + HR;
            for (int ii = tid; ii < span; ii += 256) {
              const int idx = idx_lo + ii;
              if (idx < 0 || idx >= Pd.Ds) continue;
              // &P[r - h0][ZP + A + r - idx]: one pitch plus one float per row
              const float* pd = &P[0][ZP + A + h0 - idx];
              float part[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
              if (whole) {
#pragma unroll
                for (int rl = 0; rl < HR; ++rl) part[rl & 7] += pd[rl * (PW + 1)];
              } else {
                for (int rl = ra - h0; rl < rb - h0; ++rl) part[0] += pd[rl * (PW + 1)];
              }
              const float sum = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
              if (sum != 0.f) atomicAdd(&sacc[idx], (unsigned long long)llrint((double)sum * SFIX));
            }
          }
        }
        __syncthreads();
      }

      // column sums -> vertical scores (or grid line scores)
      if (kpos_mine >= 0 && kpos_mine <= J.imax) {
        const int slot = x0 + tid;
        if (J.kind == JOB_VS_ORIG || J.kind == JOB_GRID_PLAIN) {
          wsp<float>(ws, J.pair[0].ws_v)[kpos_mine] = colsum;
        } else if (J.kind == JOB_GRID_GROUPED) {
          const int xg = (slot < dm.video_base) ? slot : dm.n_text + (slot - dm.video_base);
          wsp<float>(ws, J.pair[0].ws_v)[xg] = colsum;
        } else {
          const int pi = (J.pair[0].m_k == m_chunk) ? 0 : 1;
          wsp<float>(ws, J.pair[pi].ws_v)[slot - chunk_base] = colsum;
        }
      }
    }
  };

  // Pipeline: iteration it computes chunk c_it (positions in kp_s[it & 1],
  // keys in one register set) while the keys of c_it+1 load into the other
  // set and the positions of c_it+2 into registers.  Each iteration ends by
  // waiting for everything it issued -- the prefetches have had a whole chunk
  // of work to land -- so the compiler's waits inside the job loop, whose
  // stores would otherwise mix with loads in flight, are never needed.
  bf16x8 kA[4][NC], kB[4][NC];
  Pos p0, p1;
  const int gx = G.nwg;
  int c = xw;
  load_pos(p0, c);
  load_pos(p1, c + gx);
  load_k(kA, p0);
  kp_s[0][tid] = p0.own;
  __builtin_amdgcn_s_waitcnt(0);   // rows of Q, the first keys and positions
  __syncthreads();
  while (c < n_ck) {
    load_pos(p0, c + 2 * gx);
    load_k(kB, p1);
    body(kA, c, 0);
    __builtin_amdgcn_s_waitcnt(0);
    kp_s[1][tid] = p1.own;
    __syncthreads();
    c += gx;
    if (c >= n_ck) break;
    load_pos(p1, c + 2 * gx);
    load_k(kA, p0);
    body(kB, c, 1);
    __builtin_amdgcn_s_waitcnt(0);
    kp_s[0][tid] = p0.own;
    __syncthreads();
    c += gx;
  }
}

// Fixed-point slash sums -> float32 scores.
__global__ __launch_bounds__(256) void k_s_finalize(Tables tb, char* ws) {
  const EstJob& J = wsp<const EstJob>(ws, tb.off_jobs)[blockIdx.y >> 1];
  const int pi = blockIdx.y & 1;
  if (!(J.kind == JOB_VS_ORIG || J.kind == JOB_VS_2D) || pi >= J.n_pairs) return;
  const PairDev& Pd = J.pair[pi];
  const long long* sacc = wsp<const long long>(ws, Pd.ws_sacc);
  float* s = wsp<float>(ws, Pd.ws_s);
  for (int i = blockIdx.x * 256 + threadIdx.x; i < Pd.Ds; i += gridDim.x * 256)
    s[i] = (float)((double)sacc[i] * (1.0 / SFIX));
}

// ---------------------------------------------------------------------------
// Exact top-k of a float32 vector over [lo, hi): value descending, ties to
// the lowest index, output ascending.  Radix select on the 32-bit orderable
// key, 8 bits a round from the top, spread over the whole GPU: the vector is
// cut into slices of TK_SL elements (one workgroup each).
//   rounds 0-3  each slice's histogram of the next digit among the keys that
//               match the prefix chosen so far; every workgroup derives that
//               prefix itself from the earlier rounds' slice histograms
//   count       keys above / equal to the final threshold, per slice
//   offsets     one workgroup per vector: output offset and equal keys before
//               each slice (equal keys are taken lowest index first)
//   emit        each slice writes its selected indices in index order
// Scratch per vector (TopkTask::ws_tmp): hist [4][slices][256] u32, counts
// [slices] (greater, equal), offsets [slices] (output, equal before), state.
// ---------------------------------------------------------------------------
constexpr int TK_T = 1024;              // threads per top-k workgroup
constexpr int TK_E = TK_SL / TK_T;      // elements per thread per slice

struct TkState {
  uint32_t pref, mask, krem;   // digits fixed so far, their mask, keys still to take at the threshold
  int mode;                    // 0: select, 1: take all (k >= n), 2: take none (k <= 0)
};

// Threshold state after `rounds` rounds (identical in every workgroup): the
// state after rounds-1 (stored by the previous launch; the initial one for a
// single round) advanced by the slice histograms of round rounds-1, summed
// by all TK_T threads.  The workgroup of slice 0 stores the result for the
// next launch.  Needs all TK_T threads (barriers).
__device__ TkState tk_state(const TopkTask& T, const uint32_t* hist, uint4* stored, int n_sl, int rounds,
                            int* red, uint32_t* sh) {
  const int n = T.hi - T.lo;
  TkState st{0u, 0u, 0u, 0};
  if (T.k <= 0 || n <= 0) {
    st.mode = 2;
    return st;
  }
  if (T.k >= n) {
    st.mode = 1;
    st.krem = (uint32_t)n;
    return st;
  }
  st.krem = (uint32_t)T.k;
  if (rounds == 0) return st;
  const int r = rounds - 1, tid = threadIdx.x;
  if (r > 0) {
    const uint4 p = stored[r - 1];
    st.pref = p.x;
    st.mask = p.y;
    st.krem = p.z;
  }
  const int shift = 24 - 8 * r;
  // bin b = t & 255 over slices t>>8, t>>8 + 4, ...; then thread t (< 256)
  // holds bin 255 - t, so a prefix sum in thread order is a suffix sum over bins
  __shared__ uint32_t part[4][256];
  {
    const int b = tid & 255, g = tid >> 8;
    uint32_t c0 = 0, c1 = 0;
    int sl = g;
    for (; sl + 4 < n_sl; sl += 8) {
      c0 += hist[((int64_t)r * n_sl + sl) * 256 + b];
      c1 += hist[((int64_t)r * n_sl + sl + 4) * 256 + b];
    }
    if (sl < n_sl) c0 += hist[((int64_t)r * n_sl + sl) * 256 + b];
    part[g][b] = c0 + c1;
  }
  __syncthreads();
  const uint32_t c = tid < 256 ? part[0][255 - tid] + part[1][255 - tid] + part[2][255 - tid] + part[3][255 - tid] : 0u;
  int tot;
  const uint32_t above = (uint32_t)block_excl_sum((int)c, red, &tot);
  if (tid < 256 && above < st.krem && above + c >= st.krem) {
    sh[0] = st.pref | ((uint32_t)(255 - tid) << shift);
    sh[1] = st.krem - above;
  }
  __syncthreads();
  st.pref = sh[0];
  st.krem = sh[1];
  st.mask |= 255u << shift;
  if (blockIdx.x == 0 && tid == 0) stored[r] = make_uint4(st.pref, st.mask, st.krem, 0u);
  return st;
}

// Round `round`: this slice's histogram of digit 24 - 8*round among the keys
// matching the prefix of the earlier rounds.  grid (slices, tasks).
__global__ __launch_bounds__(TK_T) void k_topk_hist(Tables tb, char* ws, int round) {
  const TopkTask T = wsp<const TopkTask>(ws, tb.off_topk)[blockIdx.y];
  const int n = T.hi - T.lo, n_sl = (int)topk_slices(n), sl = blockIdx.x;
  if (sl >= n_sl) return;
  uint32_t* hist = wsp<uint32_t>(ws, T.ws_tmp);
  uint4* stored = reinterpret_cast<uint4*>(hist + 4ll * 256 * n_sl + 4ll * n_sl);
  __shared__ int red[17];
  __shared__ uint32_t sh[2];
  __shared__ uint32_t wh[16][256];   // one histogram per wave (keys cluster in few bins)
  const TkState st = tk_state(T, hist, stored, n_sl, round, red, sh);
  if (st.mode != 0) return;
  const int tid = threadIdx.x, wv = tid >> 6, shift = 24 - 8 * round;
  for (int i = tid; i < 16 * 256; i += TK_T) (&wh[0][0])[i] = 0;
  __syncthreads();
  const float* __restrict__ x = wsp<const float>(ws, T.ws_x);
  const int s0 = T.lo + sl * TK_SL, s1 = min(T.hi, s0 + TK_SL);
  uint32_t key[TK_E];
#pragma unroll
  for (int j = 0; j < TK_E; ++j) {
    const int i = s0 + j * TK_T + tid;
    key[j] = i < s1 ? order_key(x[i]) : 0u;
  }
#pragma unroll
  for (int j = 0; j < TK_E; ++j) {
    const int i = s0 + j * TK_T + tid;
    wave_hist_add(wh[wv], (key[j] >> shift) & 255u, i < s1 && (key[j] & st.mask) == st.pref);
  }
  __syncthreads();
  if (tid < 256) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) c += wh[w][tid];
    hist[((int64_t)round * n_sl + sl) * 256 + tid] = c;
  }
}

// Per slice: keys above and equal to the final threshold.  grid (slices, tasks).
__global__ __launch_bounds__(TK_T) void k_topk_count(Tables tb, char* ws) {
  const TopkTask T = wsp<const TopkTask>(ws, tb.off_topk)[blockIdx.y];
  const int n = T.hi - T.lo, n_sl = (int)topk_slices(n), sl = blockIdx.x;
  if (sl >= n_sl) return;
  uint32_t* hist = wsp<uint32_t>(ws, T.ws_tmp);
  int2* cnt = reinterpret_cast<int2*>(hist + 4ll * 256 * n_sl);
  uint4* stored = reinterpret_cast<uint4*>(cnt + 2ll * n_sl);
  __shared__ int red[17];
  __shared__ uint32_t sh[2];
  const TkState st = tk_state(T, hist, stored, n_sl, 4, red, sh);
  const int tid = threadIdx.x;
  // final threshold for the offsets and emit launches (after the 4 rounds' states)
  if (sl == 0 && tid == 0) stored[4] = make_uint4(st.pref, st.krem, (uint32_t)st.mode, 0u);
  const float* __restrict__ x = wsp<const float>(ws, T.ws_x);
  const int s0 = T.lo + sl * TK_SL, s1 = min(T.hi, s0 + TK_SL);
  int gt = 0, eq = 0;
  if (st.mode == 0) {
#pragma unroll
    for (int j = 0; j < TK_E; ++j) {
      const int i = s0 + j * TK_T + tid;
      if (i < s1) {
        const uint32_t key = order_key(x[i]);
        gt += key > st.pref;
        eq += key == st.pref;
      }
    }
  } else if (st.mode == 1) {
    gt = max(0, min(TK_E, (s1 - s0 - tid + TK_T - 1) / TK_T));
  }
  int tg, te;
  block_excl_sum(gt, red, &tg);
  block_excl_sum(eq, red, &te);
  if (tid == 0) cnt[sl] = make_int2(tg, te);
}

// Per vector: output offset and equal keys before each slice, and the count.
// grid (tasks).
__global__ __launch_bounds__(TK_T) void k_topk_offsets(Tables tb, char* ws) {
  const TopkTask T = wsp<const TopkTask>(ws, tb.off_topk)[blockIdx.x];
  const int n = T.hi - T.lo, n_sl = (int)topk_slices(n);
  const int tid = threadIdx.x;
  __shared__ int red[17];
  if (n_sl == 0) {
    if (tid == 0) *wsp<int32_t>(ws, T.ws_cnt) = 0;
    return;
  }
  uint32_t* hist = wsp<uint32_t>(ws, T.ws_tmp);
  const int2* cnt = reinterpret_cast<const int2*>(hist + 4ll * 256 * n_sl);
  int2* off = const_cast<int2*>(cnt) + n_sl;
  const uint4 fin = reinterpret_cast<const uint4*>(off + n_sl)[4];
  const int need = (int)fin.y;
  int out_base = 0, eq_base = 0;
  for (int c0 = 0; c0 < n_sl; c0 += TK_T) {
    const int sl = c0 + tid;
    const int2 c = sl < n_sl ? cnt[sl] : make_int2(0, 0);
    int te, ts;
    const int eq_before = eq_base + block_excl_sum(c.y, red, &te);
    const int take = c.x + max(0, min(c.y, need - eq_before));
    const int out_off = out_base + block_excl_sum(take, red, &ts);
    if (sl < n_sl) off[sl] = make_int2(out_off, eq_before);
    out_base += ts;
    eq_base += te;
  }
  if (tid == 0) *wsp<int32_t>(ws, T.ws_cnt) = out_base;
}

// Per slice: the selected indices in index order (thread t owns elements
// E t .. E t + E-1 of the slice).  grid (slices, tasks).
__global__ __launch_bounds__(TK_T) void k_topk_emit(Tables tb, char* ws) {
  const TopkTask T = wsp<const TopkTask>(ws, tb.off_topk)[blockIdx.y];
  const int n = T.hi - T.lo, n_sl = (int)topk_slices(n), sl = blockIdx.x;
  if (sl >= n_sl) return;
  const uint32_t* hist = wsp<const uint32_t>(ws, T.ws_tmp);
  const int2* cnt = reinterpret_cast<const int2*>(hist + 4ll * 256 * n_sl);
  const int2* off = cnt + n_sl;
  const uint4 fin = reinterpret_cast<const uint4*>(off + n_sl)[4];
  const int mode = (int)fin.z;
  if (mode == 2) return;
  const uint32_t thr = fin.x;
  const int need = (int)fin.y;
  const int2 o = off[sl];
  __shared__ int red[17];
  const float* __restrict__ x = wsp<const float>(ws, T.ws_x);
  int32_t* out = wsp<int32_t>(ws, T.ws_out);
  const int tid = threadIdx.x;
  const int s0 = T.lo + sl * TK_SL, s1 = min(T.hi, s0 + TK_SL);
  uint32_t key[TK_E];
  int n_eq = 0;
#pragma unroll
  for (int j = 0; j < TK_E; ++j) {
    const int i = s0 + TK_E * tid + j;
    key[j] = i < s1 ? order_key(x[i]) : 0u;
    n_eq += (mode == 0 && i < s1 && key[j] == thr) ? 1 : 0;
  }
  int eq_tot, sel_tot;
  int er = o.y + block_excl_sum(n_eq, red, &eq_tot);
  uint32_t selm = 0;
#pragma unroll
  for (int j = 0; j < TK_E; ++j) {
    const int i = s0 + TK_E * tid + j;
    const bool in = i < s1;
    const bool eq = mode == 0 && in && key[j] == thr;
    const bool sel = in && (mode == 1 || key[j] > thr || (eq && er < need));
    er += eq ? 1 : 0;
    selm |= sel ? (1u << j) : 0u;
  }
  int r = o.x + block_excl_sum(__popc(selm), red, &sel_tot);
#pragma unroll
  for (int j = 0; j < TK_E; ++j)
    if (selm & (1u << j)) out[r++] = s0 + TK_E * tid + j;
}

// ---------------------------------------------------------------------------
// Grid stride / phase rule on clipped fixed-point line scores.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t grid_u(float v, int64_t cap) {
  const int64_t u = (int64_t)floorf(v * 16777216.0f);
  return u < cap ? u : cap;
}

// Clipped fixed-point scores u (kept for the stride scan; u <= 64 * 2^24 since
// a score sums at most 64 probabilities) and their total U.
__global__ __launch_bounds__(1024) void k_grid_sum(Tables tb, char* ws) {
  const GridTask T = wsp<const GridTask>(ws, tb.off_grid)[blockIdx.x];
  const float* v = wsp<const float>(ws, T.ws_v);
  int32_t* u = wsp<int32_t>(ws, T.ws_u);
  __shared__ long long part[1024];
  long long s = 0;
  // eight loads in flight per thread (the sums are exact integers, so their
  // order does not matter)
  const int step = (int)blockDim.x;
  int x = threadIdx.x;
  for (; x + 7 * step < T.D; x += 8 * step) {
    float vv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = v[x + j * step];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t ux = grid_u(vv[j], T.cap);
      u[x + j * step] = (int32_t)ux;
      s += ux;
    }
  }
  for (; x < T.D; x += step) {
    const int64_t ux = grid_u(v[x], T.cap);
    u[x] = (int32_t)ux;
    s += ux;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int st = 512; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) part[threadIdx.x] += part[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) *wsp<long long>(ws, T.ws_U) = part[0];
}

struct GridCand {
  long long X;
  int cnt, phase;
};

// +1 if candidate a beats b (higher score; on a tie the smaller phase).
__device__ __forceinline__ bool grid_better(const GridCand& a, const GridCand& b) {
  if (a.phase < 0) return false;
  if (b.phase < 0) return true;
  const int c = grid_cmp(a.X, a.cnt, b.X, b.cnt);
  return c > 0 || (c == 0 && a.phase < b.phase);
}

// grid (strides, grid tasks), block 1024: the best phases at one stride.
__global__ __launch_bounds__(1024) void k_grid_scan(Tables tb, char* ws) {
  const GridTask T = wsp<const GridTask>(ws, tb.off_grid)[blockIdx.y];
  const int sig = T.s_lo + blockIdx.x;
  if (sig > T.s_hi) return;
  const int32_t* u = wsp<const int32_t>(ws, T.ws_u);
  const long long U = *wsp<const long long>(ws, T.ws_U);
  __shared__ GridCand c[MAX_STRIDE];
  __shared__ int idx[MAX_STRIDE];
  __shared__ long long part[MAX_STRIDE];
  const int f = threadIdx.x;
  // every thread works: phase t % sig over every S-th line position, S = slices
  {
    const int S = MAX_STRIDE / sig, ph = f % sig, sl = f / sig;
    long long F = 0;
    if (sl < S) {
      // eight loads in flight per thread (exact integer sums: any order)
      const int64_t st = (int64_t)S * sig;
      int64_t x = ph + (int64_t)sl * sig;
      for (; x + 7 * st < T.D; x += 8 * st) {
        int32_t uu[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) uu[j] = u[x + j * st];
#pragma unroll
        for (int j = 0; j < 8; ++j) F += uu[j];
      }
      for (; x < T.D; x += st) F += u[x];
    }
    part[f] = F;
  }
  __syncthreads();
  GridCand me{0, 0, -1};
  if (f < sig) {
    long long F = 0;
    for (int sl = 0; sl < MAX_STRIDE / sig; ++sl) F += part[sl * sig + f];
    const int cnt = (T.D - f + sig - 1) / sig;
    me.X = (long long)T.D * F - (long long)cnt * U;
    me.cnt = cnt;
    me.phase = f;
  }
  c[f] = me;
  const int w = min(T.w, sig);
  GridCand* outc = wsp<GridCand>(ws, T.ws_cand) + (int64_t)blockIdx.x * MAX_PHASES;
  for (int round = 0; round < w; ++round) {
    idx[f] = f;
    __syncthreads();
    for (int st = MAX_STRIDE / 2; st > 0; st >>= 1) {
      if (f < st) {
        const int a = idx[f], b = idx[f + st];
        idx[f] = grid_better(c[b], c[a]) ? b : a;
      }
      __syncthreads();
    }
    const int win = idx[0];
    if (f == 0) outc[round] = c[win];
    __syncthreads();
    if (f == win) c[f].phase = -1;
    __syncthreads();
  }
}

// grid (grid tasks), block 512: the winning stride and its phases.
__global__ __launch_bounds__(512) void k_grid_select(Tables tb, char* ws) {
  const GridTask T = wsp<const GridTask>(ws, tb.off_grid)[blockIdx.x];
  const GridCand* cand = wsp<const GridCand>(ws, T.ws_cand);
  const int ns = T.s_hi - T.s_lo + 1;
  __shared__ GridCand bc[512];
  __shared__ int bs[512];
  GridCand me{0, 0, -1};
  int msig = -1;
  for (int i = threadIdx.x; i < ns; i += 512) {   // ascending strides: strict improvement only
    const GridCand c = cand[(int64_t)i * MAX_PHASES];
    if (msig < 0 || grid_cmp(c.X, c.cnt, me.X, me.cnt) > 0) {
      me = c;
      msig = T.s_lo + i;
    }
  }
  bc[threadIdx.x] = me;
  bs[threadIdx.x] = msig;
  __syncthreads();
  for (int st = 256; st > 0; st >>= 1) {
    const int t = threadIdx.x;
    if (t < st) {
      const int sa = bs[t], sb = bs[t + st];
      bool take_b = false;
      if (sb >= 0) {
        if (sa < 0) take_b = true;
        else {
          const int cmpv = grid_cmp(bc[t + st].X, bc[t + st].cnt, bc[t].X, bc[t].cnt);
          take_b = cmpv > 0 || (cmpv == 0 && sb < sa);
        }
      }
      if (take_b) {
        bc[t] = bc[t + st];
        bs[t] = sb;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int sig = bs[0];
    const int w = min(T.w, sig);
    int32_t* out = wsp<int32_t>(ws, T.ws_out);
    int ph[MAX_PHASES];
    const GridCand* cs = cand + (int64_t)(sig - T.s_lo) * MAX_PHASES;
    for (int i = 0; i < w; ++i) ph[i] = cs[i].phase;
    for (int i = 1; i < w; ++i)
      for (int j = i; j > 0 && ph[j - 1] > ph[j]; --j) {
        int t = ph[j];
        ph[j] = ph[j - 1];
        ph[j - 1] = t;
      }
    out[0] = sig;
    out[1] = w;
    for (int i = 0; i < w; ++i) out[3 + i] = ph[i];
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_est_pass1(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k,
                            int n_wg1, hipStream_t s) {
  if (tb.n_groups1 == 0 || n_wg1 <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_wg1);
  if (dm.d == 128)
    k_est_pass1<128><<<grid, 256, 0, s>>>(dm, tb, ws, (const bf16_t*)q, (const bf16_t*)k);
  else
    k_est_pass1<64><<<grid, 256, 0, s>>>(dm, tb, ws, (const bf16_t*)q, (const bf16_t*)k);
  k_est_combine<<<(unsigned)tb.n_jobs, 1024, 0, s>>>(tb, ws);
  return hipGetLastError();
}

hipError_t launch_est_pass2(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k,
                            int n_wg2, int max_ds, hipStream_t s) {
  if (tb.n_groups2 == 0 || n_wg2 <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_wg2);
  if (dm.d == 128)
    k_est_pass2<128><<<grid, 256, 0, s>>>(dm, tb, ws, (const bf16_t*)q, (const bf16_t*)k);
  else
    k_est_pass2<64><<<grid, 256, 0, s>>>(dm, tb, ws, (const bf16_t*)q, (const bf16_t*)k);
  if (max_ds > 0) {
    dim3 g2((unsigned)min(64, (max_ds + 255) / 256), (unsigned)(2 * tb.n_jobs));
    k_s_finalize<<<g2, 256, 0, s>>>(tb, ws);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const Tables& tb, char* ws, int max_slices, hipStream_t s) {
  if (tb.n_topk == 0) return hipSuccess;
  if (max_slices > 0) {
    const dim3 g((unsigned)max_slices, (unsigned)tb.n_topk);
    for (int r = 0; r < 4; ++r) k_topk_hist<<<g, TK_T, 0, s>>>(tb, ws, r);
    k_topk_count<<<g, TK_T, 0, s>>>(tb, ws);
  }
  k_topk_offsets<<<(unsigned)tb.n_topk, TK_T, 0, s>>>(tb, ws);
  if (max_slices > 0) k_topk_emit<<<dim3((unsigned)max_slices, (unsigned)tb.n_topk), TK_T, 0, s>>>(tb, ws);
  return hipGetLastError();
}

hipError_t launch_grid(const Dims& dm, const Tables& tb, char* ws, int max_strides, hipStream_t s) {
  (void)dm;
  if (tb.n_grid == 0) return hipSuccess;
  k_grid_sum<<<(unsigned)tb.n_grid, 1024, 0, s>>>(tb, ws);
  k_grid_scan<<<dim3(max_strides, (unsigned)tb.n_grid), MAX_STRIDE, 0, s>>>(tb, ws);
  k_grid_select<<<(unsigned)tb.n_grid, 512, 0, s>>>(tb, ws);
  return hipGetLastError();
}

}  // namespace mmsa
