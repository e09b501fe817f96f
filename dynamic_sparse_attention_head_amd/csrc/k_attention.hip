// Block-sparse causal prefill over the planned key tiles and gathered columns
// (MMInference verdict page, key_machinery: FlashAttention-style kernels that
// load only the permuted blocks and keep matrix-core compute dense; the online
// softmax is the FlashAttention-2 recurrence those kernels build on).
//
// One workgroup = one pair of adjacent 64-row query tiles of one head (128
// rows), 4 waves x 32 rows.  Key chunks of 64 (a whole view tile, or 64
// gathered columns) are staged once in LDS for both tiles; the staged chunks
// are the union of the two tiles' plans and a wave computes only the chunks
// its own tile selected.  Both products run as bf16 32x32x16 MFMA with fp32
// accumulation:
//   S^T (keys x queries) = K . Q^T     -> each lane holds one query's 32 logits
//   O^T (d x queries)   += V^T . P^T   -> each lane holds one query's outputs
// so a lane owns one query row throughout: the online softmax needs one
// cross-lane exchange per chunk and its rescale is a per-lane scalar.
//
// Staging goes straight from HBM to LDS (buffer loads with the LDS bit, 16
// bytes per lane) -- no registers, no LDS stores.  K and V stay row-major with
// their 16-byte chunks XOR-swizzled per row; the V^T operand is read with the
// LDS transpose read (ds_read_b64_tr_b16), which hands each lane 4 keys of one
// d column.  The pipeline runs K one chunk ahead of V: while chunk n's softmax
// and P.V run, S^T of chunk n+1 is computed (its MFMAs interleaved with the
// softmax arithmetic), and the copies of K for chunk n+2 and V for chunk n+1
// are in flight.  Each wave issues the copies of its own rows, except in a
// step that only one tile of the pair computes: there the other tile's waves
// issue all of them, since a burst of copies stalls the issuing wave for
// hundreds of cycles.  Masking is element-wise on original positions (causal,
// A-shape window, parallel-encoding blocks) and runs only for chunks holding
// a key that some row of the wave does not see.  The running max moves only when a row's max grows by more than
// 2^LAZY, so rescales of O are rare.
#include "mmsa_device.h"

namespace mmsa {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#define MMSA_LDS __attribute__((address_space(3)))

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).  Lane l: A row l%32, k-slots
// 8*(l/32)..+8; B column l%32, same k-slots; D column l%32, rows 8i+4(l/32)+j
// held at index 4i+j.
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct AttnSmem {   // 2 stages of K and V (row-major, swizzled); key positions, their max and min, 4 slots
  bf16_t K[2][64 * D];
  bf16_t V[2][64 * D];
  int kp[4][64];
  int kmax[4];
  int kmin[4];
};

// Swizzle of the 16-byte chunks of row r: physical chunk = logical ^ swz(r).
// It is XOR-linear in the row bits and maps, for the 64 LDS banks,
//  * 16 consecutive rows read at one logical chunk (the lanes of one K
//    fragment read) to 16 different 16-byte bank groups, and
//  * 4 consecutive rows x 4 adjacent chunks (two 16-lane transpose reads of V)
//    to 16 different bank groups.
// d = 128 (256-byte rows): chunk bits (0,1,2,3) <- row bits (2,3,0,1).
// d = 64 (128-byte rows, two per bank window): chunk bits (0,1,2) <- row bits (2,3,1).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if (D == 128) return ((r >> 2) & 1) | (((r >> 3) & 1) << 1) | ((r & 1) << 2) | (((r >> 1) & 1) << 3);
  return ((r >> 2) & 1) | (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from the buffer straight into LDS at dst + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (MMSA_LDS void*)dst, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// Transpose read: within each 16-lane group, lane i receives element i%4 of the
// 8 bytes addressed by lanes 4j + i/4 (j = 0..3) as its elements j.
__device__ __forceinline__ uint2 ld_tr(const void* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MMSA_LDS bf16x4_t*)p));
}

// (x[l], x[l ^ 32]) as a pair, in registers: v_permlane32_swap exchanges the
// upper half-wave of one copy with the lower half-wave of the other, so the
// two results hold, lane by lane, x and its partner in some order.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Max over the 64 lanes in registers, no LDS round trip: DPP within each row
// of 16 (quad swaps, then the half-row and row mirrors), then the row swaps of
// v_permlane16_swap and v_permlane32_swap.  Every lane receives the result.
__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));    // lane ^ 1
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));    // lane ^ 2
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));   // 7 - lane within 8
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));   // 15 - lane within 16
  const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = max((int)r[0], (int)r[1]);
  const auto r2 = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)r2[0], (int)r2[1]);
}

constexpr uint32_t OOB = 0x80000000u;   // a buffer offset past every tensor slice
constexpr float LAZY_LOG2 = 8.0f;       // stale-max slack of the online softmax (log2 units)
__device__ constexpr bf16x2_t ONES_BF2 = {(__bf16)1.0f, (__bf16)1.0f};

// Descriptor of one staged chunk: source (-1 view tile, 0 first list, 1 second
// list), index (tile, or 64-column chunk of the list) and which tiles of the
// pair selected it (bit 0: first, bit 1: second).
struct Chunk {
  int src, idx, memb;
};

// One (head, query-tile pair) work item.  Ends with a workgroup barrier, so the
// next item may reuse the LDS at once.
template <int D>
__device__ __forceinline__ void attn_pair(AttnSmem<D>& sm, const Dims& dm, const Tables& tb, char* ws,
                                          const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                          const bf16_t* __restrict__ v, bf16_t* __restrict__ o,
                                          float* __restrict__ lse, uint32_t item) {
  constexpr int NS = D / 16, ND = D / 32;
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;       // rows per staging instruction (64 lanes x 16 bytes)
  constexpr int PPW = CPR / 4;        // staging instructions per wave per tile
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
    // all fragments in flight at once: a row without a token reads the head's
    // row 0 (or its padding slot) and is zeroed afterwards
    uint4 u[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) u[s] = ld16(qrow + 16 * s + 8 * hh);
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (qpos < 0) u[s] = make_uint4(0, 0, 0, 0);
    // Consume the fragments here, once: afterwards they are plain register values,
    // not loads in flight, so the chunk loop never has to wait for them.
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
  const int gcnt0 = grid ? max(g0, g1) : g0;
  const bool grouped_view = H.view_kind == VIEW_GROUPED;
  // grouped view without a grouped copy of K/V: its tiles are read row by row
  // through the grouped-slot map, like gathered columns
  const bool grouped_idx = grouped_view && H.ws_kgrp < 0;
  const int32_t* pgrp = wsp<const int32_t>(ws, dm.ws_pgrp);
  // A key j of row i is kept when j <= i and (j < sink or j >= klo(i)).
  // A-shape: klo = i - window + 1; parallel encoding: the start of the row's
  // context block, 0 for its sink and question rows; other patterns: no bound
  // (INT_MIN).  Both are taken once here, through empty asm, so the chunk
  // loop neither recomputes them nor branches on the pattern per element.
  // Grid heads with a sink or a local window: rows off the lines take the
  // A-shape rule on the key tiles (klo = i - window + 1, or no window at all),
  // line rows see every causal key (klo = INT_MIN).  Their gathered chunks hold
  // line keys, of which those already inside the sink or the row's window sit
  // in a listed tile too: there the rule is inverted (kept when j >= sink and
  // j < klo), so each key counts once.
  const bool ashape = H.pattern == MMSA_ASHAPE, parallel = H.pattern == MMSA_PARALLEL;
  const bool gridwin = grid && (H.sink > 0 || H.window > 0);
  int grid_line_row = 0;
  if (gridwin) {
    const int nline = wsp<const int32_t>(ws, cptr<GridTask>(ws, tb.off_grid)[H.grid_task].ws_out)[2];
    grid_line_row = slot < ((nline + 63) & ~63);
  }
  int windowed = uniform((ashape || parallel || gridwin) ? 1 : 0);
  asm volatile("" : "+s"(windowed));
  const int sink = H.sink;
  int klo = ashape ? qpos - H.window + 1
            : parallel ? par_floor(H.sink, H.window, H.qstart, qpos)
            : gridwin ? (grid_line_row ? INT_MIN : H.window > 0 ? qpos - H.window + 1 : INT_MAX)
            : INT_MIN;
  asm volatile("" : "+v"(klo));
  // the largest klo of the wave's rows: a chunk whose keys all lie at or past
  // it (and before the first row) needs no mask
  const int wave_klomax = uniform(wave_max_i32(qpos >= 0 ? klo : INT_MIN));

  // buffer views: the head's key view (tiles) and its original K/V (gathered columns)
  const bool grouped_copy = grouped_view && !grouped_idx;
  const uint32_t rb_view = grouped_copy ? 2u * D : 2u * (uint32_t)dm.k_sl;
  const uint32_t rbv_view = grouped_copy ? 2u * D : 2u * (uint32_t)dm.v_sl;
  const uint32_t rbk = 2u * (uint32_t)dm.k_sl, rbv = 2u * (uint32_t)dm.v_sl;
  const int view_rows = grouped_view ? dm.L_grp : dm.L;
  const int copy_rows = grouped_copy ? dm.L_grp : dm.L;
  const __amdgpu_buffer_rsrc_t rk_view =
      make_rsrc(grouped_copy ? (const void*)wsp<const bf16_t>(ws, H.ws_kgrp) : (const void*)(k + H.k_off),
                (uint32_t)(copy_rows - 1) * rb_view + 2u * D);
  const __amdgpu_buffer_rsrc_t rv_view =
      make_rsrc(grouped_copy ? (const void*)wsp<const bf16_t>(ws, H.ws_vgrp) : (const void*)(v + H.v_off),
                (uint32_t)(copy_rows - 1) * rbv_view + 2u * D);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + H.k_off, (uint32_t)(dm.L - 1) * rbk + 2u * D);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + H.v_off, (uint32_t)(dm.L - 1) * rbv + 2u * D);

  // ---- staging: instruction p of wave w fills chunk rows (w*PPW + p)*RPI .. +RPI-1;
  // the lane writes row srow0 + p*RPI, physical chunk lane % CPR, which holds
  // logical chunk (lane % CPR) ^ swz(row) = lchk0 ^ swz(p*RPI) (swz is linear
  // and p*RPI shares no bits with srow0's low bits).
  const int srow0 = w * PPW * RPI + lane / CPR;
  const uint32_t lchk0 = 16u * (uint32_t)((lane % CPR) ^ swz<D>(srow0));
  auto lchk = [&](int p) -> uint32_t { return lchk0 ^ (16u * (uint32_t)swz<D>(p * RPI)); };
  char* const kbuf0 = reinterpret_cast<char*>(sm.K[0]);
  char* const vbuf0 = reinterpret_cast<char*>(sm.V[0]);
  constexpr uint32_t BUFB = 64u * D * 2u;   // bytes of one K or V stage
  // Copies of this wave's rows of chunk c (key positions in LDS slot ks).
  // View tiles are contiguous rows of the view; gathered columns, and tiles of
  // an index-read grouped view, are rows listed by original position, read
  // from the chunk's key positions (KPOS_NONE: no token, copied as zeros).
  // A wave may also copy the rows of another wave slot ws: the slot moves the
  // row by a multiple of 16, which leaves the swizzle (row bits 0-3) alone.
  static_assert(PPW * RPI == 16, "16 rows per wave slot");
  auto dma_k = [&](const Chunk& c, int par, int ks, int ws) {
    char* dst = kbuf0 + par * BUFB + (ws * PPW) * 1024;
    const int srow = srow0 + 16 * (ws - w);
    if (c.src < 0 && !grouped_idx) {
      // the tile's row offset goes into the vector offset, which the buffer's
      // range check covers: rows past the view's end read as zeros
      const uint32_t s0 = (uint32_t)(64 * c.idx) * rb_view;
      const uint32_t ro = (uint32_t)srow * rb_view;
#pragma unroll
      for (int p = 0; p < PPW; ++p) dma16(rk_view, dst + p * 1024, ro + lchk(p) + s0 + (uint32_t)(p * RPI) * rb_view, 0);
    } else {
      int gi[PPW];
#pragma unroll
      for (int p = 0; p < PPW; ++p) gi[p] = sm.kp[ks][srow + p * RPI];
#pragma unroll
      for (int p = 0; p < PPW; ++p)
        dma16(rk, dst + p * 1024, gi[p] != KPOS_NONE ? (uint32_t)gi[p] * rbk + lchk(p) : OOB, 0);
    }
  };
  auto dma_v = [&](const Chunk& c, int par, int ks, int ws) {
    char* dst = vbuf0 + par * BUFB + (ws * PPW) * 1024;
    const int srow = srow0 + 16 * (ws - w);
    if (c.src < 0 && !grouped_idx) {
      const uint32_t s0 = (uint32_t)(64 * c.idx) * rbv_view;
      const uint32_t ro = (uint32_t)srow * rbv_view;
#pragma unroll
      for (int p = 0; p < PPW; ++p) dma16(rv_view, dst + p * 1024, ro + lchk(p) + s0 + (uint32_t)(p * RPI) * rbv_view, 0);
    } else {
      int gi[PPW];
#pragma unroll
      for (int p = 0; p < PPW; ++p) gi[p] = sm.kp[ks][srow + p * RPI];
#pragma unroll
      for (int p = 0; p < PPW; ++p)
        dma16(rv, dst + p * 1024, gi[p] != KPOS_NONE ? (uint32_t)gi[p] * rbv + lchk(p) : OOB, 0);
    }
  };
  // key positions of a chunk (wave 0, one per lane): the raw value, and whether
  // the slot holds a token; they are combined only when stored, so the load
  // stays in flight until then
  auto load_kp = [&](const Chunk& c, bool& valid) -> int {
    if (c.src < 0) {
      const int vr = 64 * c.idx + lane;
      valid = true;
      if (grouped_view) return pgrp[min(vr, view_rows - 1)];
      return vr < dm.L ? vr : -1;
    }
    const int32_t* gl = c.src == 0 ? gl0 : gl1;
    const int e0 = 64 * c.idx, el = (c.src == 0 ? gcnt0 : g1) - 1;
    valid = e0 + lane <= el;
    return gl[min(e0 + lane, el)];
  };
  auto store_kp = [&](int kpr, bool valid, int par) {
    const int kpos = (valid & (kpr >= 0)) ? kpr : KPOS_NONE;
    sm.kp[par][lane] = kpos;
    const int mx = wave_max_i32(kpos);
    if (lane == 0) sm.kmax[par] = mx;
    if (windowed) {
      const int mn = -wave_max_i32(-kpos);   // positions are >= 0 (KPOS_NONE is the largest int)
      if (lane == 0) sm.kmin[par] = mn;
    }
  };
  // A tile of an ungrouped key view holds the keys 64 idx .. 64 idx + 63 in
  // order (those past the end are masked as later than every row), so its
  // positions, their max and their min are arithmetic: nothing goes through
  // LDS for it, and wave 0 neither loads nor stores its positions.
  auto arith = [&](const Chunk& c) -> bool { return c.src < 0 && !grouped_view; };

  // Chunk sequence (uniform across the workgroup): the union of both tiles'
  // key tiles, then the gathered columns.  Key tiles go highest first --
  // workgroups on neighbouring query tiles then stream the same key tiles at
  // about the same time and share them in L2, and the diagonal comes first --
  // or, when one KV head's K/V exceed the last-level cache, lowest first.
  const bool asc = dm.chunk_asc != 0;
  int wi = asc ? -1 : W;
  uint64_t bits = 0, wb0 = 0, wb1 = 0;
  auto next_chunk = [&](int ci) -> Chunk {
    Chunk c{0, 0, 0};
    if (ci >= n_chunks) return c;
    if (ci < n_union) {
      while (bits == 0ull && (asc ? wi < W - 1 : wi > 0)) {
        wi += asc ? 1 : -1;
        wb0 = use0 ? bm0[wi] : 0ull;
        wb1 = use1 ? bm1[wi] : 0ull;
        bits = wb0 | wb1;
      }
      const int b = bits ? (asc ? __builtin_ctzll(bits) : 63 - __clzll((long long)bits)) : -1;
      bits &= ~(1ull << (b & 63));
      c.src = -1;
      c.idx = b < 0 ? (view_rows + 63) / 64 : 64 * wi + b;   // (b < 0 only for a corrupt plan)
      c.memb = b < 0 ? 0 : (int)(((wb0 >> b) & 1ull) | (((wb1 >> b) & 1ull) << 1));
      return c;
    }
    const int n = ci - n_union;
    if (grid) {
      c.src = 0;
      c.idx = n;
      c.memb = (64 * n < g0 ? 1 : 0) | (64 * n < g1 ? 2 : 0);
    } else if (n < nch0) {
      c.src = 0;
      c.idx = n;
      c.memb = 1;
    } else {
      c.src = 1;
      c.idx = n - nch0;
      c.memb = 2;
    }
    return c;
  };

  // ---- per-lane LDS addresses of the MFMA operands ----
  // Within a stage, rows start at multiples of 2D bytes and the chunk bits sit
  // above them untouched, so a swizzled address is a lane base XOR a constant.
  // K fragment (key block kb, d-step s): row 32kb + qc, logical chunk 2s ^ hh.
  const uint32_t ka = (uint32_t)qc * (2u * D) + 16u * (uint32_t)(hh ^ swz<D>(qc));
  // V^T fragment (d-block db, key step st): two transpose reads by 16-lane
  // groups; group g = lane/16 covers d 32db + 16(g&1) + 0..15 and keys
  // 16st + 4(g>>1) + 0..3 (+8 for the second read).  Source lane i of a group
  // addresses row 4(g>>1) + i/4, d 32db + 16(g&1) + 4(i%4), i.e. logical chunk
  // 4db ^ vcl and byte 8(i&1) within it.
  const int vg = lane >> 4, vi = lane & 15;
  const int vrow = 4 * (vg >> 1) + (vi >> 2);
  const int vcl = 2 * (vg & 1) + ((vi & 3) >> 1);
  uint32_t va[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    va[e] = (uint32_t)(vrow + 8 * e) * (2u * D) + 16u * (uint32_t)(vcl ^ swz<D>(vrow + 8 * e)) + 8u * (vi & 1);

  // The bases pass through an empty asm once per chunk: the per-fragment XORs
  // are then recomputed (one VALU each) instead of hoisted into 24 live
  // registers.
  uint32_t ka_l = ka, va_l[2] = {va[0], va[1]};
  auto launder = [&]() {
    asm volatile("" : "+v"(ka_l));
    asm volatile("" : "+v"(va_l[0]), "+v"(va_l[1]));
  };
  auto kfrag = [&](int par, int i) -> bf16x8 {   // i: key block i&1, d-step i>>1
    const int s = i >> 1, kb = i & 1;
    const char* p = kbuf0 + par * BUFB + kb * 32 * (2 * D) + (ka_l ^ (32u * s));
    return as_bf16x8(ld16(p));
  };
  auto vfrag = [&](int par, int i) -> bf16x8 {   // i: d-block i%ND, key step i/ND
    const int db = i % ND, st = i / ND;
    const char* b = vbuf0 + par * BUFB + st * 16 * (2 * D);
    const uint2 lo = ld_tr(b + (va_l[0] ^ (64u * db))), hi = ld_tr(b + (va_l[1] ^ (64u * db)));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
  };

  floatx16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = dm.scale_log2;
  const int wbit = w < 2 ? 1 : 2;
  constexpr int PF = 4, NK = 2 * NS, NV = 4 * ND;

  // S^T of one chunk into sa (fragment reads run PF ahead of their MFMAs)
  auto s_chunk = [&](floatx16 (&sa)[2], int par) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sa[kb][e] = 0.f;
    bf16x8 af[NK];
#pragma unroll
    for (int i = 0; i < PF; ++i) af[i] = kfrag(par, i);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + PF < NK) af[i + PF] = kfrag(par, i + PF);
      sa[i & 1] = mfma32(af[i], qf[i >> 1], sa[i & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // mask and running-max update of one chunk's logits (the part of the softmax
  // that may branch); returns the max to subtract
  auto soft_a = [&](floatx16 (&sa)[2], int ks, bool inv, const Chunk& c) -> float {
    const bool ar = arith(c);
    const int kmx = ar ? 64 * c.idx + 63 : uniform(sm.kmax[ks]);
    bool full = kmx <= wave_qmin;
    if (windowed) full = full && (kmx < sink || (ar ? 64 * c.idx : uniform(sm.kmin[ks])) >= wave_klomax);
    full = full && !inv;
    if (!full) {
      // one lane-dependent base, constant offsets per (kb, i)
      const char* kpb = reinterpret_cast<const char*>(sm.kp[0]) + ks * 256 + 16 * hh;
      const int kp0 = 64 * c.idx + 4 * hh;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 32 * kb + 8 * i;   // slot of kpv[0]
          const int4 kk = ar ? make_int4(kp0 + e, kp0 + e + 1, kp0 + e + 2, kp0 + e + 3)
                             : *reinterpret_cast<const int4*>(kpb + 4 * e);
          const int kpv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool ok = (kpv[j] <= qpos) & (((kpv[j] < sink) | (kpv[j] >= klo)) != inv);
            sa[kb][4 * i + j] = ok ? sa[kb][4 * i + j] : -INFINITY;
          }
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(sa[kb][e], sa[kb][e + 1]));
    mx = max_xor32(mx);
    const float m_cand = fmaxf(m_run, mx * sl2);
    if (__ballot(m_cand > m_run + LAZY_LOG2)) {
      const float m_use = (m_cand == -INFINITY) ? 0.f : m_cand;
      const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_cand;
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db] *= corr;
    }
    return (m_run == -INFINITY) ? 0.f : m_run;
  };
  // probabilities of the 2 logits e = 2i, 2i+1 (bf16, packed in MFMA k-slot order)
  auto soft_pair = [&](const floatx16 (&sa)[2], float m_use, int i) -> uint32_t {
    const int kb = i >> 3, e = 2 * (i & 7);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sa[kb][e], sl2, -m_use));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sa[kb][e + 1], sl2, -m_use));
    return pack_bf2_hw(p0, p1);
  };
  // row sum of the bf16-rounded probabilities, the values the MFMA consumes
  auto row_sum = [&](const uint32_t (&pk)[16]) {
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[e]), ONES_BF2, psum, false);
    l_run += psum;
  };
  auto soft_b = [&](const floatx16 (&sa)[2], float m_use, uint32_t (&pk)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) pk[i] = soft_pair(sa, m_use, i);
    row_sum(pk);
  };
  // S^T of the next chunk into sn, interleaved step by step with the
  // probabilities of the current chunk (one MFMA per 2 exponentials)
  auto s_and_soft = [&](floatx16 (&sn)[2], int par, const floatx16 (&sc)[2], float m_use, uint32_t (&pk)[16]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sn[kb][e] = 0.f;
    bf16x8 af[NK];
#pragma unroll
    for (int i = 0; i < PF; ++i) af[i] = kfrag(par, i);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + PF < NK) af[i + PF] = kfrag(par, i + PF);
      sn[i & 1] = mfma32(af[i], qf[i >> 1], sn[i & 1]);
      if (NK == 16) {
        pk[i] = soft_pair(sc, m_use, i);
      } else {   // 8 MFMAs: 4 exponentials each
        pk[2 * i] = soft_pair(sc, m_use, 2 * i);
        pk[2 * i + 1] = soft_pair(sc, m_use, 2 * i + 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    row_sum(pk);
  };
  auto pv_chunk = [&](const uint32_t (&pk)[16], int par) {
    bf16x8 vf[NV];
#pragma unroll
    for (int i = 0; i < PF; ++i) vf[i] = vfrag(par, i);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + PF < NV) vf[i + PF] = vfrag(par, i + PF);
      const int st = i / ND;   // 16-key step: accumulator values 8(st&1).. of key block st>>1
      const bf16x8 pb = as_bf16x8(make_uint4(pk[4 * st], pk[4 * st + 1], pk[4 * st + 2], pk[4 * st + 3]));
      oacc[i % ND] = mfma32(vf[i], pb, oacc[i % ND]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: positions of chunks 0-2; K, V of chunk 0; K of chunk 1 ----
  // Key positions of chunk m (other than an arithmetic view tile) live in LDS
  // slot m % 4 from the end of step m-3 (chunks 0-2: the prologue) until step
  // m: the copies of K (step m-2) and V (step m-1) read their rows there, so
  // no copy waits on a global load.
  Chunk c0 = next_chunk(0), c1 = next_chunk(1), c2 = next_chunk(2), c3 = next_chunk(3);
  int kpreg = -1;
  bool kpval = false;
  floatx16 sA[2], sB[2];
  if (n_chunks > 0) {
    if (w == 0) {
      bool va, vb, vc;
      const int a = load_kp(c0, va);
      const int b = n_chunks > 1 ? load_kp(c1, vb) : -1;
      const int cc = n_chunks > 2 ? load_kp(c2, vc) : -1;
      if (!arith(c0)) store_kp(a, va, 0);
      if (n_chunks > 1 && !arith(c1)) store_kp(b, vb, 1);
      if (n_chunks > 2 && !arith(c2)) store_kp(cc, vc, 2);
    }
    __syncthreads();
    dma_k(c0, 0, 0, w);
    dma_v(c0, 0, 0, w);
    if (n_chunks > 1) dma_k(c1, 1, 1, w);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    launder();
    if (wave_has && (c0.memb & wbit)) s_chunk(sA, 0);
    // step 0 copies K of chunk 2 over stage 0, which S^T of chunk 0 just read
    __syncthreads();
  }

  // ---- chunk n (parity par): S^T of n+1 while n's softmax and P.V run ----
  auto step = [&](floatx16 (&scur)[2], floatx16 (&snxt)[2], int n, int par) {
    const bool has_n1 = n + 1 < n_chunks, has_n2 = n + 2 < n_chunks, has_n3 = n + 3 < n_chunks;
    launder();
    // positions of chunk n+3 (unless arithmetic), stored at the end of this
    // step into the slot of chunk n-1 (read for the last time in the previous
    // step)
    const bool kp3 = has_n3 && w == 0 && !arith(c3);
    if (kp3) kpreg = load_kp(c3, kpval);
    const bool doS = wave_has && has_n1 && (c1.memb & wbit);
    const bool doP = wave_has && (c0.memb & wbit);
    // Copies of K(n+2) over K(n) (read by the previous step) and of V(n+1)
    // over V(n-1).  Each wave copies its own rows, except when only one tile
    // of the pair computes chunk n: then the other tile's waves, which have
    // at most S^T(n+1) to do, also copy the rows of the busy waves (slot w^2).
    const bool other_busy = (w < 2 ? use1 : use0) && (c0.memb & (w < 2 ? 2 : 1));
    const bool give = doP && !other_busy, take = !doP && other_busy;
    if (has_n2) {
      if (!give) dma_k(c2, par, (n + 2) & 3, w);
      if (take) dma_k(c2, par, (n + 2) & 3, w ^ 2);
    }
    if (has_n1) {
      if (!give) dma_v(c1, par ^ 1, (n + 1) & 3, w);
      if (take) dma_v(c1, par ^ 1, (n + 1) & 3, w ^ 2);
    }
    if (doP) {
      const float m_use = soft_a(scur, n & 3, gridwin && c0.src >= 0, c0);
      uint32_t pk[16];
      // The two branches compute the same probabilities; each takes the max
      // through its own (different) empty asm, so the compiler cannot hoist
      // them above the branch and out of the interleave with the MFMAs.
      float mu = m_use;
      if (doS) {
        asm volatile("; interleaved" : "+v"(mu));
        s_and_soft(snxt, par ^ 1, scur, mu, pk);
      } else {
        asm volatile("; plain" : "+v"(mu));
        soft_b(scur, mu, pk);
      }
      pv_chunk(pk, par);
    } else if (doS) {
      s_chunk(snxt, par ^ 1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (kp3) store_kp(kpreg, kpval, (n + 3) & 3);
    __syncthreads();
    c0 = c1;
    c1 = c2;
    c2 = c3;
    c3 = next_chunk(n + 4);
  };
  for (int n = 0; n < n_chunks; n += 2) {
    step(sA, sB, n, 0);
    if (n + 1 < n_chunks) step(sB, sA, n + 1, 1);
  }

  // ---- epilogue ----
  const float l_tot = sum_xor32(l_run);
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
  if (dm.debug) {
    // MMSA_FLAG_DEBUG: a non-finite output element (or a non-finite row sum,
    // which makes the LSE +inf or NaN) sets bit 3 of the debug word.  This
    // file is built without NaN semantics, under which the compiler may read
    // an exponent test on a float's bits as "is infinite"; the bits therefore
    // pass through an empty asm first, which hides where they came from.
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    auto nonfinite = [](float x) {
      uint32_t u = __float_as_uint(x);
      asm volatile("" : "+v"(u));
      return (u & 0x7f800000u) == 0x7f800000u;
    };
    bool bad = false;
    if (qpos >= 0) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) bad |= nonfinite(oacc[db][e] * inv);
      bad |= nonfinite(l_tot);
    }
    if (__ballot(bad) != 0ull && lane == 0) atomicOr(wsp<uint32_t>(ws, dm.ws_flag), 8u);
  }
}

// Persistent workgroups.  The queue (heads sharing a KV head together, most
// expensive pairs first) is dealt round-robin to the 8 XCDs: a workgroup pops
// items x, x+8, x+16, ... of its own XCD x (atomic counter per XCD), then
// helps the other XCDs.  All XCDs thus work on the same KV head at the same
// time, and its K/V stream through the shared last-level cache once for all of
// them.  Every workgroup exits once all counters have passed the end.
template <int D>
__global__ __launch_bounds__(256, 2) void k_attn(Dims dm, Tables tb, char* ws, const bf16_t* __restrict__ q,
                                                 const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                 bf16_t* __restrict__ o, float* __restrict__ lse) {
  __shared__ AttnSmem<D> sm;
  __shared__ int sh_j;
  int32_t* ctr = wsp<int32_t>(ws, dm.ws_ctr);
  const int32_t* items = wsp<const int32_t>(ws, dm.ws_enum_item);
  const int64_t n_items = dm.n_items;
  // this workgroup's XCD (hardware XCC id)
  const int x0 = (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (N_XCD - 1));
  for (int s = 0; s < N_XCD; ++s) {
    const int x = (x0 + s) % N_XCD;
    while (true) {
      if (threadIdx.x == 0) sh_j = atomicAdd(&ctr[x], 1);
      __syncthreads();
      // the popped index is the same in every lane; saying so keeps the item's
      // descriptors in scalar registers and its control flow uniform
      const int64_t e = x + (int64_t)N_XCD * __builtin_amdgcn_readfirstlane(sh_j);
      __syncthreads();
      if (e >= n_items) break;
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
