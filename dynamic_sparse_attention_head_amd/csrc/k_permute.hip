// Modality-aware permutation and the per-query-tile sparse plan.
//
// Pages: MMInference verdict page, core_discovery (row-wise permutation
// grouping same-modality queries, column-wise permutation aligning key
// strides, 2D permutation isolating each modality pair) and key_machinery
// (tensors permuted so grid lines become contiguous; kernels load only the
// permuted blocks).
//
// Row orders:  grid heads put their line rows first (x mod stride in the kept
// phases), then the other rows, each group ascending and padded to 64;
// boundary heads use the modality-grouped order (text, then video, each
// ascending and padded to 256); per-segment heads the segment-grouped order
// (every segment ascending and padded to 64, in segment order).  Grid key lines are the same positions, so the
// first rows of a grid head's row order are also its gathered key list.
//
// The plan of one query tile is a bitmap over the 64-key tiles of the head's
// key view (identity, or modality-grouped for 2D-boundary heads) plus a list of
// gathered key positions that no listed tile holds, the exact number of
// selected (query, key) pairs, and a cost (tiles + gathered chunks) used to
// order the attention work queue from most to least expensive.
#include "block_scan.h"

namespace mmsa {

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* p, uint32_t value, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = value;
}

hipError_t launch_fill_u32(void* p, uint32_t value, int64_t n_words, hipStream_t s) {
  if (n_words <= 0) return hipSuccess;
  int64_t blocks = (n_words + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  k_fill_u32<<<(unsigned)blocks, 256, 0, s>>>((uint32_t*)p, value, n_words);
  return hipGetLastError();
}

// Modality, rank and grouped slot of every position.  grid (L/256), block 256.
__global__ __launch_bounds__(256) void k_seg_tables(Dims dm, Tables tb, char* ws) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= dm.L) return;
  const SegDev* segs = wsp<const SegDev>(ws, tb.off_segs);
  int lo = 0, hi = (int)tb.n_segs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].start <= p) lo = mid;
    else hi = mid - 1;
  }
  const SegDev sg = segs[lo];
  const int rank = sg.rank_start + (int)(p - sg.start);
  const int slot = (sg.modality == MMSA_VIDEO ? dm.video_base : dm.text_base) + rank;
  wsp<int32_t>(ws, dm.ws_gslot)[p] = slot;
  wsp<int32_t>(ws, dm.ws_pgrp)[slot] = p;
  if (dm.ws_pseg >= 0) wsp<int32_t>(ws, dm.ws_pseg)[sg.slot0 + (int)(p - sg.start)] = p;
}

hipError_t launch_seg_tables(const Dims& dm, const Tables& tb, char* ws, hipStream_t s) {
  hipError_t e = launch_fill_u32(ws + dm.ws_pgrp, 0xffffffffu, dm.L_grp, s);
  if (e != hipSuccess) return e;
  if (dm.ws_pseg >= 0) {
    e = launch_fill_u32(ws + dm.ws_pseg, 0xffffffffu, dm.L_seg, s);
    if (e != hipSuccess) return e;
  }
  if (dm.L > 0) k_seg_tables<<<(dm.L + 255) / 256, 256, 0, s>>>(dm, tb, ws);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grid row orders.  cl(y) = number of grid-line coordinates in [0, y).
// ---------------------------------------------------------------------------
struct GridLines {
  int sig, w, ph[MAX_PHASES];
};

__device__ __forceinline__ GridLines load_lines(const int32_t* out) {
  // clamped so that a result never written (calls out of order) stays harmless
  GridLines g;
  g.sig = max(out[0], 1);
  g.w = min(max(out[1], 0), min(MAX_PHASES, g.sig));
#pragma unroll
  for (int i = 0; i < MAX_PHASES; ++i) g.ph[i] = (i < g.w) ? min(max(out[3 + i], 0), g.sig - 1) : 0;
  return g;
}
__device__ __forceinline__ int lines_below(const GridLines& g, int y) {
  int c = 0;
  for (int i = 0; i < g.w; ++i) c += (y > g.ph[i]) ? (y - g.ph[i] + g.sig - 1) / g.sig : 0;
  return c;
}
__device__ __forceinline__ bool on_line(const GridLines& g, int x) {
  const int r = x % g.sig;
  bool on = false;
  for (int i = 0; i < g.w; ++i) on |= (r == g.ph[i]);
  return on;
}

// grid (L/256, grid tasks), block 256.
__global__ __launch_bounds__(256) void k_grid_rows(Dims dm, Tables tb, char* ws) {
  const GridTask T = wsp<const GridTask>(ws, tb.off_grid)[blockIdx.y];
  const HeadDev& H = wsp<const HeadDev>(ws, tb.off_heads)[T.bh];
  int32_t* gout = wsp<int32_t>(ws, T.ws_out);
  const GridLines gl = load_lines(gout);
  const int n_line = lines_below(gl, dm.L);
  const int nl_pad = (n_line + 63) & ~63;
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x == 0) gout[2] = n_line;
  if (p >= dm.L) return;
  int x, prefix;
  if (T.grouped) {
    const int slot = wsp<const int32_t>(ws, dm.ws_gslot)[p];
    const bool vid = slot >= dm.video_base && dm.n_video > 0 && (dm.video_base > 0 || dm.n_text == 0);
    const int rank = vid ? slot - dm.video_base : slot - dm.text_base;
    x = vid ? dm.n_text + rank : rank;
    const int kt = vid ? p - rank : rank;      // text positions before p
    const int kv = p - kt;                      // video positions before p
    prefix = lines_below(gl, kt) + lines_below(gl, dm.n_text + kv) - lines_below(gl, dm.n_text);
  } else {
    x = p;
    prefix = lines_below(gl, p);
  }
  const int slot = on_line(gl, x) ? prefix : nl_pad + (p - prefix);
  if (slot >= 0 && slot < H.n_row_slots) wsp<int32_t>(ws, H.ws_row_order)[slot] = p;
}

hipError_t launch_grid_rows(const Dims& dm, const Tables& tb, char* ws, hipStream_t s) {
  if (tb.n_grid == 0 || dm.L == 0) return hipSuccess;
  k_grid_rows<<<dim3((dm.L + 255) / 256, (unsigned)tb.n_grid), 256, 0, s>>>(dm, tb, ws);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row gathers (Q of permuted heads, grouped K/V) and the output scatter.
// grid (slots*chunks/256, tasks), block 256; one thread moves 16 bytes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gather(Dims dm, Tables tb, char* ws, const bf16_t* __restrict__ q,
                                                const bf16_t* __restrict__ k, const bf16_t* __restrict__ v) {
  const GatherTask T = wsp<const GatherTask>(ws, tb.off_gather)[blockIdx.y];
  const int CH = dm.d / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int slot = (int)(idx / CH), ch = (int)(idx % CH);
  if (slot >= T.n_slots) return;
  const bf16_t* src = (T.which == 0 ? q : T.which == 1 ? k : v) + T.src_off;
  const int row = wsp<const int32_t>(ws, T.ws_rows)[slot];
  uint4 val = make_uint4(0, 0, 0, 0);
  if (row >= 0) val = ld16(src + (int64_t)row * T.row_stride + 8 * ch);
  st16(wsp<bf16_t>(ws, T.ws_dst) + (int64_t)slot * dm.d + 8 * ch, val);
}

hipError_t launch_gather(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k, const void* v,
                         int max_slots, hipStream_t s) {
  if (tb.n_gather == 0) return hipSuccess;
  const int64_t n = (int64_t)max_slots * (dm.d / 8);
  k_gather<<<dim3((unsigned)((n + 255) / 256), (unsigned)tb.n_gather), 256, 0, s>>>(
      dm, tb, ws, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_unpermute(Dims dm, Tables tb, char* ws, bf16_t* __restrict__ o) {
  const UnpermTask T = wsp<const UnpermTask>(ws, tb.off_unperm)[blockIdx.y];
  const int CH = dm.d / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int slot = (int)(idx / CH), ch = (int)(idx % CH);
  if (slot >= T.n_slots) return;
  const int row = wsp<const int32_t>(ws, T.ws_rows)[slot];
  if (row < 0) return;
  const uint4 val = ld16(wsp<const bf16_t>(ws, T.ws_src) + (int64_t)slot * dm.d + 8 * ch);
  st16(o + T.o_off + (int64_t)row * dm.o_sl + 8 * ch, val);
}

hipError_t launch_unpermute(const Dims& dm, const Tables& tb, char* ws, void* o, int max_slots, hipStream_t s) {
  if (tb.n_unperm == 0) return hipSuccess;
  const int64_t n = (int64_t)max_slots * (dm.d / 8);
  k_unpermute<<<dim3((unsigned)((n + 255) / 256), (unsigned)tb.n_unperm), 256, 0, s>>>(dm, tb, ws, (bf16_t*)o);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Plan compile: one workgroup per (head, query tile).
// grid (max query tiles, heads), block 256, dynamic LDS = bitmap words.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bm_set(uint64_t* bm, int bit) {
  atomicOr((unsigned long long*)&bm[bit >> 6], 1ull << (bit & 63));
}
__device__ __forceinline__ bool bm_get(const uint64_t* bm, int bit) { return (bm[bit >> 6] >> (bit & 63)) & 1ull; }

// set bits [a, b] (inclusive), words split across the workgroup
__device__ __forceinline__ void bm_set_range(uint64_t* bm, int a, int b) {
  if (a > b) return;
  const int w0 = a >> 6, w1 = b >> 6;
  for (int w = w0 + (int)threadIdx.x; w <= w1; w += blockDim.x) {
    const int lo = max(a, w << 6) - (w << 6), hi = min(b, (w << 6) + 63) - (w << 6);
    const uint64_t m = (hi == 63 ? ~0ull : ((1ull << (hi + 1)) - 1)) & ~((1ull << lo) - 1);
    atomicOr((unsigned long long*)&bm[w], m);
  }
}

__device__ __forceinline__ int count_le(const int32_t* a, int n, int p) {   // entries <= p of an ascending array
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= p) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Index sets in original coordinates (plain, Q-boundary and per-segment
// vertical-slash heads): a selected diagonal at offset o = 64q + r crosses key
// tile t0 - q of a full query tile whose rows are 64t0 .. 64t0+63, and tile
// t0 - q - 1 too when r > 0.  Bit q of this per-index-set bitmap says whether
// some selected diagonal reaches key tile t0 - q; such a tile's key tiles are
// then a reversed shift of it (k_plan).  grid (estimation jobs), block 256,
// dynamic LDS = bitmap words.
//
// 2D-boundary index sets work in compacted coordinates (ranks within each
// modality) with signed offsets o = S - (n_k - 1) >= -(n_k - 1): the bitmap is
// taken over o + 64 * ceil((n_k - 1) / 64) >= 0, one per key modality (pair),
// and k_plan shifts by that many tiles more.
__global__ __launch_bounds__(256) void k_vs_shift(Tables tb, char* ws) {
  const EstJob& J = wsp<const EstJob>(ws, tb.off_jobs)[blockIdx.x];
  if (J.kind != JOB_VS_ORIG && J.kind != JOB_VS_2D) return;
  extern __shared__ uint64_t mb[];
  const int tid = threadIdx.x;
  for (int pi = 0; pi < J.n_pairs; ++pi) {
    const PairDev& Pd = J.pair[pi];
    if (Pd.ws_shift < 0) continue;
    const int SW = Pd.shift_words;
    for (int w = tid; w < SW; w += 256) mb[w] = 0ull;
    __syncthreads();
    const int ns = min(max(wsp<const int32_t>(ws, Pd.ws_nsel)[1], 0), Pd.ks);
    const int32_t* S = wsp<const int32_t>(ws, Pd.ws_sidx);
    const int shift = J.kind == JOB_VS_2D ? 64 * ((Pd.n_k - 1 + 63) >> 6) - (Pd.n_k - 1) : 0;
    for (int e = tid; e < ns; e += 256) {
      const int o = max(S[e] + shift, 0), q = o >> 6;
      if (q < 64 * SW) bm_set(mb, q);
      if ((o & 63) && q + 1 < 64 * SW) bm_set(mb, q + 1);
    }
    __syncthreads();
    uint64_t* out = wsp<uint64_t>(ws, Pd.ws_shift);
    for (int w = tid; w < SW; w += 256) out[w] = mb[w];
    __syncthreads();
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void k_plan(Dims dm, Tables tb, char* ws) {
  constexpr int NW = NT / 64;   // waves
  const int bh = blockIdx.y, t = blockIdx.x;
  const HeadDev& H = wsp<const HeadDev>(ws, tb.off_heads)[bh];
  if (t >= H.nT_rows) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  extern __shared__ uint64_t bm[];
  __shared__ int rows_s[64];
  __shared__ int red[8];
  __shared__ long long pred[4];
  __shared__ int sh_run_r0[64], sh_run_len[64], sh_nruns, sh_gpart;
  const int W = H.bm_words;
  const int32_t* pgrp = wsp<const int32_t>(ws, dm.ws_pgrp);

  for (int w = tid; w < W; w += NT) bm[w] = 0ull;
  int pos = -1;
  if (tid < 64) {
    const int slot = 64 * t + tid;
    if (H.row_kind == ROW_IDENTITY) pos = slot < dm.L ? slot : -1;
    else pos = wsp<const int32_t>(ws, H.ws_row_order)[slot];
    rows_s[tid] = pos;
  }
  // tile row statistics (wave 0)
  int qmin = 0x7fffffff, qmax = -1, nrows = 0;
  if (wv == 0) {
    int mn = pos >= 0 ? pos : 0x7fffffff, mx = pos, nv = pos >= 0 ? 1 : 0;
    for (int m = 1; m < 64; m <<= 1) {
      mn = min(mn, __shfl_xor(mn, m, 64));
      mx = max(mx, __shfl_xor(mx, m, 64));
      nv += __shfl_xor(nv, m, 64);
    }
    if (lane == 0) {
      red[0] = mn;
      red[1] = mx;
      red[2] = nv;
    }
  }
  __syncthreads();
  qmin = red[0];
  qmax = red[1];
  nrows = red[2];
  int4* info = wsp<int4>(ws, H.ws_info) + t;
  long long* pairs_out = wsp<long long>(ws, H.ws_pairs) + t;
  uint64_t* bm_out = wsp<uint64_t>(ws, H.ws_bm) + (int64_t)t * W;
  if (nrows == 0) {
    for (int w = tid; w < W; w += NT) bm_out[w] = 0ull;
    if (tid == 0) {
      *info = make_int4(0, 0, 0, 0);
      *pairs_out = 0;
    }
    return;
  }
  int g_cnt = 0;
  int32_t* gl = (H.gcap > 0) ? wsp<int32_t>(ws, H.ws_gather) + (int64_t)t * H.gcap : nullptr;
  // per-row pair counting needs, per pattern, different data
  int grid_nline = 0, grid_is_line = 0;
  const int32_t* grid_lines = nullptr;
  __syncthreads();

  if (H.pattern == MMSA_ASHAPE) {
    const int tmax = qmax >> 6;
    const int ns = min((H.sink + 63) / 64, tmax + 1);
    bm_set_range(bm, 0, ns - 1);
    bm_set_range(bm, max(0, qmin - H.window + 1) >> 6, tmax);
  } else if (H.pattern == MMSA_PARALLEL) {
    // the sink tiles, then every tile from the lowest first-visible key of the
    // tile's context and question rows up to its last row (sink rows need
    // only sink tiles)
    const int tmax = qmax >> 6;
    const int ns = min((H.sink + 63) / 64, tmax + 1);
    bm_set_range(bm, 0, ns - 1);
    if (wv == 0) {
      int lo = pos >= H.sink ? par_floor(H.sink, H.window, H.qstart, pos) : 0x7fffffff;
      for (int m = 1; m < 64; m <<= 1) lo = min(lo, __shfl_xor(lo, m, 64));
      if (lane == 0) red[3] = lo;
    }
    __syncthreads();
    if (red[3] != 0x7fffffff) bm_set_range(bm, red[3] >> 6, tmax);
  } else if (H.pattern == MMSA_BLOCK) {
    const int32_t* ci = wsp<const int32_t>(ws, H.ws_blk_idx) + (int64_t)t * H.k_blocks;
    for (int i = tid; i < H.k_blocks; i += NT) {
      const int c = ci[i];
      if (c >= 0) bm_set(bm, c);
    }
  } else if (H.pattern == MMSA_GRID) {
    const GridTask& G = wsp<const GridTask>(ws, tb.off_grid)[H.grid_task];
    grid_nline = min(max(wsp<const int32_t>(ws, G.ws_out)[2], 0), dm.L);
    const int nl_pad = (grid_nline + 63) & ~63;
    grid_is_line = (64 * t) < nl_pad;
    grid_lines = wsp<const int32_t>(ws, H.ws_row_order);
    if (grid_is_line) {
      bm_set_range(bm, 0, qmax >> 6);
    } else {
      // the line keys up to the tile's last row are gathered; a sink and a
      // local window add their key tiles (line keys inside those tiles are
      // masked out of the gathered chunks by the attention kernel)
      g_cnt = count_le(grid_lines, grid_nline, qmax);
      const int tmax = qmax >> 6;
      if (H.sink > 0) bm_set_range(bm, 0, min((H.sink + 63) / 64, tmax + 1) - 1);
      if (H.window > 0) bm_set_range(bm, max(0, qmin - H.window + 1) >> 6, tmax);
    }
  } else {  // vertical-slash family
    const bool twod = H.layout == MMSA_BOUNDARY_2D;
    const bool grouped_rows = H.row_kind == ROW_GROUPED;
    int m_q = MMSA_TEXT;
    if (grouped_rows) m_q = (64 * t >= dm.video_base && dm.n_video > 0 && (dm.video_base > 0 || dm.n_text == 0)) ? MMSA_VIDEO : MMSA_TEXT;
    int jidx = H.job[grouped_rows ? m_q : 0];
    if (H.row_kind == ROW_SEGMENT) {
      // the segment whose padded slots hold this tile, and its estimation job
      const SegDev* segs = wsp<const SegDev>(ws, tb.off_segs);
      int lo = 0, hi = (int)tb.n_segs - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (segs[mid].slot0 <= 64 * t) lo = mid;
        else hi = mid - 1;
      }
      jidx = wsp<const int32_t>(ws, tb.off_segjob)[H.segjob + lo];
    }
    const EstJob& J = wsp<const EstJob>(ws, tb.off_jobs)[jidx];
    // runs of the tile's rows in the slash coordinate (positions; ranks for 2D)
    if (tid == 0) {
      if (twod) {
        sh_nruns = 1;
        sh_run_r0[0] = 64 * t - (m_q == MMSA_VIDEO ? dm.video_base : dm.text_base);  // first rank
        sh_run_len[0] = nrows;
      } else {
        int nr = 0, r = 0;
        while (r < 64 && rows_s[r] >= 0) {
          int e = r + 1;
          while (e < 64 && rows_s[e] == rows_s[e - 1] + 1) ++e;
          sh_run_r0[nr] = rows_s[r];   // first position of the run
          sh_run_len[nr] = e - r;
          ++nr;
          r = e;
        }
        sh_nruns = nr;
      }
    }
    __syncthreads();
    const int nruns = sh_nruns;
    // a full tile whose rows are one run starting on a tile boundary (rows
    // 64t0 .. 64t0+63): its key tiles are the index set's shift bitmap
    // reversed and shifted by t0 (no per-diagonal work)
    const int64_t shift_off = twod ? -1 : J.pair[0].ws_shift;
    const bool shifted = shift_off >= 0 && nrows == 64 && nruns == 1 && (sh_run_r0[0] & 63) == 0;
    if (shifted) {
      const uint64_t* M = wsp<const uint64_t>(ws, shift_off);
      const int SW = J.pair[0].shift_words;
      const int t0 = sh_run_r0[0] >> 6;
      for (int w = tid; w < W; w += NT) {
        const int base = t0 - 64 * w - 63;   // bit b of word w (key tile 64w + b) <- shift bit t0 - 64w - b
        const int wi = base >> 6, sh = base & 63;
        uint64_t X = (wi >= 0 && wi < SW) ? M[wi] >> sh : 0ull;
        if (sh && wi + 1 >= 0 && wi + 1 < SW) X |= M[wi + 1] << (64 - sh);
        bm[w] = __builtin_bitreverse64(X);
      }
    }
    // a full 2D-boundary tile (64 consecutive ranks from a multiple of 64):
    // per key modality, the pair's shift bitmap reversed and shifted by the
    // tile's rank tile plus the offset shift, clipped to that modality's
    // key tiles of the grouped view
    bool shifted2 = twod && nrows == 64 && (sh_run_r0[0] & 63) == 0;
    for (int pi = 0; pi < J.n_pairs; ++pi) shifted2 = shifted2 && J.pair[pi].ws_shift >= 0;
    if (shifted2) {
      const int tr = sh_run_r0[0] >> 6;
      for (int pi = 0; pi < J.n_pairs; ++pi) {
        const PairDev& Pd = J.pair[pi];
        const uint64_t* M = wsp<const uint64_t>(ws, Pd.ws_shift);
        const int SW = Pd.shift_words;
        const int tb0 = (Pd.m_k == MMSA_VIDEO ? dm.video_base : dm.text_base) >> 6;
        const int ntk = (Pd.n_k + 63) >> 6;
        const int T = tr + ((Pd.n_k - 1 + 63) >> 6) + tb0;   // shift bit of view tile v: T - v
        for (int w = tid; w < W; w += NT) {
          const int lo = max(tb0, 64 * w), hi = min(tb0 + ntk, 64 * w + 64);
          if (lo >= hi) continue;
          const int base = T - 64 * w - 63;
          const int wi = base >> 6, sh = base & 63;
          uint64_t X = (wi >= 0 && wi < SW) ? M[wi] >> sh : 0ull;
          if (sh && wi + 1 >= 0 && wi + 1 < SW) X |= M[wi + 1] << (64 - sh);
          const uint64_t keep = (hi - 64 * w == 64 ? ~0ull : ((1ull << (hi - 64 * w)) - 1)) & ~((1ull << (lo - 64 * w)) - 1);
          bm[w] |= __builtin_bitreverse64(X) & keep;
        }
      }
      __syncthreads();
      // A partial last key tile of a modality: the bitmap cannot tell whether a
      // diagonal enters it before or after its last real key, so its bit is
      // decided from the diagonals themselves.
      for (int pi = 0; pi < J.n_pairs; ++pi) {
        const PairDev& Pd = J.pair[pi];
        if ((Pd.n_k & 63) == 0) continue;
        const int ns = min(max(wsp<const int32_t>(ws, Pd.ws_nsel)[1], 0), Pd.ks);
        const int32_t* S = wsp<const int32_t>(ws, Pd.ws_sidx);
        const int r_lo = Pd.n_k & ~63, r_hi = Pd.n_k - 1, a = sh_run_r0[0];
        int hit = 0;
        for (int e = tid; e < ns; e += NT) {
          const int o = S[e] - (Pd.n_k - 1);
          hit |= (a - o <= r_hi) && (a + 63 - o >= r_lo);
        }
        hit = __syncthreads_or(hit);
        if (tid == 0) {
          const int v = ((Pd.m_k == MMSA_VIDEO ? dm.video_base : dm.text_base) >> 6) + (Pd.n_k >> 6);
          if (hit) bm[v >> 6] |= 1ull << (v & 63);
          else bm[v >> 6] &= ~(1ull << (v & 63));
        }
        __syncthreads();
      }
    }
    for (int pi = 0; pi < ((shifted || shifted2) ? 0 : J.n_pairs); ++pi) {
      const PairDev& Pd = J.pair[pi];
      const int32_t* nsel = wsp<const int32_t>(ws, Pd.ws_nsel);
      const int ns = min(max(nsel[1], 0), Pd.ks);
      const int32_t* S = wsp<const int32_t>(ws, Pd.ws_sidx);
      const int tile_base = twod ? ((Pd.m_k == MMSA_VIDEO ? dm.video_base : dm.text_base) >> 6) : 0;
      for (int e = tid; e < ns; e += NT) {
        const int o = twod ? S[e] - (Pd.n_k - 1) : max(S[e], 0);
        for (int ru = 0; ru < nruns; ++ru) {
          const int a = sh_run_r0[ru], len = sh_run_len[ru];
          int khi = a + len - 1 - o, klo = a - o;
          if (twod) {
            khi = min(khi, Pd.n_k - 1);
            klo = max(klo, 0);
          } else {
            klo = max(klo, 0);
          }
          if (khi < klo) continue;
          for (int c = klo >> 6; c <= (khi >> 6); ++c) bm_set(bm, tile_base + c);
        }
      }
    }
    __syncthreads();
    if (twod) {
      // Drop view tiles whose first key comes after the tile's last row.  The
      // tiles of a modality part of the grouped view hold that modality's keys
      // by rank, so the first key of its k-th tile is the key of rank 64 k and
      // the kept tiles are the first ceil(n / 64), n = keys of the modality at
      // or before the last row, counted over the segments by wave 0.
      if (wv == 0) {
        const SegDev* segs = wsp<const SegDev>(ws, tb.off_segs);
        long long n_m[2] = {0, 0};
        for (int i = lane; i < (int)tb.n_segs; i += 64) {
          const SegDev sg = segs[i];
          const long long c = min((long long)sg.len, max(0ll, (long long)qmax + 1 - sg.start));
          n_m[sg.modality == MMSA_VIDEO ? 1 : 0] += c;
        }
        for (int m = 1; m < 64; m <<= 1) {
          n_m[0] += __shfl_xor(n_m[0], m, 64);
          n_m[1] += __shfl_xor(n_m[1], m, 64);
        }
        if (lane == 0) {
          red[4] = (int)((n_m[0] + 63) >> 6);
          red[5] = (int)((n_m[1] + 63) >> 6);
        }
      }
      __syncthreads();
      const int tt0 = dm.text_base >> 6, tv0 = dm.video_base >> 6;
      const int tt1 = tt0 + red[4], tv1 = tv0 + red[5];
      auto range_bits = [](int w, int a, int b) -> uint64_t {   // bits of word w in [a, b)
        const int lo = max(a, 64 * w) - 64 * w, hi = min(b, 64 * w + 64) - 64 * w;
        if (lo >= hi) return 0ull;
        return (hi == 64 ? ~0ull : ((1ull << hi) - 1)) & ~((1ull << lo) - 1);
      };
      for (int w = tid; w < W; w += NT) bm[w] &= range_bits(w, tt0, tt1) | range_bits(w, tv0, tv1);
      __syncthreads();
    }
    // gathered verticals not held by a listed tile, ascending per key modality
    int gbase = 0;
    for (int pi = 0; pi < J.n_pairs; ++pi) {
      const PairDev& Pd = J.pair[pi];
      const int nv = min(max(wsp<const int32_t>(ws, Pd.ws_nsel)[0], 0), Pd.kv);
      const int32_t* V = wsp<const int32_t>(ws, Pd.ws_vidx);
      const int kbase = twod ? (Pd.m_k == MMSA_VIDEO ? dm.video_base : dm.text_base) : 0;
      for (int s0 = 0; s0 < nv; s0 += NT) {
        const int e = s0 + tid;
        bool keep = false;
        int p = -1;
        if (e < nv) {
          const int c = V[e];
          const bool inr = c >= 0 && c < (twod ? Pd.n_k : dm.L);
          p = inr ? (twod ? pgrp[kbase + c] : c) : -1;
          const int vt = twod ? ((kbase + c) >> 6) : (c >> 6);
          keep = inr && p >= 0 && p <= qmax && !bm_get(bm, vt);
        }
        int tot;
        const int r = block_excl_count(keep, red, &tot);
        if (keep) gl[gbase + r] = p;
        gbase += tot;
      }
      if (pi == 0 && tid == 0) sh_gpart = gbase;
    }
    g_cnt = gbase;
    __syncthreads();
  }
  __syncthreads();

  // popcount prefix of the bitmap words (wpre[w]: set bits in words < w), so
  // a row's count of listed tiles below its own is one lookup, not a walk
  // over up to L/4096 words
  int* wpre = reinterpret_cast<int*>(bm + W);
  const bool use_pre = W > 16;   // short bitmaps: the walk is cheaper than the scan's barriers
  if (use_pre) {
    int carry = 0;
    for (int base = 0; base < W; base += NT) {
      const int w = base + tid;
      const int c = w < W ? __popcll(bm[w]) : 0;
      int tot;
      const int ex = block_excl_sum(c, red, &tot);
      if (w < W) wpre[w] = carry + ex;
      carry += tot;
    }
    if (tid == 0) wpre[W] = carry;
  }
  __syncthreads();
  auto popc_below = [&](int bit) -> int {   // set bits strictly below `bit`
    const int wl = bit >> 6;
    int c = 0;
    if (use_pre) {
      c = wpre[wl];
    } else {
      for (int w = 0; w < wl; ++w) c += __popcll(bm[w]);
    }
    return c + ((bit & 63) ? __popcll(bm[wl] & ((1ull << (bit & 63)) - 1)) : 0);
  };

  // exact selected pairs of each row
  long long my_pairs = 0;
  if (tid < 64 && pos >= 0) {
    const int p = pos;
    if (H.pattern == MMSA_ASHAPE) {
      my_pairs = min(p + 1, H.window) + max(0, min(H.sink, p + 1 - H.window));
    } else if (H.pattern == MMSA_PARALLEL) {
      // a context row: the sink block and its own block up to itself
      const bool ctx = p >= H.sink && p < H.qstart;
      my_pairs = ctx ? (long long)H.sink + (p - par_floor(H.sink, H.window, H.qstart, p) + 1) : (long long)(p + 1);
    } else if (H.pattern == MMSA_GRID) {
      const int lines_le_p = count_le(grid_lines, grid_nline, p);
      my_pairs = grid_is_line ? (p + 1) : lines_le_p;
      if (!grid_is_line && (H.sink > 0 || H.window > 0)) {
        // keys of the sink [0, s_end) and the window [w0, p] that are not line keys
        const int s_end = min(H.sink, p + 1);
        const int w0 = H.window > 0 ? max(0, p - H.window + 1) : p + 1;
        if (s_end >= w0) {
          my_pairs += (p + 1) - lines_le_p;
        } else {
          const int lines_in = count_le(grid_lines, grid_nline, s_end - 1) + lines_le_p -
                               count_le(grid_lines, grid_nline, w0 - 1);
          my_pairs += s_end + (p - w0 + 1) - lines_in;
        }
      }
    } else if (H.view_kind == VIEW_IDENTITY) {
      const int cp = p >> 6;
      my_pairs = 64ll * popc_below(cp) + (bm_get(bm, cp) ? (p - 64 * cp + 1) : 0);
      if (H.pattern == MMSA_VS) my_pairs += count_le(gl, g_cnt, p);
    } else {  // grouped key view (2D boundary)
      const int slot = wsp<const int32_t>(ws, dm.ws_gslot)[p];
      const bool vid = dm.n_video > 0 && slot >= dm.video_base && (dm.video_base > 0 || dm.n_text == 0);
      const int rank = vid ? slot - dm.video_base : slot - dm.text_base;
      const int kt = vid ? (p - rank) : (rank + 1);          // text keys <= p
      const int kv = (p + 1) - kt;                             // video keys <= p
      const int ntt = (dm.n_text + 63) >> 6;
      const int tb0 = dm.text_base >> 6, vb0 = dm.video_base >> 6;
      long long c = 0;
      if (kt > 0) {
        const int ct = kt >> 6;
        c += 64ll * (popc_below(tb0 + ct) - popc_below(tb0));
        if ((kt & 63) && ct < ntt && bm_get(bm, tb0 + ct)) c += kt & 63;
      }
      if (kv > 0) {
        const int ntv = (dm.n_video + 63) >> 6;
        const int cv = kv >> 6;
        c += 64ll * (popc_below(vb0 + cv) - popc_below(vb0));
        if ((kv & 63) && cv < ntv && bm_get(bm, vb0 + cv)) c += kv & 63;
      }
      const int gp = sh_gpart;
      c += count_le(gl, gp, p) + count_le(gl + gp, g_cnt - gp, p);
      my_pairs = c;
    }
  }
  for (int m = 1; m < 64; m <<= 1) my_pairs += __shfl_xor(my_pairs, m, 64);
  // tiles in the bitmap
  int nt = 0;
  for (int w = tid; w < W; w += NT) {
    nt += __popcll(bm[w]);
    bm_out[w] = bm[w];
  }
  for (int m = 1; m < 64; m <<= 1) nt += __shfl_xor(nt, m, 64);
  if (lane == 0) {
    red[wv] = nt;
    pred[wv] = my_pairs;
  }
  __syncthreads();
  if (tid == 0) {
    int ntiles = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) ntiles += red[i];
    const int cost = ntiles + (g_cnt + 63) / 64;
    *info = make_int4(ntiles, g_cnt, cost, nrows);
    *pairs_out = pred[0];
  }
}

// ---------------------------------------------------------------------------
// Attention work queue.  Items (head, pair of adjacent query tiles) are ordered
// by queue group (q heads sharing one b, KV head) and, within a group, by pair
// descending, then head: the most expensive pairs of a KV head come first, and
// the attention kernel deals the order round-robin to the XCDs (queue position
// e goes to XCD e % 8).
// Groups whose heads walk long key prefixes (a vertical-slash or grid head
// among them) are instead ordered by head, then pair descending, and dealt in
// runs of XCD_RUN consecutive pairs per XCD once the K/V of the KV head (4·L·d
// bytes) reach WALK_KV_BYTES: the workgroups running at one time then belong
// to one head, an XCD's workgroups walk neighbouring pairs and share key tiles
// in its L2, and the chip's advance through K/V stays within the 256 MB
// last-level cache.  Other groups switch to the head-major order, still dealt
// round-robin, only at HEAD_MAJOR_KV_BYTES (block heads select scattered
// tiles, parallel-encoding heads short local ones; runs make both slower).
// Runs are 128 pairs long when every head has at most 1024 pairs (each XCD
// then takes one contiguous eighth of a head), else XCD_RUN.
// Measured against the interleaved order: 128K 75.9 -> 73.4 ms (runs of 64;
// 128 took 1.6 % off that), 314K 169 -> 158 ms, 1M 3560 -> 3160 ms, the 256K
// block layer (head-major only) 52.9 -> 51.4 ms; with runs the 101K
// parallel-encoding layer took 11.4 ms, not 10.0.
// ---------------------------------------------------------------------------
constexpr int64_t WALK_KV_BYTES = 32ll << 20;
constexpr int64_t HEAD_MAJOR_KV_BYTES = 128ll << 20;
constexpr int XCD_RUN = 64;

// Queue position and cost of every (head, pair of adjacent query tiles).
// grid (pairs/64, heads).
__global__ __launch_bounds__(64) void k_queue_enum(Dims dm, Tables tb, char* ws) {
  const int bh = blockIdx.y;
  const HeadDev* heads = wsp<const HeadDev>(ws, tb.off_heads);
  const HeadDev& H = heads[bh];
  const int np = (H.nT_rows + 1) / 2;
  const int pr = blockIdx.x * 64 + threadIdx.x;
  if (pr >= np) return;
  const QGroup G = wsp<const QGroup>(ws, tb.off_qgroups)[H.qgroup];
  const int32_t* gh = wsp<const int32_t>(ws, tb.off_qgroup_heads);
  int64_t e = G.item_base;
  bool walk = false;
  for (int i = G.head_begin; i < G.head_end; ++i) {
    const int p = heads[gh[i]].pattern;
    walk = walk || p == MMSA_VS || p == MMSA_GRID;
  }
  const int64_t kv_bytes = 4ll * dm.L * dm.d;
  const bool runs = walk && kv_bytes >= WALK_KV_BYTES;
  if (runs || kv_bytes >= HEAD_MAJOR_KV_BYTES) {
    int64_t n = 0;
    for (int i = G.head_begin; i < G.head_end; ++i) {
      const int h2 = gh[i];
      const int np2 = (heads[h2].nT_rows + 1) / 2;
      if (h2 < bh) e += np2;                            // every item of an earlier head
      n += np2;
    }
    e += np - 1 - pr;                                   // larger pairs of this head
    // runs of `run` positions per XCD: within each whole block of 8 runs,
    // local position l = 8*run*sb + run*x + i moves to 8*run*sb + 8*i + x,
    // which the kernel deals to XCD x (the tail of the group keeps its order)
    int nmax = 0;
    for (int i = G.head_begin; i < G.head_end; ++i) nmax = max(nmax, (heads[gh[i]].nT_rows + 1) / 2);
    // heads of at most 8 runs of 128 pairs: one contiguous run per XCD and head
    const int run = nmax <= 8 * 128 ? 128 : XCD_RUN;
    const int64_t l = e - G.item_base, SB = 8ll * run;
    if (runs && l < n / SB * SB) {
      const int64_t sb = l / SB, rem = l % SB;
      e = G.item_base + sb * SB + (rem % run) * 8 + rem / run;
    }
  } else {
    for (int i = G.head_begin; i < G.head_end; ++i) {
      const int h2 = gh[i];
      const int np2 = (heads[h2].nT_rows + 1) / 2;
      e += max(0, np2 - 1 - pr);               // items of larger pairs
      if (h2 < bh && np2 > pr) e += 1;          // same pair, earlier head
    }
  }
  const int4 i0 = wsp<const int4>(ws, H.ws_info)[2 * pr];
  const int4 i1 = (2 * pr + 1 < H.nT_rows) ? wsp<const int4>(ws, H.ws_info)[2 * pr + 1] : make_int4(0, 0, 0, 0);
  const int c0 = i0.w > 0 ? i0.z : 0, c1 = i1.w > 0 ? i1.z : 0;
  // the union of the two tiles' chunks, estimated; a pair with rows but no
  // selected key still costs a visit (zero output)
  const int cost = max(c0, c1) + min(c0, c1) / 2;
  wsp<int32_t>(ws, dm.ws_enum_item)[e] = (bh << 16) | pr;
  wsp<int32_t>(ws, dm.ws_enum_cost)[e] = (i0.w > 0 || i1.w > 0) ? max(cost, 1) : 0;
}

// Per-XCD pop counters of the attention kernel back to zero.
__global__ __launch_bounds__(64) void k_queue_reset(Dims dm, char* ws) {
  int32_t* ctr = wsp<int32_t>(ws, dm.ws_ctr);
  if (threadIdx.x < N_XCD) ctr[threadIdx.x] = 0;
}

hipError_t launch_plan(const Dims& dm, const Tables& tb, char* ws, int max_tiles, int max_bm_words,
                       int max_shift_words, hipStream_t s) {
  if (max_tiles > 0 && tb.n_heads > 0) {
    if (tb.n_jobs > 0 && max_shift_words > 0)
      k_vs_shift<<<(unsigned)tb.n_jobs, 256, (size_t)max_shift_words * 8, s>>>(tb, ws);
    // dynamic LDS: the bitmap words, then their popcount prefix
    k_plan<64><<<dim3(max_tiles, (unsigned)tb.n_heads), 64, (size_t)max_bm_words * 12 + 4, s>>>(dm, tb, ws);
    k_queue_enum<<<dim3((max_tiles / 2 + 64) / 64, (unsigned)tb.n_heads), 64, 0, s>>>(dm, tb, ws);
  }
  return hipGetLastError();
}

hipError_t launch_queue_reset(const Dims& dm, char* ws, hipStream_t s) {
  k_queue_reset<<<1, 64, 0, s>>>(dm, ws);
  return hipGetLastError();
}

}  // namespace mmsa
