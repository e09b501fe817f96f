// Host side of libmmsa: argument validation, workspace layout, the tables the
// kernels read, and the five ABI entry points declared in include/mmsa.h.
//
// Everything here runs on the host before any HIP call, so an invalid
// descriptor is rejected without touching the device.  The tables (heads,
// estimation regions, tasks) are built from the descriptor once and kept in a
// small cache keyed by the descriptor's contents, so the five calls of a layer
// build them once; every call uploads them with one asynchronous copy to the
// start of the workspace.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "mmsa_internal.h"

using namespace mmsa;

// Device memory of mmsa_prefill_noalloc: the workspace of one layer whose
// mmsa_workspace_bytes() is at most MMSA_NOALLOC_SCRATCH_BYTES.  Each device
// the library runs on holds its own copy until the process ends; every
// mmsa_prefill_noalloc call on a device reuses it.
static __device__ __align__(256) char scratch[MMSA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

void set_err(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
}

int64_t pad_to(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Bump {
  int64_t off = 0;
  int64_t take(int64_t bytes) {
    off = pad_to(off, 256);
    const int64_t r = off;
    off += std::max<int64_t>(bytes, 0);
    return r;
  }
};

struct Seg {
  int64_t start, len;
  int modality, rank_start;
  int slot0;   // first slot in the segment-grouped order
};

struct Layout {
  Dims dm{};
  Tables tb{};
  int B = 0, Hq = 0, Hkv = 0, L = 0, d = 0, nT = 0, BH = 0;
  std::vector<int> kvmap;
  std::vector<mmsa_head_cfg> cfg;
  std::vector<Seg> segs;
  int n_mod[2] = {0, 0};
  std::vector<HeadDev> heads;
  std::vector<EstJob> jobs;
  std::vector<EstGroup> g1, g2;
  std::vector<TopkTask> topk;
  std::vector<GridTask> grids;
  std::vector<PoolTask> pools;
  std::vector<BlockTask> blocks;
  std::vector<GatherTask> gathers;
  std::vector<UnpermTask> unperms;
  std::vector<QGroup> qgroups;
  std::vector<int32_t> qgroup_heads;
  std::vector<char> blob;
  int64_t ws_total = 0;
  int n_chunks1 = 0, n_wg1 = 0, n_chunks2 = 0, n_wg2 = 0, max_ds = 0, max_strides = 0, nB = 0, max_tiles = 0, max_bm_words = 0;
  int max_gather_slots = 0, max_unperm_slots = 0, max_shift_words = 0;
  int64_t max_items = 0;
  int64_t max_topk_slices = 0;
  int64_t zero_off = 0, zero_bytes = 0;       // vertical scores and slash accumulators
  int64_t gridrow_off = 0, gridrow_bytes = 0; // grid row orders (filled with -1)
  bool need_seg = false, any_vs_est = false, any_block = false;
  bool need_pseg = false;                 // some head uses the segment-grouped row order
  std::vector<int32_t> segjob;            // per Q_SEGMENT head: the job of each segment
  bool empty = false;
  bool materialize = false;   // explicit gathers and output scatter (MMSA_FLAG_MATERIALIZE)
  // per (bh, part) index-set facts for mmsa_index_meta / views: job index and pair index
  std::vector<std::vector<std::pair<int, int>>> set_of;   // [bh][part] -> (job, pair) or (-1,-1)
};

// number of tokens of modality m at positions <= i
int64_t count_mod_le(const Layout& Lo, int m, int64_t i) {
  int64_t c = 0;
  for (const Seg& s : Lo.segs) {
    if (s.start > i) break;
    if (s.modality == m) c += std::min<int64_t>(s.len, i - s.start + 1);
  }
  return c;
}

// the last `count` positions of modality m, ascending
std::vector<int> last_positions(const Layout& Lo, int m, int count) {
  std::vector<int> out;
  for (int si = (int)Lo.segs.size() - 1; si >= 0 && (int)out.size() < count; --si) {
    const Seg& s = Lo.segs[si];
    if (s.modality != m) continue;
    for (int64_t p = s.start + s.len - 1; p >= s.start && (int)out.size() < count; --p) out.push_back((int)p);
  }
  std::reverse(out.begin(), out.end());
  return out;
}

void set_runs(EstJob& J) {
  J.n_runs = 0;
  int r = 0;
  while (r < J.n_rows) {
    int e = r + 1;
    while (e < J.n_rows && J.rows[e] == J.rows[e - 1] + 1) ++e;
    J.run_r0[J.n_runs] = r;
    J.run_len[J.n_runs] = e - r;
    ++J.n_runs;
    r = e;
  }
}

bool valid_combo(int pattern, int layout) {
  switch (pattern) {
    case MMSA_ASHAPE:
    case MMSA_PARALLEL:
    case MMSA_BLOCK: return layout == MMSA_PLAIN;
    case MMSA_VS:
      return layout == MMSA_PLAIN || layout == MMSA_Q_BOUNDARY || layout == MMSA_BOUNDARY_2D ||
             layout == MMSA_Q_SEGMENT;
    case MMSA_GRID: return layout == MMSA_PLAIN || layout == MMSA_MODALITY_GROUPED;
    default: return false;
  }
}

mmsa_status build_layout(const mmsa_layer_desc* desc, Layout& Lo) {
  if (!desc) {
    set_err("desc is NULL");
    return MMSA_INVALID_ARGUMENT;
  }
  const mmsa_layer_desc& D = *desc;
  if (D.B < 0 || D.L < 0 || D.Hq < 0 || D.Hkv < 0) {
    set_err("negative shape (B=%d Hq=%d Hkv=%d L=%d)", D.B, D.Hq, D.Hkv, D.L);
    return MMSA_INVALID_ARGUMENT;
  }
  if (D.d != 64 && D.d != 128) {
    set_err("head dimension d=%d is not supported (64 or 128)", D.d);
    return MMSA_UNSUPPORTED;
  }
  const uint32_t known = MMSA_FLAG_MATERIALIZE | MMSA_FLAG_DEBUG | MMSA_FLAG_KEYS_ASCENDING | MMSA_FLAG_KEYS_DESCENDING;
  if ((D.flags & ~known) != 0) {
    set_err("flags 0x%x hold bits outside the MMSA_FLAG_* set", D.flags);
    return MMSA_INVALID_ARGUMENT;
  }
  if ((D.flags & MMSA_FLAG_KEYS_ASCENDING) && (D.flags & MMSA_FLAG_KEYS_DESCENDING)) {
    set_err("MMSA_FLAG_KEYS_ASCENDING and MMSA_FLAG_KEYS_DESCENDING are exclusive");
    return MMSA_INVALID_ARGUMENT;
  }
  if (D.L >= (1 << 22)) {
    set_err("L=%d exceeds the supported 2^22 tokens", D.L);
    return MMSA_UNSUPPORTED;
  }
  if ((int64_t)D.B * D.Hq > 4096) {
    set_err("B*Hq=%lld exceeds 4096", (long long)D.B * D.Hq);
    return MMSA_UNSUPPORTED;
  }
  Lo.B = D.B;
  Lo.Hq = D.Hq;
  Lo.Hkv = D.Hkv;
  Lo.L = D.L;
  Lo.d = D.d;
  Lo.BH = D.B * D.Hq;
  Lo.nT = (D.L + TILE - 1) / TILE;
  if (D.Hq > 0 && D.Hkv <= 0) {
    set_err("Hkv must be >= 1");
    return MMSA_INVALID_ARGUMENT;
  }
  if (!(std::isfinite(D.scale)) || D.scale < 0.f) {
    set_err("scale must be finite and >= 0");
    return MMSA_INVALID_ARGUMENT;
  }
  const int64_t* st[4] = {D.q_strides, D.k_strides, D.v_strides, D.o_strides};
  const char* nm[4] = {"q", "k", "v", "o"};
  for (int i = 0; i < 4; ++i) {
    if (st[i][0] < 0 || st[i][1] < 0 || st[i][2] < D.d || (st[i][2] % 8) != 0 || (st[i][1] % 8) != 0 ||
        (st[i][0] % 8) != 0) {
      set_err("%s strides (%lld, %lld, %lld) must be non-negative multiples of 8 with row stride >= d", nm[i],
              (long long)st[i][0], (long long)st[i][1], (long long)st[i][2]);
      return MMSA_INVALID_ARGUMENT;
    }
  }
  // The attention kernel copies K and V rows through buffer views of one
  // (batch, KV head) slice with 32-bit offsets, and uses offset 2^31 as "past
  // the slice" for key slots without a token: every slice must stay below 2 GiB.
  for (int i = 1; i <= 2; ++i) {
    const int64_t slice = D.L > 0 ? (int64_t)(D.L - 1) * st[i][2] * 2 + 2ll * D.d : 0;
    if (slice >= (1ll << 31)) {
      set_err("one (batch, KV head) slice of %s spans %lld bytes (L=%d, row stride %lld); the limit is 2 GiB", nm[i],
              (long long)slice, D.L, (long long)st[i][2]);
      return MMSA_UNSUPPORTED;
    }
  }
  // heads
  Lo.kvmap.assign(D.Hq, 0);
  if (D.Hq > 0) {
    if (!D.heads) {
      set_err("heads is NULL");
      return MMSA_INVALID_ARGUMENT;
    }
    if (D.kv_head_of) {
      for (int h = 0; h < D.Hq; ++h) {
        if (D.kv_head_of[h] < 0 || D.kv_head_of[h] >= D.Hkv) {
          set_err("kv_head_of[%d]=%d out of range [0,%d)", h, D.kv_head_of[h], D.Hkv);
          return MMSA_INVALID_ARGUMENT;
        }
        Lo.kvmap[h] = D.kv_head_of[h];
      }
    } else {
      if (D.Hq % D.Hkv != 0) {
        set_err("Hq=%d is not a multiple of Hkv=%d and kv_head_of is NULL", D.Hq, D.Hkv);
        return MMSA_INVALID_ARGUMENT;
      }
      for (int h = 0; h < D.Hq; ++h) Lo.kvmap[h] = h / (D.Hq / D.Hkv);
    }
  }
  Lo.cfg.assign(D.heads, D.heads + D.Hq);
  for (int h = 0; h < D.Hq; ++h) {
    mmsa_head_cfg& c = Lo.cfg[h];
    if (!valid_combo(c.pattern, c.layout)) {
      set_err("head %d: pattern %d with layout %d is not a valid combination", h, c.pattern, c.layout);
      return MMSA_INVALID_ARGUMENT;
    }
    if (c.pattern == MMSA_ASHAPE && (c.sink < 0 || c.window < 1)) {
      set_err("head %d: A-shape needs sink >= 0 and window >= 1", h);
      return MMSA_INVALID_ARGUMENT;
    }
    if (c.pattern == MMSA_PARALLEL && (c.sink < 0 || c.window < 1 || c.question < 0)) {
      set_err("head %d: parallel encoding needs sink >= 0, window >= 1 and question >= 0", h);
      return MMSA_INVALID_ARGUMENT;
    }
    if (c.pattern == MMSA_VS && (c.k_vertical < 0 || c.k_slash < 0)) {
      set_err("head %d: negative vertical/slash budget", h);
      return MMSA_INVALID_ARGUMENT;
    }
    if (c.pattern == MMSA_BLOCK) {
      if (c.k_blocks < 0) {
        set_err("head %d: negative block budget", h);
        return MMSA_INVALID_ARGUMENT;
      }
      if (D.L > (1 << 20)) {
        set_err("head %d: BLOCK heads support L <= 2^20", h);
        return MMSA_UNSUPPORTED;
      }
    }
    if (c.pattern == MMSA_GRID) {
      if (c.sink < 0 || c.window < 0) {
        set_err("head %d: grid needs sink >= 0 and window >= 0", h);
        return MMSA_INVALID_ARGUMENT;
      }
      if (c.grid_clip == 0) c.grid_clip = 8;
      if (c.grid_phases < 1 || c.grid_phases > MAX_PHASES || c.stride_lo < 16 || c.stride_hi < c.stride_lo ||
          c.stride_hi > MAX_STRIDE || c.grid_clip < 1 || c.grid_clip > 64) {
        set_err("head %d: grid needs 1<=phases<=%d, 16<=stride_lo<=stride_hi<=%d, 1<=clip<=64", h, MAX_PHASES,
                MAX_STRIDE);
        return MMSA_INVALID_ARGUMENT;
      }
    }
  }
  // segments
  Lo.segs.clear();
  if (D.segs && D.n_segs > 0) {
    int64_t pos = 0;
    int rank[2] = {0, 0};
    for (int i = 0; i < D.n_segs; ++i) {
      const mmsa_segment& s = D.segs[i];
      if (s.start != pos || s.len <= 0 || (s.modality != MMSA_TEXT && s.modality != MMSA_VIDEO)) {
        set_err("segment %d (start %lld, len %lld, modality %d) does not continue the tiling of [0, L)", i,
                (long long)s.start, (long long)s.len, s.modality);
        return MMSA_INVALID_ARGUMENT;
      }
      Lo.segs.push_back(Seg{s.start, s.len, s.modality, rank[s.modality], 0});
      rank[s.modality] += (int)s.len;
      pos += s.len;
    }
    if (pos != D.L) {
      set_err("segments cover %lld tokens, L=%d", (long long)pos, D.L);
      return MMSA_INVALID_ARGUMENT;
    }
  } else if (D.n_segs < 0 || (D.n_segs > 0 && !D.segs)) {
    set_err("n_segs=%d with segs=%p", D.n_segs, (const void*)D.segs);
    return MMSA_INVALID_ARGUMENT;
  } else if (D.L > 0) {
    Lo.segs.push_back(Seg{0, D.L, MMSA_TEXT, 0, 0});
  }
  int64_t seg_slots = 0;
  for (Seg& s : Lo.segs) {
    Lo.n_mod[s.modality] += (int)s.len;
    s.slot0 = (int)seg_slots;
    seg_slots += pad_to(s.len, TILE);
  }

  Dims& dm = Lo.dm;
  dm.B = D.B;
  dm.Hq = D.Hq;
  dm.Hkv = D.Hkv;
  dm.L = D.L;
  dm.d = D.d;
  dm.nT = Lo.nT;
  dm.n_text = Lo.n_mod[MMSA_TEXT];
  dm.n_video = Lo.n_mod[MMSA_VIDEO];
  dm.text_base = 0;
  dm.video_base = (int)pad_to(dm.n_text, GRP_PAD);
  dm.L_grp = (int)(pad_to(dm.n_text, GRP_PAD) + pad_to(dm.n_video, GRP_PAD));
  dm.L_seg = (int)seg_slots;
  dm.scale = D.scale > 0.f ? D.scale : 1.0f / std::sqrt((float)D.d);
  dm.scale_log2 = dm.scale * 1.4426950408889634f;
  // Key tiles lowest first once one KV head's K/V (4·L·d bytes) exceed the
  // 256 MB last-level cache: the workgroups then enter each head's K/V
  // together from its start instead of each from its own diagonal (1M
  // tokens: 3186 -> 3086 ms; at 128K-314K, and on the 256K block layer, the
  // highest-first order measured equal or faster).
  dm.chunk_asc = 4ll * D.L * D.d > (256ll << 20) ? 1 : 0;
  if (D.flags & MMSA_FLAG_KEYS_ASCENDING) dm.chunk_asc = 1;
  if (D.flags & MMSA_FLAG_KEYS_DESCENDING) dm.chunk_asc = 0;
  dm.debug = (D.flags & MMSA_FLAG_DEBUG) ? 1 : 0;
  dm.q_sb = D.q_strides[0];
  dm.q_sh = D.q_strides[1];
  dm.q_sl = D.q_strides[2];
  dm.k_sb = D.k_strides[0];
  dm.k_sh = D.k_strides[1];
  dm.k_sl = D.k_strides[2];
  dm.v_sb = D.v_strides[0];
  dm.v_sh = D.v_strides[1];
  dm.v_sl = D.v_strides[2];
  dm.o_sb = D.o_strides[0];
  dm.o_sh = D.o_strides[1];
  dm.o_sl = D.o_strides[2];

  Lo.empty = (Lo.BH == 0 || D.L == 0);
  Lo.materialize = (D.flags & MMSA_FLAG_MATERIALIZE) != 0;
  if (Lo.empty) {
    Lo.ws_total = 256;
    return MMSA_OK;
  }

  // Work items pack a head and a pair of query tiles into 32 bits, the pair in
  // the low 16.  Per-segment heads pad every segment to 64 rows, so many short
  // segments can give such a head more pairs than that: refused here.
  for (int h = 0; h < D.Hq; ++h) {
    const mmsa_head_cfg& c = Lo.cfg[h];
    const int64_t tiles = dm.L_seg / TILE;
    if (c.pattern == MMSA_VS && c.layout == MMSA_Q_SEGMENT && (tiles + 1) / 2 > 0xffff) {
      set_err("head %d: its segments, each padded to 64 rows, make %lld query tiles; a head may have at most 131070",
              h, (long long)tiles);
      return MMSA_UNSUPPORTED;
    }
  }
  const int L = D.L, nT = Lo.nT;
  Lo.nB = nT;
  Lo.set_of.assign(Lo.BH, std::vector<std::pair<int, int>>(std::max<size_t>(4, Lo.segs.size()), {-1, -1}));
  // ---- heads, estimation jobs, tasks (offsets filled later) ----
  Lo.heads.resize(Lo.BH);
  for (int b = 0; b < D.B; ++b) {
    for (int h = 0; h < D.Hq; ++h) {
      const int bh = b * D.Hq + h;
      const mmsa_head_cfg& c = Lo.cfg[h];
      HeadDev& H = Lo.heads[bh];
      std::memset(&H, 0, sizeof H);
      H.b = b;
      H.h = h;
      H.g = Lo.kvmap[h];
      H.pattern = c.pattern;
      H.layout = c.layout;
      H.sink = c.sink;
      H.window = c.window;
      H.qstart = L - std::min(c.question, L);
      H.segjob = -1;
      H.k_blocks = std::min(c.k_blocks, Lo.nB);
      H.grid_task = -1;
      H.job[0] = H.job[1] = -1;
      H.q_off = b * dm.q_sb + h * dm.q_sh;
      H.k_off = b * dm.k_sb + H.g * dm.k_sh;
      H.v_off = b * dm.v_sb + H.g * dm.v_sh;
      H.o_off = b * dm.o_sb + h * dm.o_sh;
      H.ws_row_order = H.ws_qperm = H.ws_operm = H.ws_kgrp = H.ws_vgrp = -1;
      H.ws_gather = H.ws_blk_idx = H.ws_qp = H.ws_kp = H.ws_z = -1;
      H.row_kind = ROW_IDENTITY;
      H.view_kind = VIEW_IDENTITY;
      H.n_row_slots = nT * TILE;
      if (c.pattern == MMSA_VS && c.layout == MMSA_Q_SEGMENT) {
        H.row_kind = ROW_SEGMENT;
        H.n_row_slots = dm.L_seg;
        Lo.need_seg = Lo.need_pseg = true;
      }
      if (c.pattern == MMSA_VS && (c.layout == MMSA_Q_BOUNDARY || c.layout == MMSA_BOUNDARY_2D)) {
        H.row_kind = ROW_GROUPED;
        H.n_row_slots = dm.L_grp;
        if (c.layout == MMSA_BOUNDARY_2D) H.view_kind = VIEW_GROUPED;
        Lo.need_seg = true;
      }
      if (c.pattern == MMSA_GRID) {
        H.row_kind = ROW_GRID;
        H.n_row_slots = (int)pad_to(L, TILE) + TILE;
        if (c.layout == MMSA_MODALITY_GROUPED) Lo.need_seg = true;
      }
      H.nT_rows = H.n_row_slots / TILE;
      H.nT_view = H.view_kind == VIEW_GROUPED ? dm.L_grp / TILE : nT;
      H.bm_words = (H.nT_view + 63) / 64;
      if (c.pattern == MMSA_BLOCK) Lo.any_block = true;

      // estimation jobs
      auto new_job = [&](int kind, int view, int m_q, const std::vector<int>& rows) -> int {
        EstJob J;
        std::memset(&J, 0, sizeof J);
        J.bh = bh;
        J.kind = kind;
        J.view = view;
        J.m_q = m_q;
        J.n_rows = (int)rows.size();
        for (int i = 0; i < J.n_rows; ++i) J.rows[i] = rows[i];
        J.imax = rows.back();
        J.q_off = H.q_off;
        J.k_off = H.k_off;
        set_runs(J);
        Lo.jobs.push_back(J);
        return (int)Lo.jobs.size() - 1;
      };
      auto orig_pair = [&](EstJob& J) {
        PairDev& P = J.pair[0];
        std::memset(&P, 0, sizeof P);
        P.m_k = -1;
        P.Dv = L;
        P.Ds = L;
        P.n_k = L;
        P.v_lo = 0;
        P.v_hi = J.imax + 1;
        P.s_lo = 0;
        P.s_hi = J.imax + 1;
        P.kv = std::min(c.k_vertical, P.v_hi - P.v_lo);
        P.ks = std::min(c.k_slash, P.s_hi - P.s_lo);
        J.n_pairs = 1;
      };
      if (c.pattern == MMSA_VS) {
        Lo.any_vs_est = true;
        if (c.layout == MMSA_PLAIN) {
          std::vector<int> rows;
          for (int p = std::max(0, L - EST_ROWS); p < L; ++p) rows.push_back(p);
          const int j = new_job(JOB_VS_ORIG, VIEW_IDENTITY, -1, rows);
          orig_pair(Lo.jobs[j]);
          H.job[0] = j;
          Lo.set_of[bh][0] = {j, 0};
          H.gcap = Lo.jobs[j].pair[0].kv;
        } else if (c.layout == MMSA_Q_SEGMENT) {
          // one estimation per segment: its last 64 queries, in original
          // coordinates, for the rows of that segment
          int gcap = 0;
          H.segjob = (int)Lo.segjob.size();
          for (size_t si = 0; si < Lo.segs.size(); ++si) {
            const Seg& sg = Lo.segs[si];
            std::vector<int> rows;
            for (int64_t p = std::max<int64_t>(sg.start, sg.start + sg.len - EST_ROWS); p < sg.start + sg.len; ++p)
              rows.push_back((int)p);
            const int j = new_job(JOB_VS_ORIG, VIEW_IDENTITY, sg.modality, rows);
            orig_pair(Lo.jobs[j]);
            Lo.segjob.push_back(j);
            if (si == 0) H.job[0] = j;
            Lo.set_of[bh][si] = {j, 0};
            gcap = std::max(gcap, Lo.jobs[j].pair[0].kv);
          }
          H.gcap = gcap;
        } else {
          int gcap = 0;
          for (int m = 0; m < 2; ++m) {
            if (Lo.n_mod[m] == 0) continue;
            const std::vector<int> rows = last_positions(Lo, m, EST_ROWS);
            const bool twod = c.layout == MMSA_BOUNDARY_2D;
            const int j = new_job(twod ? JOB_VS_2D : JOB_VS_ORIG, twod ? VIEW_GROUPED : VIEW_IDENTITY, m, rows);
            EstJob& J = Lo.jobs[j];
            H.job[m] = j;
            if (!twod) {
              orig_pair(J);
              Lo.set_of[bh][m] = {j, 0};
              gcap = std::max(gcap, J.pair[0].kv);
            } else {
              const int n_q = Lo.n_mod[m];
              J.rho0 = n_q - J.n_rows;
              J.n_pairs = 0;
              int gsum = 0;
              for (int mk = 0; mk < 2; ++mk) {
                if (Lo.n_mod[mk] == 0) continue;
                PairDev& P = J.pair[J.n_pairs];
                std::memset(&P, 0, sizeof P);
                const int n_k = Lo.n_mod[mk];
                P.m_k = mk;
                P.n_k = n_k;
                P.Dv = n_k;
                P.Ds = n_q + n_k - 1;
                // candidates: columns and diagonals met by the causal part of the rows
                int lo = 1 << 30, hi = -1, vhi = 0;
                for (int r = 0; r < J.n_rows; ++r) {
                  const int nv = (int)count_mod_le(Lo, mk, J.rows[r]);
                  vhi = std::max(vhi, nv);
                  if (nv >= 1) {
                    const int rho = J.rho0 + r;
                    hi = std::max(hi, rho);
                    lo = std::min(lo, rho - nv + 1);
                  }
                }
                P.v_lo = 0;
                P.v_hi = vhi;
                if (hi >= 0) {
                  P.s_lo = lo + n_k - 1;
                  P.s_hi = hi + n_k;
                } else {
                  P.s_lo = P.s_hi = 0;
                }
                P.kv = std::min(c.k_vertical, P.v_hi - P.v_lo);
                P.ks = std::min(c.k_slash, P.s_hi - P.s_lo);
                gsum += P.kv;
                Lo.set_of[bh][2 * m + mk] = {j, J.n_pairs};
                ++J.n_pairs;
              }
              H.n_pairs = J.n_pairs;
              gcap = std::max(gcap, gsum);
            }
          }
          H.gcap = gcap;
        }
      } else if (c.pattern == MMSA_GRID) {
        const bool grouped = c.layout == MMSA_MODALITY_GROUPED;
        std::vector<int> rows;
        if (!grouped) {
          for (int p = std::max(0, L - EST_ROWS); p < L; ++p) rows.push_back(p);
        } else {
          rows = last_positions(Lo, MMSA_VIDEO, EST_ROWS);
          if ((int)rows.size() < EST_ROWS) {
            std::vector<int> t = last_positions(Lo, MMSA_TEXT, EST_ROWS - (int)rows.size());
            rows.insert(rows.end(), t.begin(), t.end());
            std::sort(rows.begin(), rows.end());
          }
        }
        const int j = new_job(grouped ? JOB_GRID_GROUPED : JOB_GRID_PLAIN, grouped ? VIEW_GROUPED : VIEW_IDENTITY,
                              -1, rows);
        EstJob& J = Lo.jobs[j];
        PairDev& P = J.pair[0];
        std::memset(&P, 0, sizeof P);
        P.m_k = -1;
        P.Dv = L;
        J.n_pairs = 1;
        H.job[0] = j;
        Lo.set_of[bh][0] = {j, 0};
        GridTask T;
        std::memset(&T, 0, sizeof T);
        T.job = j;
        T.bh = bh;
        int Dg;
        if (!grouped) {
          Dg = J.imax + 1;
        } else {
          const int64_t nt = count_mod_le(Lo, MMSA_TEXT, J.imax), nv = count_mod_le(Lo, MMSA_VIDEO, J.imax);
          int64_t mx = nt - 1;
          if (nv >= 1) mx = std::max<int64_t>(mx, dm.n_text + nv - 1);
          Dg = (int)mx + 1;
        }
        T.D = Dg;
        T.n_rows = J.n_rows;
        T.s_lo = std::min(c.stride_lo, Dg);
        T.s_hi = std::min(c.stride_hi, Dg);
        T.w = c.grid_phases;
        T.grouped = grouped ? 1 : 0;
        const long long capll = ((long long)c.grid_clip * T.n_rows * (1ll << 24)) / Dg;
        T.cap = capll;
        H.grid_task = (int)Lo.grids.size();
        Lo.grids.push_back(T);
        Lo.max_strides = std::max(Lo.max_strides, T.s_hi - T.s_lo + 1);
      }
    }
  }
  // ---- groups (jobs sorted by (b, g, view)) ----
  {
    std::vector<int> order(Lo.jobs.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b2) {
      const HeadDev& A = Lo.heads[Lo.jobs[a].bh];
      const HeadDev& Bq = Lo.heads[Lo.jobs[b2].bh];
      if (A.b != Bq.b) return A.b < Bq.b;
      if (A.g != Bq.g) return A.g < Bq.g;
      return Lo.jobs[a].view < Lo.jobs[b2].view;
    });
    std::vector<int> newidx(order.size());
    std::vector<EstJob> sorted;
    for (size_t i = 0; i < order.size(); ++i) {
      newidx[order[i]] = (int)i;
      sorted.push_back(Lo.jobs[order[i]]);
    }
    Lo.jobs.swap(sorted);
    for (HeadDev& H : Lo.heads)
      for (int m = 0; m < 2; ++m)
        if (H.job[m] >= 0) H.job[m] = newidx[H.job[m]];
    for (GridTask& T : Lo.grids) T.job = newidx[T.job];
    for (int32_t& j : Lo.segjob) j = newidx[j];
    for (auto& v : Lo.set_of)
      for (auto& pr : v)
        if (pr.first >= 0) pr.first = newidx[pr.first];
    for (size_t i = 0; i < Lo.jobs.size();) {
      const HeadDev& H0 = Lo.heads[Lo.jobs[i].bh];
      size_t e = i;
      while (e < Lo.jobs.size() && Lo.heads[Lo.jobs[e].bh].b == H0.b && Lo.heads[Lo.jobs[e].bh].g == H0.g) ++e;
      // pass 1: batches of at most EST1_JB jobs, sizes as equal as possible
      const int nj = (int)(e - i), nb = (nj + EST1_JB - 1) / EST1_JB;
      for (int bi = 0; bi < nb; ++bi) {
        const int j0 = (int)i + bi * nj / nb, j1 = (int)i + (bi + 1) * nj / nb;
        EstGroup G1{H0.b, H0.g, 0, j0, j1, L, H0.k_off, -1, 0, 0};
        Lo.g1.push_back(G1);
      }
      for (size_t s = i; s < e;) {
        size_t f = s;
        while (f < e && Lo.jobs[f].view == Lo.jobs[s].view) ++f;
        const int view = Lo.jobs[s].view;
        // pass 2: batches of at most EST2_JB jobs of one key view
        const int nv = (int)(f - s), nb2 = (nv + EST2_JB - 1) / EST2_JB;
        for (int bi = 0; bi < nb2; ++bi) {
          const int j0 = (int)s + bi * nv / nb2, j1 = (int)s + (bi + 1) * nv / nb2;
          EstGroup G2{H0.b, H0.g, view, j0, j1, view == VIEW_GROUPED ? dm.L_grp : L, H0.k_off, -1, 0, 0};
          Lo.g2.push_back(G2);
        }
        s = f;
      }
      i = e;
    }
  }
  Lo.n_chunks1 = (L + EST_CK - 1) / EST_CK;
  // Workgroups of each estimation batch: EST1_WG per pass in all (one wave of
  // two workgroups per CU), shared in proportion to each batch's work (jobs x
  // key chunks it reads) by largest remainders, at least one each and at most
  // one per chunk.  Equal batches (the usual case) get equal counts; when
  // those are multiples of 8, workgroup x of every batch of a KV head runs on
  // the same XCD and their reads of a key chunk meet in its L2.
  auto spread = [&](std::vector<EstGroup>& gs, int& total) {
    const size_t n = gs.size();
    std::vector<double> work(n);
    std::vector<int> cap(n);
    double sum = 0;
    for (size_t i = 0; i < n; ++i) {
      int imax = -1;
      for (int j = gs[i].job_begin; j < gs[i].job_end; ++j) imax = std::max(imax, Lo.jobs[j].imax);
      const int all = (gs[i].n_keys + EST_CK - 1) / EST_CK;
      const int chunks = gs[i].view == VIEW_GROUPED ? all : std::min(all, imax / EST_CK + 1);
      work[i] = (double)(gs[i].job_end - gs[i].job_begin) * std::max(chunks, 1);
      cap[i] = std::max(all, 1);
      sum += work[i];
    }
    std::vector<int> cnt(n);
    std::vector<std::pair<double, size_t>> rem;
    int used = 0;
    for (size_t i = 0; i < n; ++i) {
      const double share = EST1_WG * work[i] / std::max(sum, 1.0);
      cnt[i] = std::min(cap[i], std::max(1, (int)share));
      used += cnt[i];
      rem.push_back({share - (int)share, i});
    }
    std::sort(rem.begin(), rem.end(), [](const auto& a, const auto& b) { return a.first > b.first || (a.first == b.first && a.second < b.second); });
    for (size_t r = 0; r < rem.size() && used < EST1_WG; ++r) {
      const size_t i = rem[r].second;
      if (cnt[i] < cap[i]) {
        ++cnt[i];
        ++used;
      }
    }
    total = 0;
    for (size_t i = 0; i < n; ++i) {
      gs[i].wg0 = total;
      gs[i].nwg = cnt[i];
      total += cnt[i];
    }
  };
  spread(Lo.g1, Lo.n_wg1);
  spread(Lo.g2, Lo.n_wg2);
  for (const EstGroup& G : Lo.g1)
    for (int j = G.job_begin; j < G.job_end; ++j) Lo.jobs[j].n_part1 = G.nwg;
  Lo.n_chunks2 = (std::max(L, dm.L_grp) + EST_CK - 1) / EST_CK;

  // ---- queue groups: q heads sharing one (b, KV head) ----
  {
    int64_t base = 0;
    for (int b = 0; b < D.B; ++b) {
      for (int g = 0; g < D.Hkv; ++g) {
        QGroup G{(int32_t)Lo.qgroup_heads.size(), 0, base};
        for (int h = 0; h < D.Hq; ++h) {
          if (Lo.kvmap[h] != g) continue;
          const int bh = b * D.Hq + h;
          Lo.heads[bh].qgroup = (int32_t)Lo.qgroups.size();
          Lo.qgroup_heads.push_back(bh);
          base += (Lo.heads[bh].nT_rows + 1) / 2;   // queue items are pairs of query tiles
        }
        G.head_end = (int32_t)Lo.qgroup_heads.size();
        if (G.head_end > G.head_begin) Lo.qgroups.push_back(G);
      }
    }
  }

  // ---- sizes of the uploaded tables ----
  Tables& tb = Lo.tb;
  tb.n_heads = Lo.BH;
  tb.n_jobs = (int64_t)Lo.jobs.size();
  tb.n_groups1 = (int64_t)Lo.g1.size();
  tb.n_groups2 = (int64_t)Lo.g2.size();
  tb.n_grid = (int64_t)Lo.grids.size();
  tb.n_segs = (int64_t)Lo.segs.size();
  // topk / pool / block / gather / unpermute task counts are known once offsets exist; reserve the maxima
  int64_t n_topk = 0;
  for (const EstJob& J : Lo.jobs)
    if (J.kind == JOB_VS_ORIG || J.kind == JOB_VS_2D) n_topk += 2 * J.n_pairs;
  int64_t n_block = 0, n_perm = 0;
  std::vector<int> kv_pool, kv_grp;   // (b*Hkv + g) needing pooled K / grouped K,V
  for (const HeadDev& H : Lo.heads) {
    if (H.pattern == MMSA_BLOCK) {
      ++n_block;
      kv_pool.push_back(H.b * D.Hkv + H.g);
    }
    if (Lo.materialize && H.row_kind != ROW_IDENTITY) ++n_perm;
    if (Lo.materialize && H.view_kind == VIEW_GROUPED) kv_grp.push_back(H.b * D.Hkv + H.g);
  }
  std::sort(kv_pool.begin(), kv_pool.end());
  kv_pool.erase(std::unique(kv_pool.begin(), kv_pool.end()), kv_pool.end());
  std::sort(kv_grp.begin(), kv_grp.end());
  kv_grp.erase(std::unique(kv_grp.begin(), kv_grp.end()), kv_grp.end());
  tb.n_topk = n_topk;
  tb.n_pool = n_block + (int64_t)kv_pool.size();
  tb.n_block = n_block;
  tb.n_gather = n_perm + 2 * (int64_t)kv_grp.size();
  tb.n_unperm = n_perm;
  tb.n_qgroups = (int64_t)Lo.qgroups.size();
  tb.n_segjob = (int64_t)Lo.segjob.size();

  Bump bp;
  tb.off_heads = bp.take((int64_t)sizeof(HeadDev) * tb.n_heads);
  tb.off_jobs = bp.take((int64_t)sizeof(EstJob) * tb.n_jobs);
  tb.off_groups1 = bp.take((int64_t)sizeof(EstGroup) * tb.n_groups1);
  tb.off_groups2 = bp.take((int64_t)sizeof(EstGroup) * tb.n_groups2);
  tb.off_topk = bp.take((int64_t)sizeof(TopkTask) * tb.n_topk);
  tb.off_grid = bp.take((int64_t)sizeof(GridTask) * tb.n_grid);
  tb.off_segs = bp.take((int64_t)sizeof(SegDev) * tb.n_segs);
  tb.off_pool = bp.take((int64_t)sizeof(PoolTask) * tb.n_pool);
  tb.off_block = bp.take((int64_t)sizeof(BlockTask) * tb.n_block);
  tb.off_gather = bp.take((int64_t)sizeof(GatherTask) * tb.n_gather);
  tb.off_unperm = bp.take((int64_t)sizeof(UnpermTask) * tb.n_unperm);
  tb.off_qgroups = bp.take((int64_t)sizeof(QGroup) * tb.n_qgroups);
  tb.off_qgroup_heads = bp.take((int64_t)sizeof(int32_t) * (int64_t)Lo.qgroup_heads.size());
  tb.off_segjob = bp.take((int64_t)sizeof(int32_t) * tb.n_segjob);
  const int64_t blob_bytes = pad_to(bp.off, 256);

  // ---- device buffers ----
  const int dd = D.d;
  dm.ws_flag = bp.take(256);
  dm.ws_pgrp = bp.take(4ll * std::max(dm.L_grp, 1));
  dm.ws_gslot = bp.take(4ll * L);
  dm.ws_pseg = Lo.need_pseg ? bp.take(4ll * std::max(dm.L_seg, 1)) : -1;
  for (const HeadDev& H : Lo.heads) Lo.max_items += (H.nT_rows + 1) / 2;
  dm.n_items = Lo.max_items;
  dm.ws_enum_item = bp.take(4 * Lo.max_items);
  dm.ws_enum_cost = bp.take(4 * Lo.max_items);
  dm.ws_ctr = bp.take(4 * N_XCD);
  // estimation: stats and partials
  for (EstJob& J : Lo.jobs) {
    J.ws_stats = bp.take(8ll * EST_ROWS);
    J.ws_part = bp.take(8ll * EST_ROWS * std::max(J.n_part1, 1));
  }
  // zero region: vertical scores and slash accumulators
  bp.off = pad_to(bp.off, 256);
  Lo.zero_off = bp.off;
  for (EstJob& J : Lo.jobs) {
    for (int pi = 0; pi < J.n_pairs; ++pi) {
      PairDev& P = J.pair[pi];
      P.ws_v = bp.take(4ll * P.Dv);
      P.ws_sacc = P.Ds > 0 ? bp.take(8ll * P.Ds) : -1;
    }
  }
  bp.off = pad_to(bp.off, 256);
  Lo.zero_bytes = bp.off - Lo.zero_off;
  for (EstJob& J : Lo.jobs) {
    for (int pi = 0; pi < J.n_pairs; ++pi) {
      PairDev& P = J.pair[pi];
      if (J.kind == JOB_VS_ORIG || J.kind == JOB_VS_2D) {
        P.ws_s = bp.take(4ll * P.Ds);
        // shift bitmap of the index set: bits up to the last query tile of
        // the region's modality plus the shift that makes 2D-boundary offsets
        // non-negative (a diagonal further out reaches no key tile), and two
        // more
        {
          const int64_t n_q = J.kind == JOB_VS_2D ? Lo.n_mod[J.m_q] : L;
          const int64_t offt = J.kind == JOB_VS_2D ? (P.n_k - 1 + 63) / 64 : 0;
          P.shift_words = (int)(((n_q + 63) / 64 + offt + 2 + 63) / 64);
          P.ws_shift = bp.take(8ll * P.shift_words);
          Lo.max_shift_words = std::max(Lo.max_shift_words, P.shift_words);
        }
        P.ws_vidx = bp.take(4ll * std::max(P.kv, 1));
        P.ws_sidx = bp.take(4ll * std::max(P.ks, 1));
        P.ws_nsel = bp.take(8);
        Lo.max_ds = std::max(Lo.max_ds, P.Ds);
        Lo.topk.push_back(TopkTask{P.ws_v, P.ws_vidx, P.ws_nsel, P.v_lo, P.v_hi, P.kv, 0,
                                   bp.take(topk_tmp_bytes(P.v_hi - P.v_lo))});
        Lo.topk.push_back(TopkTask{P.ws_s, P.ws_sidx, P.ws_nsel + 4, P.s_lo, P.s_hi, P.ks, 0,
                                   bp.take(topk_tmp_bytes(P.s_hi - P.s_lo))});
        Lo.max_topk_slices = std::max<int64_t>(Lo.max_topk_slices, std::max(topk_slices(P.v_hi - P.v_lo),
                                                                            topk_slices(P.s_hi - P.s_lo)));
      } else {
        P.ws_s = P.ws_vidx = P.ws_sidx = P.ws_nsel = P.ws_shift = -1;
        P.shift_words = 0;
      }
    }
  }
  for (GridTask& T : Lo.grids) {
    T.ws_v = Lo.jobs[T.job].pair[0].ws_v;
    T.ws_U = bp.take(8);
    T.ws_u = bp.take(4ll * std::max(T.D, 1));
    T.ws_cand = bp.take(16ll * MAX_PHASES * std::max(T.s_hi - T.s_lo + 1, 1));
    T.ws_out = bp.take(4ll * GRID_OUT);
  }
  // blocks
  {
    std::vector<int64_t> kp_off(kv_pool.size());
    for (size_t i = 0; i < kv_pool.size(); ++i) {
      kp_off[i] = bp.take(4ll * Lo.nB * dd);
      const int b = kv_pool[i] / D.Hkv, g = kv_pool[i] % D.Hkv;
      Lo.pools.push_back(PoolTask{b * dm.k_sb + g * dm.k_sh, dm.k_sl, kp_off[i], 1, 0});
    }
    for (HeadDev& H : Lo.heads) {
      if (H.pattern != MMSA_BLOCK) continue;
      H.ws_qp = bp.take(4ll * Lo.nB * dd);
      H.ws_z = bp.take(4ll * Lo.nB * Lo.nB);
      H.ws_blk_idx = bp.take(4ll * Lo.nB * std::max(H.k_blocks, 1));
      const int key = H.b * D.Hkv + H.g;
      const size_t pi = std::lower_bound(kv_pool.begin(), kv_pool.end(), key) - kv_pool.begin();
      H.ws_kp = kp_off[pi];
      Lo.pools.push_back(PoolTask{H.q_off, dm.q_sl, H.ws_qp, 0, 0});
      Lo.blocks.push_back(BlockTask{(int)(&H - &Lo.heads[0]), H.k_blocks, H.ws_qp, H.ws_kp, H.ws_z, H.ws_blk_idx});
    }
  }
  // permutation buffers
  bp.off = pad_to(bp.off, 256);
  Lo.gridrow_off = bp.off;
  for (HeadDev& H : Lo.heads)
    if (H.row_kind == ROW_GRID) H.ws_row_order = bp.take(4ll * H.n_row_slots);
  bp.off = pad_to(bp.off, 256);
  Lo.gridrow_bytes = bp.off - Lo.gridrow_off;
  {
    std::vector<int64_t> kg_off(kv_grp.size()), vg_off(kv_grp.size());
    for (size_t i = 0; i < kv_grp.size(); ++i) {
      kg_off[i] = bp.take(2ll * dm.L_grp * dd);
      vg_off[i] = bp.take(2ll * dm.L_grp * dd);
      const int b = kv_grp[i] / D.Hkv, g = kv_grp[i] % D.Hkv;
      Lo.gathers.push_back(GatherTask{b * dm.k_sb + g * dm.k_sh, dm.k_sl, dm.ws_pgrp, kg_off[i], dm.L_grp, 1});
      Lo.gathers.push_back(GatherTask{b * dm.v_sb + g * dm.v_sh, dm.v_sl, dm.ws_pgrp, vg_off[i], dm.L_grp, 2});
      Lo.max_gather_slots = std::max(Lo.max_gather_slots, dm.L_grp);
    }
    for (HeadDev& H : Lo.heads) {
      if (H.row_kind == ROW_GROUPED) H.ws_row_order = dm.ws_pgrp;
      if (H.row_kind == ROW_SEGMENT) H.ws_row_order = dm.ws_pseg;
      if (Lo.materialize && H.row_kind != ROW_IDENTITY) {
        H.ws_qperm = bp.take(2ll * H.n_row_slots * dd);
        H.ws_operm = bp.take(2ll * H.n_row_slots * dd);
        Lo.gathers.push_back(GatherTask{H.q_off, dm.q_sl, H.ws_row_order, H.ws_qperm, H.n_row_slots, 0});
        Lo.unperms.push_back(UnpermTask{H.ws_operm, H.ws_row_order, H.o_off, H.n_row_slots, 0});
        Lo.max_gather_slots = std::max(Lo.max_gather_slots, H.n_row_slots);
        Lo.max_unperm_slots = std::max(Lo.max_unperm_slots, H.n_row_slots);
      }
      if (Lo.materialize && H.view_kind == VIEW_GROUPED) {
        const int key = H.b * D.Hkv + H.g;
        const size_t i = std::lower_bound(kv_grp.begin(), kv_grp.end(), key) - kv_grp.begin();
        H.ws_kgrp = kg_off[i];
        H.ws_vgrp = vg_off[i];
      }
    }
  }
  // plans
  for (HeadDev& H : Lo.heads) {
    H.ws_bm = bp.take(8ll * H.nT_rows * H.bm_words);
    H.ws_info = bp.take(16ll * H.nT_rows);
    H.ws_pairs = bp.take(8ll * H.nT_rows);
    if (H.gcap > 0) H.ws_gather = bp.take(4ll * H.nT_rows * H.gcap);
    Lo.max_tiles = std::max(Lo.max_tiles, H.nT_rows);
    Lo.max_bm_words = std::max(Lo.max_bm_words, H.bm_words);
  }
  Lo.ws_total = pad_to(bp.off, 256);

  // ---- serialize the tables ----
  Lo.blob.assign(blob_bytes, 0);
  auto put = [&](int64_t off, const void* src, size_t bytes) {
    if (bytes) std::memcpy(Lo.blob.data() + off, src, bytes);
  };
  std::vector<SegDev> sd;
  for (const Seg& s : Lo.segs) sd.push_back(SegDev{s.start, s.len, s.modality, s.rank_start, s.slot0, 0});
  put(tb.off_heads, Lo.heads.data(), sizeof(HeadDev) * Lo.heads.size());
  put(tb.off_jobs, Lo.jobs.data(), sizeof(EstJob) * Lo.jobs.size());
  put(tb.off_groups1, Lo.g1.data(), sizeof(EstGroup) * Lo.g1.size());
  put(tb.off_groups2, Lo.g2.data(), sizeof(EstGroup) * Lo.g2.size());
  put(tb.off_topk, Lo.topk.data(), sizeof(TopkTask) * Lo.topk.size());
  put(tb.off_grid, Lo.grids.data(), sizeof(GridTask) * Lo.grids.size());
  put(tb.off_segs, sd.data(), sizeof(SegDev) * sd.size());
  put(tb.off_pool, Lo.pools.data(), sizeof(PoolTask) * Lo.pools.size());
  put(tb.off_block, Lo.blocks.data(), sizeof(BlockTask) * Lo.blocks.size());
  put(tb.off_gather, Lo.gathers.data(), sizeof(GatherTask) * Lo.gathers.size());
  put(tb.off_unperm, Lo.unperms.data(), sizeof(UnpermTask) * Lo.unperms.size());
  put(tb.off_qgroups, Lo.qgroups.data(), sizeof(QGroup) * Lo.qgroups.size());
  put(tb.off_qgroup_heads, Lo.qgroup_heads.data(), sizeof(int32_t) * Lo.qgroup_heads.size());
  put(tb.off_segjob, Lo.segjob.data(), sizeof(int32_t) * Lo.segjob.size());
  return MMSA_OK;
}

// Layouts of recently seen descriptors.  A layout is a pure function of the
// descriptor's values and of the arrays it points to (head configurations,
// segments, KV-head map), so the key is those bytes; equal keys give the same
// layout.  Descriptors the key cannot be read from safely (NULL arrays, sizes
// out of range) and invalid descriptors are not cached: build_layout reports
// them.  Entries are shared: one that is evicted stays alive for the calls
// still holding it.
constexpr int LAYOUT_CACHE_SIZE = 16;

bool layout_key(const mmsa_layer_desc* desc, std::string& key) {
  if (!desc) return false;
  const mmsa_layer_desc& D = *desc;
  if (D.Hq < 0 || D.Hq > 4096 || D.n_segs < 0 || D.n_segs > (1 << 20)) return false;
  if (D.Hq > 0 && !D.heads) return false;
  if (D.n_segs > 0 && !D.segs) return false;
  key.clear();
  key.reserve(128 + sizeof(mmsa_head_cfg) * D.Hq + 24ll * D.n_segs + 4ll * D.Hq);
  auto put = [&](const void* p, size_t n) { key.append(static_cast<const char*>(p), n); };
  const int32_t dims[6] = {D.B, D.Hq, D.Hkv, D.L, D.d, D.n_segs};
  put(dims, sizeof dims);
  put(D.q_strides, sizeof D.q_strides);
  put(D.k_strides, sizeof D.k_strides);
  put(D.v_strides, sizeof D.v_strides);
  put(D.o_strides, sizeof D.o_strides);
  put(&D.scale, sizeof D.scale);
  put(&D.flags, sizeof D.flags);
  if (D.Hq > 0) put(D.heads, sizeof(mmsa_head_cfg) * (size_t)D.Hq);   // twelve int32, no padding
  for (int i = 0; i < D.n_segs; ++i) {
    put(&D.segs[i].start, sizeof(int64_t));
    put(&D.segs[i].len, sizeof(int64_t));
    put(&D.segs[i].modality, sizeof(int32_t));
  }
  const char has_map = D.kv_head_of ? 1 : 0;
  put(&has_map, 1);
  if (D.kv_head_of && D.Hq > 0) put(D.kv_head_of, sizeof(int32_t) * (size_t)D.Hq);
  return true;
}

mmsa_status get_layout(const mmsa_layer_desc* desc, std::shared_ptr<const Layout>& out) {
  struct Entry {
    std::string key;
    std::shared_ptr<const Layout> lo;
    uint64_t used;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  static uint64_t clock = 0;
  std::string key;
  const bool keyed = layout_key(desc, key);
  if (keyed) {
    std::lock_guard<std::mutex> lock(mu);
    for (Entry& e : cache)
      if (e.key == key) {
        e.used = ++clock;
        out = e.lo;
        return MMSA_OK;
      }
  }
  auto lo = std::make_shared<Layout>();
  const mmsa_status st = build_layout(desc, *lo);
  if (st != MMSA_OK) return st;
  out = lo;
  if (keyed) {
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() < LAYOUT_CACHE_SIZE) {
      cache.push_back(Entry{std::move(key), out, ++clock});
    } else {
      auto lru = std::min_element(cache.begin(), cache.end(),
                                  [](const Entry& a, const Entry& b) { return a.used < b.used; });
      *lru = Entry{std::move(key), out, ++clock};
    }
  }
  return MMSA_OK;
}

mmsa_status check_ptr(const void* p, const char* name) {
  if (!p) {
    set_err("%s is NULL", name);
    return MMSA_INVALID_ARGUMENT;
  }
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) {
    set_err("%s is not 16-byte aligned", name);
    return MMSA_UNSUPPORTED;
  }
  return MMSA_OK;
}

mmsa_status prepare(const mmsa_layer_desc* desc, void* ws, size_t ws_bytes, std::shared_ptr<const Layout>& lo) {
  mmsa_status st = get_layout(desc, lo);
  if (st != MMSA_OK) return st;
  const Layout& Lo = *lo;
  if (Lo.empty) return MMSA_OK;
  if (!ws) {
    set_err("workspace is NULL");
    return MMSA_INVALID_ARGUMENT;
  }
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) {
    set_err("workspace is not 256-byte aligned");
    return MMSA_UNSUPPORTED;
  }
  if ((int64_t)ws_bytes < Lo.ws_total) {
    set_err("workspace has %zu bytes, %lld needed", ws_bytes, (long long)Lo.ws_total);
    return MMSA_WORKSPACE_TOO_SMALL;
  }
  return MMSA_OK;
}

mmsa_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MMSA_OK;
  set_err("%s: %s", where, hipGetErrorString(e));
  return MMSA_HIP_ERROR;
}

// Architecture and compute-unit count of each device, looked up once.  The
// kernels use gfx950-only instructions (32x32x16 bf16 MFMA, buffer-to-LDS
// copies, LDS transpose reads, permlane swaps), so any other device is refused
// before anything is enqueued.
struct DevInfo {
  int state = 0;   // 0 unknown, 1 gfx950, -1 another architecture
  int n_cu = 0;
  char arch[64] = {0};
  void* scratch = nullptr;   // this device's copy of `scratch` (mmsa_prefill_noalloc)
};

mmsa_status check_device(int* n_cu_out = nullptr, void** scratch_out = nullptr) {
  static std::mutex mu;
  static std::vector<DevInfo> info;
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    set_err("no gfx950 device: %s", hipGetErrorString(e));
    return MMSA_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(mu);
  if ((int)info.size() <= dev) info.resize(dev + 1);
  DevInfo& di = info[dev];
  if (di.state == 0) {
    hipDeviceProp_t p;
    const hipError_t e2 = hipGetDeviceProperties(&p, dev);
    if (e2 != hipSuccess) {
      set_err("device %d properties: %s", dev, hipGetErrorString(e2));
      return MMSA_HIP_ERROR;
    }
    std::snprintf(di.arch, sizeof di.arch, "%s", p.gcnArchName);
    const char* a = p.gcnArchName;
    di.state = (std::strncmp(a, "gfx950", 6) == 0 && (a[6] == 0 || a[6] == ':')) ? 1 : -1;
    di.n_cu = p.multiProcessorCount;
  }
  if (di.state < 0) {
    set_err("device %d is %s; libmmsa runs on gfx950 only", dev, di.arch);
    return MMSA_UNSUPPORTED;
  }
  if (scratch_out) {
    // The array's name is only a host-side handle: its address on this
    // device (the current one) comes from the runtime, once per device.
    if (!di.scratch) {
      void* p = nullptr;
      const hipError_t e3 = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e3 != hipSuccess || !p) {
        set_err("device %d: address of the static scratch: %s", dev, hipGetErrorString(e3));
        return MMSA_HIP_ERROR;
      }
      di.scratch = p;
    }
    *scratch_out = di.scratch;
  }
  if (n_cu_out) *n_cu_out = di.n_cu;
  return MMSA_OK;
}

// The descriptor tables go up with every call.  A copy enqueued while the
// stream is being captured into a graph reads its host source again at each
// replay, and the layout cache may by then have evicted and freed the
// layout's own tables: under capture the copy reads from a private copy of
// them that is kept until the process ends (a few KB per captured call).
mmsa_status upload(const Layout& Lo, void* ws, hipStream_t s) {
  const void* src = Lo.blob.data();
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const mmsa_status st = hip_status(hipStreamIsCapturing(s, &cs), "capture status");
  if (st != MMSA_OK) return st;
  if (cs == hipStreamCaptureStatusActive) {
    static std::mutex mu;
    static std::vector<std::unique_ptr<const std::vector<char>>> kept;
    std::lock_guard<std::mutex> lock(mu);
    kept.push_back(std::make_unique<const std::vector<char>>(Lo.blob));
    src = kept.back()->data();
  }
  return hip_status(hipMemcpyAsync(ws, src, Lo.blob.size(), hipMemcpyHostToDevice, s), "table upload");
}

#define MMSA_TRY(expr)                       \
  do {                                       \
    mmsa_status _st = (expr);                \
    if (_st != MMSA_OK) return _st;          \
  } while (0)
#define MMSA_HIP(expr, where) MMSA_TRY(hip_status((expr), where))

// The five steps on a validated layout, a workspace `w` and a stream: shared
// by the entry points (caller workspace) and mmsa_prefill_noalloc (static
// scratch).  Each uploads the tables it reads first.
mmsa_status run_estimate_vs(const Layout& Lo, const void* q, const void* k, char* w, hipStream_t s) {
  MMSA_TRY(upload(Lo, w, s));
  if (Lo.need_seg) MMSA_HIP(launch_seg_tables(Lo.dm, Lo.tb, w, s), "segment tables");
  MMSA_HIP(launch_est_pass1(Lo.dm, Lo.tb, w, q, k, Lo.n_wg1, s), "estimation pass 1");
  MMSA_HIP(launch_fill_u32(w + Lo.zero_off, 0u, Lo.zero_bytes / 4, s), "score clear");
  MMSA_HIP(launch_est_pass2(Lo.dm, Lo.tb, w, q, k, Lo.n_wg2, Lo.max_ds, s), "estimation pass 2");
  MMSA_HIP(launch_topk(Lo.tb, w, (int)Lo.max_topk_slices, s), "top-k");
  MMSA_HIP(launch_grid(Lo.dm, Lo.tb, w, Lo.max_strides, s), "grid rule");
  return MMSA_OK;
}

mmsa_status run_estimate_blocks(const Layout& Lo, const void* q, const void* k, char* w, hipStream_t s) {
  MMSA_TRY(upload(Lo, w, s));
  MMSA_HIP(launch_block_estimate(Lo.dm, Lo.tb, w, q, k, Lo.nB, s), "block estimation");
  return MMSA_OK;
}

mmsa_status run_permute(const Layout& Lo, const void* q, const void* k, const void* v, char* w, hipStream_t s) {
  MMSA_TRY(upload(Lo, w, s));
  if (Lo.dm.debug) {
    MMSA_HIP(launch_fill_u32(w + Lo.dm.ws_flag, 0u, 1, s), "debug word clear");
    MMSA_HIP(launch_nonfinite_scan(Lo.dm, w, q, k, v, s), "non-finite scan");
  }
  if (Lo.need_seg) MMSA_HIP(launch_seg_tables(Lo.dm, Lo.tb, w, s), "segment tables");
  if (Lo.gridrow_bytes > 0) {
    MMSA_HIP(launch_fill_u32(w + Lo.gridrow_off, 0xffffffffu, Lo.gridrow_bytes / 4, s), "row order clear");
    MMSA_HIP(launch_grid_rows(Lo.dm, Lo.tb, w, s), "grid row order");
  }
  MMSA_HIP(launch_gather(Lo.dm, Lo.tb, w, q, k, v, Lo.max_gather_slots, s), "gather");
  MMSA_HIP(launch_plan(Lo.dm, Lo.tb, w, Lo.max_tiles, Lo.max_bm_words, Lo.max_shift_words, s), "plan");
  return MMSA_OK;
}

mmsa_status run_sparse_prefill(const Layout& Lo, const void* q, const void* k, const void* v, void* o, float* lse,
                               int n_cu, char* w, hipStream_t s) {
  MMSA_TRY(upload(Lo, w, s));
  // the pop counters start at zero on every call, so the call can be repeated
  MMSA_HIP(launch_queue_reset(Lo.dm, w, s), "queue reset");
  // two resident workgroups per CU (the kernel's LDS and register budget)
  MMSA_HIP(launch_attention(Lo.dm, Lo.tb, w, q, k, v, o, lse, 2 * std::max(n_cu, 1), s), "attention");
  return MMSA_OK;
}

mmsa_status run_unpermute(const Layout& Lo, void* o, char* w, hipStream_t s) {
  MMSA_TRY(upload(Lo, w, s));
  MMSA_HIP(launch_unpermute(Lo.dm, Lo.tb, w, o, Lo.max_unperm_slots, s), "unpermute");
  return MMSA_OK;
}

}  // namespace

extern "C" {

int32_t mmsa_abi_version(void) { return MMSA_ABI_VERSION; }

const char* mmsa_status_string(mmsa_status s) {
  switch (s) {
    case MMSA_OK: return "ok";
    case MMSA_INVALID_ARGUMENT: return "invalid argument";
    case MMSA_UNSUPPORTED: return "unsupported";
    case MMSA_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MMSA_HIP_ERROR: return "HIP error";
    default: return "unknown status";
  }
}

const char* mmsa_last_error(void) { return g_err.c_str(); }

size_t mmsa_workspace_bytes(const mmsa_layer_desc* desc) {
  std::shared_ptr<const Layout> lo;
  if (get_layout(desc, lo) != MMSA_OK) return 0;
  return (size_t)lo->ws_total;
}

mmsa_status mmsa_workspace_view(const mmsa_layer_desc* desc, int32_t buf, int32_t bh, int32_t part,
                                int64_t* offset_bytes, int64_t* count) {
  if (!offset_bytes || !count) {
    set_err("offset_bytes/count is NULL");
    return MMSA_INVALID_ARGUMENT;
  }
  std::shared_ptr<const Layout> lo;
  MMSA_TRY(get_layout(desc, lo));
  const Layout& Lo = *lo;
  *offset_bytes = 0;
  *count = 0;
  if (Lo.empty) return MMSA_OK;
  if (bh < 0 || bh >= Lo.BH || part < 0 || part >= (int)Lo.set_of[bh].size()) {
    set_err("bh=%d / part=%d out of range", bh, part);
    return MMSA_INVALID_ARGUMENT;
  }
  const HeadDev& H = Lo.heads[bh];
  const std::pair<int, int> sp = Lo.set_of[bh][part];
  const PairDev* P = sp.first >= 0 ? &Lo.jobs[sp.first].pair[sp.second] : nullptr;
  const EstJob* J = sp.first >= 0 ? &Lo.jobs[sp.first] : nullptr;
  switch (buf) {
    case MMSA_BUF_V_SCORES:
      if (P) *offset_bytes = P->ws_v, *count = P->Dv;
      break;
    case MMSA_BUF_S_SCORES:
      if (P && P->ws_s >= 0) *offset_bytes = P->ws_s, *count = P->Ds;
      break;
    case MMSA_BUF_V_INDEX:
      if (P && P->ws_vidx >= 0) *offset_bytes = P->ws_vidx, *count = P->kv;
      break;
    case MMSA_BUF_S_INDEX:
      if (P && P->ws_sidx >= 0) *offset_bytes = P->ws_sidx, *count = P->ks;
      break;
    case MMSA_BUF_NSEL:
      if (P && P->ws_nsel >= 0) *offset_bytes = P->ws_nsel, *count = 2;
      break;
    case MMSA_BUF_GRID:
      if (H.grid_task >= 0) {
        const GridTask& T = Lo.grids[H.grid_task];
        *offset_bytes = T.ws_out;
        *count = 3 + std::min(T.w, MAX_PHASES);
      }
      break;
    case MMSA_BUF_BLOCK_INDEX:
      if (H.pattern == MMSA_BLOCK) *offset_bytes = H.ws_blk_idx, *count = (int64_t)Lo.nB * H.k_blocks;
      break;
    case MMSA_BUF_BLOCK_SCORES:
      if (H.pattern == MMSA_BLOCK) *offset_bytes = H.ws_z, *count = (int64_t)Lo.nB * Lo.nB;
      break;
    case MMSA_BUF_ROW_ORDER:
      if (H.row_kind != ROW_IDENTITY) *offset_bytes = H.ws_row_order, *count = H.n_row_slots;
      break;
    case MMSA_BUF_TILE_PAIRS: *offset_bytes = H.ws_pairs, *count = H.nT_rows; break;
    case MMSA_BUF_TILE_INFO: *offset_bytes = H.ws_info, *count = 4ll * H.nT_rows; break;
    case MMSA_BUF_EST_STATS:
      if (J) *offset_bytes = J->ws_stats, *count = 2 * EST_ROWS;
      break;
    case MMSA_BUF_TILE_BITMAP: *offset_bytes = H.ws_bm, *count = (int64_t)H.nT_rows * H.bm_words; break;
    case MMSA_BUF_DEBUG_FLAGS: *offset_bytes = Lo.dm.ws_flag, *count = 1; break;
    default: set_err("unknown buffer %d", buf); return MMSA_INVALID_ARGUMENT;
  }
  return MMSA_OK;
}

mmsa_status mmsa_index_meta(const mmsa_layer_desc* desc, int32_t bh, int32_t part, int32_t out[8]) {
  if (!out) {
    set_err("out is NULL");
    return MMSA_INVALID_ARGUMENT;
  }
  std::shared_ptr<const Layout> lo;
  MMSA_TRY(get_layout(desc, lo));
  const Layout& Lo = *lo;
  for (int i = 0; i < 8; ++i) out[i] = 0;
  if (Lo.empty) return MMSA_OK;
  if (bh < 0 || bh >= Lo.BH || part < 0 || part >= (int)Lo.set_of[bh].size()) {
    set_err("bh=%d / part=%d out of range", bh, part);
    return MMSA_INVALID_ARGUMENT;
  }
  const std::pair<int, int> sp = Lo.set_of[bh][part];
  if (sp.first < 0) return MMSA_OK;
  const EstJob& J = Lo.jobs[sp.first];
  const PairDev& P = J.pair[sp.second];
  const HeadDev& H = Lo.heads[bh];
  if (H.grid_task >= 0) {
    out[0] = 0;
    out[1] = Lo.grids[H.grid_task].D;
  } else {
    out[0] = P.v_lo;
    out[1] = P.v_hi;
    out[2] = P.s_lo;
    out[3] = P.s_hi;
    out[4] = P.kv;
    out[5] = P.ks;
    out[6] = J.kind == JOB_VS_2D ? P.n_k - 1 : 0;
  }
  out[7] = J.n_rows;
  return MMSA_OK;
}

mmsa_status mmsa_estimate_vs(const mmsa_layer_desc* desc, const void* q, const void* k, void* ws, size_t ws_bytes,
                             void* stream) {
  std::shared_ptr<const Layout> lo;
  MMSA_TRY(prepare(desc, ws, ws_bytes, lo));
  const Layout& Lo = *lo;
  if (Lo.empty || Lo.jobs.empty()) return MMSA_OK;
  MMSA_TRY(check_ptr(q, "q"));
  MMSA_TRY(check_ptr(k, "k"));
  MMSA_TRY(check_device());
  return run_estimate_vs(Lo, q, k, (char*)ws, (hipStream_t)stream);
}

mmsa_status mmsa_estimate_blocks(const mmsa_layer_desc* desc, const void* q, const void* k, void* ws,
                                 size_t ws_bytes, void* stream) {
  std::shared_ptr<const Layout> lo;
  MMSA_TRY(prepare(desc, ws, ws_bytes, lo));
  const Layout& Lo = *lo;
  if (Lo.empty || !Lo.any_block) return MMSA_OK;
  MMSA_TRY(check_ptr(q, "q"));
  MMSA_TRY(check_ptr(k, "k"));
  MMSA_TRY(check_device());
  return run_estimate_blocks(Lo, q, k, (char*)ws, (hipStream_t)stream);
}

mmsa_status mmsa_permute(const mmsa_layer_desc* desc, const void* q, const void* k, const void* v, void* ws,
                         size_t ws_bytes, void* stream) {
  std::shared_ptr<const Layout> lo;
  MMSA_TRY(prepare(desc, ws, ws_bytes, lo));
  const Layout& Lo = *lo;
  if (Lo.empty) return MMSA_OK;
  MMSA_TRY(check_ptr(q, "q"));
  MMSA_TRY(check_ptr(k, "k"));
  MMSA_TRY(check_ptr(v, "v"));
  MMSA_TRY(check_device());
  return run_permute(Lo, q, k, v, (char*)ws, (hipStream_t)stream);
}

mmsa_status mmsa_sparse_prefill(const mmsa_layer_desc* desc, const void* q, const void* k, const void* v, void* ws,
                                size_t ws_bytes, void* o, float* lse, void* stream) {
  std::shared_ptr<const Layout> lo;
  MMSA_TRY(prepare(desc, ws, ws_bytes, lo));
  const Layout& Lo = *lo;
  if (Lo.empty) return MMSA_OK;
  MMSA_TRY(check_ptr(q, "q"));
  MMSA_TRY(check_ptr(k, "k"));
  MMSA_TRY(check_ptr(v, "v"));
  MMSA_TRY(check_ptr(o, "o"));
  int n_cu = 0;
  MMSA_TRY(check_device(&n_cu));
  return run_sparse_prefill(Lo, q, k, v, o, lse, n_cu, (char*)ws, (hipStream_t)stream);
}

mmsa_status mmsa_unpermute(const mmsa_layer_desc* desc, void* ws, size_t ws_bytes, void* o, void* stream) {
  std::shared_ptr<const Layout> lo;
  MMSA_TRY(prepare(desc, ws, ws_bytes, lo));
  const Layout& Lo = *lo;
  if (Lo.empty) return MMSA_OK;
  MMSA_TRY(check_ptr(o, "o"));
  MMSA_TRY(check_device());
  return run_unpermute(Lo, o, (char*)ws, (hipStream_t)stream);
}

mmsa_status mmsa_prefill_noalloc(const mmsa_layer_desc* desc, const void* q, const void* k, const void* v, void* o,
                                 float* lse, void* stream) {
  std::shared_ptr<const Layout> lo;
  MMSA_TRY(get_layout(desc, lo));
  const Layout& Lo = *lo;
  if (Lo.empty) return MMSA_OK;
  if (Lo.ws_total > (int64_t)MMSA_NOALLOC_SCRATCH_BYTES) {
    set_err("this layer needs %lld bytes of workspace; the static scratch of mmsa_prefill_noalloc holds %lld "
            "(use the five calls with a caller workspace)",
            (long long)Lo.ws_total, (long long)MMSA_NOALLOC_SCRATCH_BYTES);
    return MMSA_WORKSPACE_TOO_SMALL;
  }
  MMSA_TRY(check_ptr(q, "q"));
  MMSA_TRY(check_ptr(k, "k"));
  MMSA_TRY(check_ptr(v, "v"));
  MMSA_TRY(check_ptr(o, "o"));
  int n_cu = 0;
  void* sp = nullptr;
  MMSA_TRY(check_device(&n_cu, &sp));
  char* w = (char*)sp;
  hipStream_t s = (hipStream_t)stream;
  // the five steps in their order, on the static scratch; each step rebuilds
  // what it reads (tables, cleared scores and counters), so nothing left there
  // by an earlier call is used
  if (!Lo.jobs.empty()) MMSA_TRY(run_estimate_vs(Lo, q, k, w, s));
  if (Lo.any_block) MMSA_TRY(run_estimate_blocks(Lo, q, k, w, s));
  MMSA_TRY(run_permute(Lo, q, k, v, w, s));
  MMSA_TRY(run_sparse_prefill(Lo, q, k, v, o, lse, n_cu, w, s));
  return run_unpermute(Lo, o, w, s);
}

}  // extern "C"
