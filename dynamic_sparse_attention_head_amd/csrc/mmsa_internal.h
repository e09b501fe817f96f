// Internal declarations shared by the host API and the gfx950 kernels of
// libmmsa.  Not part of the public ABI (include/mmsa.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "mmsa.h"

namespace mmsa {

constexpr int TILE = 64;        // query / key tile and pooling block
constexpr int EST_ROWS = 64;    // estimation rows per region
constexpr int EST_CK = 256;     // keys per workgroup chunk in the estimation passes
constexpr int EST1_JB = 4;      // estimation jobs per pass-1 batch (their Q rows stay in LDS)
constexpr int EST1_WG = 512;    // workgroups per estimation pass to aim for (two per compute unit)
constexpr int EST2_JB = 2;      // estimation jobs per pass-2 batch
constexpr int GRP_PAD = 256;    // modality parts of the grouped order are padded to this
constexpr int MAX_PHASES = 16;  // grid phases kept at most
constexpr int MAX_STRIDE = 1024;// largest grid stride searched
constexpr int GRID_OUT = 3 + MAX_PHASES;  // stride, w, n_line, phases
constexpr int N_XCD = 8;          // L2 domains (XCDs); workgroup i runs on XCD i % 8
constexpr int32_t KPOS_NONE = 0x7fffffff;  // key slot without a token (never causal)
constexpr double SFIX = 1099511627776.0;   // 2^40: fixed-point scale of slash sums

enum RowKind : int32_t { ROW_IDENTITY = 0, ROW_GROUPED = 1, ROW_GRID = 2, ROW_SEGMENT = 3 };
enum ViewKind : int32_t { VIEW_IDENTITY = 0, VIEW_GROUPED = 1 };
enum JobKind : int32_t { JOB_VS_ORIG = 0, JOB_VS_2D = 1, JOB_GRID_PLAIN = 2, JOB_GRID_GROUPED = 3 };

// One modality segment, with the count of same-modality tokens before it.
struct SegDev {
  int64_t start, len;
  int32_t modality, rank_start;
  int32_t slot0, _pad;         // first slot in the segment-grouped order (segments padded to 64)
};

// Per (batch, q head): everything a kernel needs to find this head's data.
// Offsets named ws_* are byte offsets into the workspace (-1: absent).
// Parallel-encoding mask (PEVLM verdict page, key_machinery): the first key
// past the sink block that row i sees -- the start of its context block, whose
// blocks of `window` tokens start at `sink`; 0 for sink rows and for question
// rows (from `qstart` on), which see every earlier token.
__host__ __device__ inline int par_floor(int sink, int window, int qstart, int i) {
  if (i < sink || i >= qstart) return 0;
  return sink + ((i - sink) / window) * window;
}

struct HeadDev {
  int32_t b, h, g, pattern, layout;
  int32_t sink, window, k_blocks;
  int32_t qstart;            // PARALLEL: first row of the question block
  int32_t segjob;            // Q_SEGMENT: first entry of its per-segment job list, else -1
  int32_t row_kind, view_kind;
  int32_t n_row_slots;       // slots of the row order (a multiple of 64)
  int32_t nT_rows;           // query tiles = n_row_slots / 64
  int32_t nT_view;           // key tiles of the key view
  int32_t bm_words;          // 64-bit words of the per-tile key-tile bitmap
  int32_t gcap;              // gathered-column capacity per query tile
  int32_t grid_task;         // GRID: index into the grid task table, else -1
  int32_t job[2];            // VS family: estimation job per query modality (or [0] only)
  int32_t n_pairs;           // 2D: key modalities with tokens (index sets per region)
  int32_t qgroup;            // queue group: the q heads sharing this head's (b, KV head)
  int64_t q_off, k_off, v_off, o_off;  // element offsets of (b,h) in Q/O and (b,g) in K/V
  int64_t ws_row_order;      // int32[n_row_slots]
  int64_t ws_qperm, ws_operm;// bf16 [n_row_slots][d]
  int64_t ws_kgrp, ws_vgrp;  // bf16 [L_grp][d] of (b,g) for grouped key views
  int64_t ws_bm;             // uint64 [nT_rows][bm_words]
  int64_t ws_info;           // int4 [nT_rows]: (n_tiles, n_gather, cost, n_rows)
  int64_t ws_pairs;          // int64 [nT_rows]
  int64_t ws_gather;         // int32 [nT_rows][gcap]
  int64_t ws_blk_idx;        // int32 [nB][k_blocks]
  int64_t ws_qp, ws_kp, ws_z;// BLOCK: pooled Q (fp32 [nB][d]), pooled K of (b,g), logits [nB][nB]
};

// One score pair of an estimation job: the vectors a region produces for one
// key coordinate system.
struct PairDev {
  int32_t m_k;               // key modality (2D) or -1 (all keys)
  int32_t Dv, Ds;            // lengths of v and s
  int32_t kv, ks;            // budgets after clamping
  int32_t v_lo, v_hi, s_lo, s_hi;  // candidate ranges
  int32_t n_k;               // keys of m_k (2D), else L
  int32_t shift_words;       // uint64 words of ws_shift
  int32_t _pad_pair;
  int64_t ws_v, ws_s, ws_sacc;     // float[Dv], float[Ds], int64[Ds]
  int64_t ws_vidx, ws_sidx, ws_nsel; // int32[kv], int32[ks], int32[2]
  int64_t ws_shift;          // uint64 [shift_words], bit q = some selected diagonal reaches key tile
                             // t0 - q from a full query tile whose rows (ranks, for 2D pairs, with the
                             // offsets shifted to be non-negative) start at 64 * t0; else -1
};

// One estimation region: up to 64 rows of one head.
struct EstJob {
  int32_t bh, kind, view, m_q;
  int32_t n_rows, rho0, n_runs, n_pairs;
  int32_t imax;
  int32_t n_part1;           // pass-1 partials of this job (workgroups of its batch)
  int64_t q_off, k_off;
  int64_t ws_stats;          // float2 [64] final (max in log2 units, sum)
  int64_t ws_part;           // float2 [n_part1][64] partials of pass 1
  int32_t rows[EST_ROWS];    // ascending original positions
  int32_t run_r0[EST_ROWS];  // runs of consecutive positions: first row index
  int32_t run_len[EST_ROWS];
  PairDev pair[2];
};

// A set of jobs sharing (b, g) [pass 1: at most EST1_JB of them] or (b, g, view)
// [pass 2: at most EST2_JB].
struct EstGroup {
  int32_t b, g, view, job_begin, job_end, n_keys;
  int64_t k_off;             // element offset of K of (b,g)
  int64_t ws_kgrp;           // grouped K (view 1), else -1
  int32_t wg0, nwg;          // its workgroups wg0 .. wg0+nwg-1 of the (1-D) launch
};

struct TopkTask {
  int64_t ws_x, ws_out, ws_cnt;
  int32_t lo, hi, k, _pad;
  int64_t ws_tmp;            // slice histograms, counts, offsets and threshold (topk_tmp_bytes)
};
constexpr int TK_SL = 16384;   // elements per top-k slice (one workgroup)
__host__ __device__ inline int64_t topk_slices(int n) { return n > 0 ? (n + TK_SL - 1) / TK_SL : 0; }
// 4 rounds of 256-bin histograms per slice, (greater, equal) counts and
// (output offset, equal keys before) per slice, then the threshold state after
// rounds 1-4 and the final threshold (16 bytes each)
__host__ __device__ inline int64_t topk_tmp_bytes(int n) { return 16ll * 256 * topk_slices(n) + 16ll * topk_slices(n) + 80; }

struct GridTask {
  int32_t job, bh, D, n_rows;
  int32_t s_lo, s_hi, w, grouped;
  int64_t cap;               // clip level of the fixed-point scores
  int64_t ws_v;              // float [L] vertical scores in grid coordinates
  int64_t ws_U;              // int64 sum of clipped scores
  int64_t ws_u;              // int32 [D] clipped fixed-point scores
  int64_t ws_cand;           // per stride: MAX_PHASES x (X, cnt, phase)
  int64_t ws_out;            // int32 [GRID_OUT]: stride, w, n_line, phases
};

// Mean pooling of one 64-row-blocked (b, head) slice of Q or K.
struct PoolTask {
  int64_t src_off, row_stride, ws_dst;
  int32_t is_k, _pad;
};

// Pooled logits and top-k of one BLOCK head.
struct BlockTask {
  int32_t bh, kb;
  int64_t ws_qp, ws_kp, ws_z, ws_idx;
};

// Row gather: dst[slot] = src[rows[slot]] (zero row where rows[slot] < 0).
struct GatherTask {
  int64_t src_off, row_stride, ws_rows, ws_dst;
  int32_t n_slots, which;     // which: 0 q, 1 k, 2 v
};

// Row scatter of one permuted head: O[rows[slot]] = src[slot].
struct UnpermTask {
  int64_t ws_src, ws_rows, o_off;
  int32_t n_slots, _pad;
};

// Q heads sharing one (b, KV head): their query tiles are queued together,
// tile-descending, so concurrent workgroups stream the same K/V through L2.
struct QGroup {
  int32_t head_begin, head_end;   // range in the flat head list
  int64_t item_base;              // first queue position of the group
};

// Everything the kernels read, placed at the start of the workspace.
struct Tables {
  int64_t n_heads, n_jobs, n_groups1, n_groups2, n_topk, n_grid, n_segs;
  int64_t n_pool, n_block, n_gather, n_unperm, n_qgroups, n_segjob;
  int64_t off_heads, off_jobs, off_groups1, off_groups2, off_topk, off_grid, off_segs;
  int64_t off_pool, off_block, off_gather, off_unperm, off_qgroups, off_qgroup_heads;
  int64_t off_segjob;        // int32: estimation job of each segment, per Q_SEGMENT head
};

// Shapes shared by every kernel of one call.
struct Dims {
  int32_t B, Hq, Hkv, L, d, nT;
  int32_t n_text, n_video, text_base, video_base, L_grp, L_seg;
  float scale, scale_log2;
  int64_t q_sb, q_sh, q_sl, k_sb, k_sh, k_sl, v_sb, v_sh, v_sl, o_sb, o_sh, o_sl;
  int64_t ws_pgrp;           // int32[L_grp]: original position at each grouped slot (-1 pad)
  int64_t ws_gslot;          // int32[L]: grouped slot of each position
  int64_t ws_pseg;           // int32[L_seg]: original position at each segment-grouped slot (-1 pad), or -1
  int64_t n_items;           // queue length: every (head, pair of adjacent query tiles)
  int64_t ws_enum_item;      // int32 [n_items]: (bh << 16) | pair in queue order
  int64_t ws_enum_cost;      // int32 [n_items]: cost of each queued item
  int64_t ws_ctr;            // int32 [N_XCD] pop counters of the attention queue
  int64_t ws_flag;           // uint32 debug word (MMSA_FLAG_DEBUG)
  int32_t chunk_asc;         // attention walks key tiles lowest first (else highest first)
  int32_t debug;             // MMSA_FLAG_DEBUG: record non-finite inputs / outputs in the word at ws_flag
};

// ---------------------------------------------------------------------------
// Kernel launchers (each returns hipGetLastError() after its launches)
// ---------------------------------------------------------------------------
hipError_t launch_fill_u32(void* p, uint32_t value, int64_t n_words, hipStream_t s);
hipError_t launch_seg_tables(const Dims& dm, const Tables& tb, char* ws, hipStream_t s);

hipError_t launch_est_pass1(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k,
                            int n_wg1, hipStream_t s);   // n_wg1: workgroups of all pass-1 batches
hipError_t launch_est_pass2(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k,
                            int n_wg2, int max_ds, hipStream_t s);
hipError_t launch_topk(const Tables& tb, char* ws, int max_slices, hipStream_t s);
hipError_t launch_grid(const Dims& dm, const Tables& tb, char* ws, int max_strides, hipStream_t s);

hipError_t launch_block_estimate(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k,
                                 int nB, hipStream_t s);

hipError_t launch_grid_rows(const Dims& dm, const Tables& tb, char* ws, hipStream_t s);
hipError_t launch_gather(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k,
                         const void* v, int max_slots, hipStream_t s);
hipError_t launch_plan(const Dims& dm, const Tables& tb, char* ws, int max_tiles, int max_bm_words,
                       int max_shift_words, hipStream_t s);

hipError_t launch_queue_reset(const Dims& dm, char* ws, hipStream_t s);
hipError_t launch_attention(const Dims& dm, const Tables& tb, char* ws, const void* q, const void* k,
                            const void* v, void* o, float* lse, int n_workgroups, hipStream_t s);
hipError_t launch_unpermute(const Dims& dm, const Tables& tb, char* ws, void* o, int max_slots, hipStream_t s);

// MMSA_FLAG_DEBUG: OR into the word at ws_flag bit 0 / 1 / 2 when Q / K / V
// holds a NaN or an infinity
hipError_t launch_nonfinite_scan(const Dims& dm, char* ws, const void* q, const void* k, const void* v,
                                 hipStream_t s);

}  // namespace mmsa
