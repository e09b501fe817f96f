/*
 * mmsa.h — C ABI of libmmsa: modality-aware dynamic sparse-attention prefill
 * for one causal attention layer on an AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources: the MInference 1.0 summary page, "Approach";
 * the MMInference summary page, "Approach"; the MMInference verdict page,
 * fields key_machinery and core_discovery):
 *   per attention head, online index estimation from the last 64 queries
 *   (vertical / slash lines), from 64-token mean-pooled blocks (block-sparse),
 *   or from a stride/phase scan (grid); a modality-aware permutation of rows
 *   and key columns; a FlashAttention-style causal prefill over only the
 *   selected 64x64 tiles; and the inverse permutation of the output.
 *
 * Call order, all on one HIP stream, with one descriptor and one workspace:
 *   mmsa_estimate_vs     (vertical-slash, boundary and grid heads)
 *   mmsa_estimate_blocks (block-sparse heads)          -- 1 and 2 in any order
 *   mmsa_permute         (row orders, gathers, per-tile sparse plan)
 *   mmsa_sparse_prefill  (the attention itself)
 *   mmsa_unpermute       (inverse permutation into O)
 *
 * Conventions shared by every entry point:
 *  - Ownership: the caller owns all device memory (Q, K, V, O, LSE and the
 *    workspace).  The library never allocates or frees device memory and keeps
 *    no pointer after a call returns.  Host arrays named in the descriptor are
 *    read only during the call.  The tables derived from a descriptor are kept
 *    in a small host-side cache (16 layouts, least recently used out), keyed by
 *    the values of the descriptor and of its host arrays, so the five calls of
 *    one layer build them once; a changed descriptor or array is a new key.
 *  - Asynchrony: every call enqueues work on `stream` (a hipStream_t; NULL is
 *    the null stream) and returns without waiting for the device.
 *  - Graph capture: the calls, and mmsa_prefill_noalloc, may be captured into
 *    a HIP graph.  Each call uploads its tables (a few KB) from host memory;
 *    under capture it uploads them from a private copy kept until the process
 *    ends, so replays stay valid after the cache above has dropped the layout.
 *    No call records a memset.
 *  - Tensors: bf16, element strides (batch, head, row) with the last (head
 *    dimension) contiguous; base pointers 16-byte aligned; row strides a
 *    multiple of 8 elements.  d is 64 or 128.
 *  - Errors: arguments are validated on the host before anything is enqueued;
 *    on any error nothing is launched or written, and mmsa_last_error() gives
 *    a thread-local message.  No C++ exception crosses this interface.
 *  - Budgets above the number of candidates are clamped, not errors.
 *  - NaN or Inf in Q/K/V give undefined (but memory-safe) results; with
 *    MMSA_FLAG_DEBUG the calls record that they met one (see below).
 *  - Device: gfx950 only.  Every call that enqueues work first checks the
 *    architecture of the current HIP device and returns MMSA_UNSUPPORTED, with
 *    nothing enqueued, on any other device or when there is none.
 *  - Limits: L < 2^22 tokens (tile indices are packed in 16 bits), B*Hq <= 4096;
 *    BLOCK heads need L <= 2^20 (one pooled-logit row per query block in LDS);
 *    a Q_SEGMENT head needs its segments, each padded to a multiple of 64
 *    rows, to fit in 131070 query tiles (else MMSA_UNSUPPORTED).
 */
#ifndef MMSA_H
#define MMSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MMSA_ABI_VERSION 4
#define MMSA_TILE 64       /* query and key tile (the 64-token blocks)      */
#define MMSA_EST_ROWS 64   /* estimation rows: the last 64 queries          */

typedef int32_t mmsa_status;
enum {
  MMSA_OK = 0,
  MMSA_INVALID_ARGUMENT = 1,  /* null pointer, shape, stride, budget, segments, combination */
  MMSA_UNSUPPORTED = 2,       /* d, alignment, size limits, device architecture             */
  MMSA_WORKSPACE_TOO_SMALL = 3,
  MMSA_HIP_ERROR = 4          /* a launch failed; detail in mmsa_last_error()               */
};

/* Per-head sparse pattern (the offline per-head assignment; MInference summary
 * page, "Approach": A-shape, vertical-slash, block-sparse; MMInference
 * verdict page, core_discovery: grid, Q-boundary, 2D-boundary).
 * MMSA_PARALLEL is the static parallel-encoding mask of the PEVLM verdict page
 * (key_machinery): tokens [0, sink) form the sink block, the last `question`
 * tokens the question block, and the tokens between are cut into context
 * blocks of `window` tokens from `sink` on (the last may be shorter).  A
 * context row sees the sink block and its own block; sink and question rows
 * see every earlier token; j <= i throughout.  It needs no estimation. */
enum { MMSA_ASHAPE = 0, MMSA_VS = 1, MMSA_BLOCK = 2, MMSA_GRID = 3, MMSA_PARALLEL = 4 };
/* Layout (how modality boundaries are handled; MMInference verdict page,
 * core_discovery: row-wise permutation grouping same-modality queries, 2D
 * permutation isolating each modality pair). */
enum {
  MMSA_PLAIN = 0,             /* no modality handling                              */
  MMSA_Q_BOUNDARY = 1,        /* VS only: rows grouped by modality, one index set per query modality */
  MMSA_BOUNDARY_2D = 2,       /* VS only: rows and keys grouped, one index set per (query, key) modality pair */
  MMSA_MODALITY_GROUPED = 3,  /* GRID only: stride/phase measured on the modality-grouped order */
  MMSA_Q_SEGMENT = 4          /* VS only: rows grouped by segment (each padded to 64), one index set
                                 per segment from its own last 64 queries (original coordinates) */
};
enum { MMSA_TEXT = 0, MMSA_VIDEO = 1 };

/* mmsa_layer_desc.flags (MMInference verdict page, key_machinery: the
 * permutation is realised as index-based loading inside the attention kernel).
 *  0 (default): index-based.  mmsa_sparse_prefill reads the Q rows of permuted
 *    heads at their original positions through the row order and the keys of
 *    the modality-grouped view through the grouped-slot map, and writes every
 *    output row at its original position; mmsa_permute copies no tensor and
 *    mmsa_unpermute has nothing left to move.
 *  MMSA_FLAG_MATERIALIZE: mmsa_permute also copies the permuted Q rows and the
 *    grouped K/V into the workspace, mmsa_sparse_prefill reads those copies and
 *    writes the rows of permuted heads to the workspace, and mmsa_unpermute
 *    scatters them into o.  The results are bit-identical; the workspace is
 *    larger (2*d bytes per row slot of each permuted head, twice, and 4*d
 *    bytes per grouped slot of each KV head a 2D-boundary head uses).
 *  MMSA_FLAG_DEBUG: mmsa_permute clears the debug word (MMSA_BUF_DEBUG_FLAGS)
 *    and scans every element of Q, K and V, setting bit 0 when Q holds a NaN
 *    or an infinity, bit 1 for K and bit 2 for V; mmsa_sparse_prefill sets
 *    bit 3 when it writes a non-finite output element or LSE value (an LSE
 *    of -inf, for a row with no selected key, does not count).  The word can
 *    be read once the stream has drained.  Without the flag the word is not
 *    touched.
 *  MMSA_FLAG_KEYS_ASCENDING / MMSA_FLAG_KEYS_DESCENDING: the order in which
 *    the attention call walks the key tiles of a query tile, lowest first or
 *    highest (diagonal) first.  Without either, the library picks by size:
 *    lowest first once one KV head's K and V exceed 256 MB.  Outputs agree to
 *    fp32 rounding (the online softmax sums in another order); index sets,
 *    plans and pair counts are identical.  Setting both is an error.
 * Any other bit is an error. */
#define MMSA_FLAG_MATERIALIZE 1u
#define MMSA_FLAG_DEBUG 2u
#define MMSA_FLAG_KEYS_ASCENDING 4u
#define MMSA_FLAG_KEYS_DESCENDING 8u

typedef struct {
  int32_t pattern;      /* MMSA_ASHAPE / VS / BLOCK / GRID / PARALLEL               */
  int32_t layout;       /* MMSA_PLAIN / Q_BOUNDARY / BOUNDARY_2D / MODALITY_GROUPED  */
  int32_t sink;         /* A-shape: keys j < sink are kept; PARALLEL: sink block length;
                           GRID: rows off the lines also keep keys j < sink (0: none) */
  int32_t window;       /* A-shape: keys with i - j < window are kept (>= 1);
                           PARALLEL: context block length (>= 1);
                           GRID: rows off the lines also keep keys with i - j < window
                           (0: none)                                                  */
  int32_t k_vertical;   /* VS: vertical columns kept (per index set)                 */
  int32_t k_slash;      /* VS: slash diagonals kept (per index set)                  */
  int32_t k_blocks;     /* BLOCK: key blocks kept per query block                    */
  int32_t grid_phases;  /* GRID: number of phases w kept at the winning stride (>=1) */
  int32_t stride_lo;    /* GRID: smallest stride searched (>= 16)                    */
  int32_t stride_hi;    /* GRID: largest stride searched (>= stride_lo, <= 1024)     */
  int32_t grid_clip;    /* GRID: clip constant C of the line score (1..64; 0 -> 8)   */
  int32_t question;     /* PARALLEL: question block length (>= 0; clamped to L)     */
} mmsa_head_cfg;

/* A run of tokens of one modality.  Segments must tile [0, L) in order. */
typedef struct {
  int64_t start, len;
  int32_t modality;     /* MMSA_TEXT or MMSA_VIDEO */
  int32_t _pad;
} mmsa_segment;

typedef struct {
  int32_t B, Hq, Hkv, L, d;
  int32_t _pad0;
  int64_t q_strides[3], k_strides[3], v_strides[3], o_strides[3]; /* elements: batch, head, row;
                                       (L-1) * k/v row stride * 2 + 2d must stay below 2 GiB
                                       (MMSA_UNSUPPORTED otherwise)                     */
  float scale;                      /* softmax scale; 0 -> 1/sqrt(d)                 */
  uint32_t flags;                   /* MMSA_FLAG_* bits                              */
  const int32_t* kv_head_of;        /* host [Hq] or NULL -> h / (Hq / Hkv)           */
  const mmsa_head_cfg* heads;       /* host [Hq]                                     */
  const mmsa_segment* segs;         /* host [n_segs]; NULL / 0 -> one text segment   */
  int32_t n_segs;
  int32_t _pad1;
} mmsa_layer_desc;

/* Bytes of device workspace the five calls need for this descriptor; 0 on an
 * invalid descriptor (then mmsa_last_error() says why).  The workspace must be
 * 256-byte aligned and is used by all five calls in sequence. */
size_t mmsa_workspace_bytes(const mmsa_layer_desc* desc);

/* Where a named intermediate of one (batch*Hq + head) `bh` lives in the
 * workspace, so a caller can read it after the stream has drained.
 * `part` selects the index set: 0 for plain heads; the query modality for
 * Q-boundary heads; 2*query_modality + key_modality for 2D-boundary heads;
 * the segment index for Q-segment heads.
 * On success *offset_bytes and *count (elements) are set; a buffer that does
 * not exist for that head gives count 0.  Buffers: */
enum {
  MMSA_BUF_V_SCORES = 0,    /* float[count]  vertical (column) scores; grid heads: line scores
                               per grid coordinate                                          */
  MMSA_BUF_S_SCORES = 1,    /* float[count]  slash (diagonal) scores                         */
  MMSA_BUF_V_INDEX = 2,     /* int32[count]  selected vertical indices, ascending            */
  MMSA_BUF_S_INDEX = 3,     /* int32[count]  selected slash indices, ascending               */
  MMSA_BUF_NSEL = 4,        /* int32[2]      number selected (vertical, slash)               */
  MMSA_BUF_GRID = 5,        /* int32[3+w]    stride, w, number of line positions, w phases   */
  MMSA_BUF_BLOCK_INDEX = 6, /* int32[nB*kb]  per query block, kb key blocks ascending, -1 pad */
  MMSA_BUF_BLOCK_SCORES = 7,/* float[nB*nB]  pooled logits, row b valid for columns 0..b     */
  MMSA_BUF_ROW_ORDER = 8,   /* int32[count]  original position of each permuted row, -1 pad  */
  MMSA_BUF_TILE_PAIRS = 9,  /* int64[count]  selected (query, key) pairs per query tile       */
  MMSA_BUF_TILE_INFO = 10,  /* int32[4*count] per query tile: key tiles, gathered columns,
                               cost, rows                                                    */
  MMSA_BUF_EST_STATS = 11,  /* float[2*64]   per estimation row: max of scale*log2(e)*q.k and
                               the sum of 2^(x - max) over its causal keys                   */
  MMSA_BUF_TILE_BITMAP = 12,/* uint64[count] per query tile, words of a bitmap over the key
                               tiles of the head's key view (bit c of word w: key tile 64w+c);
                               count = tiles * words per tile                                */
  MMSA_BUF_DEBUG_FLAGS = 13 /* uint32[1]     the debug word of MMSA_FLAG_DEBUG (any bh, part) */
};
mmsa_status mmsa_workspace_view(const mmsa_layer_desc* desc, int32_t buf, int32_t bh, int32_t part,
                                int64_t* offset_bytes, int64_t* count);

/* Host-side facts of one index set (same `bh` / `part` as above), all int32:
 * out[0..1] vertical candidates [lo, hi); out[2..3] slash candidates [lo, hi);
 * out[4] vertical budget after clamping; out[5] slash budget after clamping;
 * out[6] slash index shift (2D: keys of the key modality - 1; else 0);
 * out[7] number of estimation rows.  For grid heads out[0..1] is the grid
 * coordinate range [0, D) the stride rule reads. */
mmsa_status mmsa_index_meta(const mmsa_layer_desc* desc, int32_t bh, int32_t part, int32_t out[8]);

/* 1. Vertical-slash, boundary and grid estimation (MInference summary page,
 *    "Approach": last-64-query attention for vertical/slash lines; MMInference
 *    verdict page, key_machinery: grid stride and phase searched on the
 *    approximate attention of the last 64 queries; pith_summary: index from the
 *    last 64 queries of each modality segment).
 *    q, k: device bf16 with the descriptor's strides.  No-op when no head needs it. */
mmsa_status mmsa_estimate_vs(const mmsa_layer_desc* desc, const void* q, const void* k,
                             void* ws, size_t ws_bytes, void* stream);

/* 2. Block-sparse estimation: 64-row mean pooling of Q and K, pooled logits,
 *    top-k key blocks per query block (MInference summary page, "Approach":
 *    mean-pooled 64-block attention).  No-op when there is no BLOCK head. */
mmsa_status mmsa_estimate_blocks(const mmsa_layer_desc* desc, const void* q, const void* k,
                                 void* ws, size_t ws_bytes, void* stream);

/* 3. Permutation and plan: row orders (grid: line rows first; boundary:
 *    modality-grouped), with MMSA_FLAG_MATERIALIZE gathered copies of permuted Q
 *    rows and grouped K/V, and the per-query-tile list of key tiles and
 *    gathered key columns
 *    (MMInference verdict page, core_discovery: row-wise, column-wise and 2D
 *    permutations; key_machinery: kernels load only the permuted blocks). */
mmsa_status mmsa_permute(const mmsa_layer_desc* desc, const void* q, const void* k, const void* v,
                         void* ws, size_t ws_bytes, void* stream);

/* 4. Block-sparse causal prefill over the planned tiles (MMInference verdict
 *    page, key_machinery: block-sparse FlashAttention-style kernels that keep
 *    matrix-core compute dense).  q, k, v as above; o: device bf16 [B,Hq,L,d]
 *    with o_strides — every row is written here at its original position
 *    (with MMSA_FLAG_MATERIALIZE only the rows of heads whose row order is the
 *    identity; the others go to the workspace until mmsa_unpermute).  lse: device
 *    float [B,Hq,L] (contiguous) or NULL; natural-log sum of exp of the scaled
 *    logits over the selected keys, -inf for a row with none.  The call resets
 *    its own work queue, so it may be repeated on the plan the last
 *    mmsa_permute built (for example to time it, or into another o). */
mmsa_status mmsa_sparse_prefill(const mmsa_layer_desc* desc, const void* q, const void* k,
                                const void* v, void* ws, size_t ws_bytes, void* o, float* lse,
                                void* stream);

/* 5. Inverse permutation (MMInference verdict page, core_discovery: the
 *    permutation leaves the model unchanged): with MMSA_FLAG_MATERIALIZE the
 *    rows of permuted heads are scattered from the workspace back to their
 *    original positions in o; by default mmsa_sparse_prefill already wrote
 *    them there and this call only validates its arguments.  After this call
 *    every row of o holds the attention output (0 for a row with no selected
 *    key). */
mmsa_status mmsa_unpermute(const mmsa_layer_desc* desc, void* ws, size_t ws_bytes, void* o,
                           void* stream);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc): the five calls above
 * in order, on a workspace the library holds itself, a static device array of
 * MMSA_NOALLOC_SCRATCH_BYTES per GPU that stays allocated until the process
 * ends.  q, k, v, o, lse and the descriptor as for the five calls; nothing
 * else is needed and nothing is allocated.  A layer whose
 * mmsa_workspace_bytes() exceeds MMSA_NOALLOC_SCRATCH_BYTES is refused with
 * MMSA_WORKSPACE_TOO_SMALL before anything is enqueued (64 MiB holds, for
 * example, a 32K-token layer of 32 q / 8 KV heads with d = 128 and
 * vertical-slash, block and A-shape heads).  Every call on one GPU uses the
 * same array, so calls that overlap on one GPU (two streams, two threads)
 * race and give undefined results; calls in one stream are ordered and safe.
 * The outputs equal those of the five calls bit for bit.  The index sets,
 * plan and debug word of MMSA_FLAG_DEBUG stay in the library's array and
 * cannot be viewed. */
#define MMSA_NOALLOC_SCRATCH_BYTES (64ull << 20)
mmsa_status mmsa_prefill_noalloc(const mmsa_layer_desc* desc, const void* q, const void* k, const void* v,
                                 void* o, float* lse, void* stream);

const char* mmsa_status_string(mmsa_status s);
const char* mmsa_last_error(void);
int32_t mmsa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MMSA_H */
