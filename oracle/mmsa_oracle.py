"""Plain CPU oracle of modality-aware dynamic sparse-attention prefill.

TEST INFRASTRUCTURE.  This module is the slow, obviously-correct definition
that the GPU library is checked against.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it; the product path never
does, and it shares no code, table or helper with the HIP library.

Sources (cited by page title and section; the pages print no pseudocode,
constant or worked example for any step, so every step below is the plainest
reading of their prose):
  [MI]  "MInference 1.0: Accelerating Pre-filling for Long-Context LLMs via
        Dynamic Sparse Attention" summary page, section "Approach":
        A-shape, vertical-slash and block-sparse patterns; indices estimated
        online from the attention of the last 64 queries (vertical and slash
        lines) and from mean-pooled 64-token blocks (block-sparse).
  [MM]  "MMInference: Accelerating Pre-filling for Long-Context Visual
        Language Models via Modality-Aware Permutation Sparse Attention"
        summary page, section "Approach": grid pattern, Q-boundary and
        2D-boundary patterns, row/column and modality-wise permutations.
  [MMV] the MMInference verdict page, fields key_machinery (grid stride and
        phase searched online on an approximate attention matrix built from the
        last 64 queries; kernels load only the permuted blocks) and
        core_discovery (row-wise permutation grouping same-modality queries,
        column-wise permutation aligning key strides, 2D permutation isolating
        each modality pair; index estimated from the last 64 queries of each
        modality segment).
  [PE]  the PEVLM verdict page (arXiv 2506.19651), field key_machinery: the
        parallel-encoding mask (a sink block, frame-aligned context blocks that
        each see themselves and the sink, a question block that sees
        everything) and its operation count over those blocks.

Precision: attention and estimation are computed in float64; the estimation
scores are rounded to float32 before any selection, because the selection
(top-k, grid rule) is defined on float32 scores so that it can be replayed
on scores exported by the GPU.

Parity pins live in tests/test_oracle_*.py.  Parity unpinned against the pages
themselves: the slash-to-tile reading, the grid stride/phase rule and the
boundary coordinates are this project's readings; they are pinned against
brute force and mathematics, not against the authors' implementation, which
is not available.  The parallel-encoding mask is the exception: its pair
count is pinned against the operation count [PE] prints, made causal.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

TILE = 64          # [MI] "Approach": 64-token blocks
N_EST = 64         # [MI] "Approach": the last 64 queries
TEXT, VIDEO = 0, 1
Q24 = 1 << 24      # grid rule fixed-point quantum 2^-24


# ---------------------------------------------------------------------------
# Head description (plain dicts in, dataclass inside)
# ---------------------------------------------------------------------------
@dataclass
class HeadCfg:
    pattern: str                 # 'ashape' | 'vs' | 'block' | 'grid' | 'parallel'
    layout: str = 'plain'        # 'plain' | 'q_boundary' | 'boundary_2d' | 'q_segment' | 'modality_grouped'
    sink: int = 0                # ashape / parallel / grid: sink keys (grid: 0, none)
    window: int = 1              # ashape: local window; parallel: context block; grid: window (0, none)
    k_vertical: int = 0
    k_slash: int = 0
    k_blocks: int = 0
    grid_phases: int = 1
    stride_lo: int = 64
    stride_hi: int = 512
    grid_clip: int = 8
    question: int = 0            # parallel: length of the trailing question block

    @staticmethod
    def of(d) -> "HeadCfg":
        if isinstance(d, HeadCfg):
            return d
        return HeadCfg(**d)


def _segments(L, segs):
    if not segs:
        return [(0, L, TEXT)] if L > 0 else []
    out = []
    pos = 0
    for s in segs:
        start, ln, m = int(s[0]), int(s[1]), int(s[2])
        if start != pos or ln <= 0 or m not in (TEXT, VIDEO):
            raise ValueError("segments must tile [0, L) in order")
        out.append((start, ln, m))
        pos += ln
    if pos != L:
        raise ValueError("segments must tile [0, L)")
    return out


def modality_tables(L, segs):
    """Modality m[p] and rank[p] (index of p among tokens of its modality)."""
    m = np.zeros(L, np.int64)
    for start, ln, mod in _segments(L, segs):
        m[start:start + ln] = mod
    rank = np.zeros(L, np.int64)
    n = [0, 0]
    for mod in (TEXT, VIDEO):
        sel = np.nonzero(m == mod)[0]
        rank[sel] = np.arange(sel.size)
        n[mod] = sel.size
    return m, rank, n


def segment_index(L, segs):
    """Index of the segment holding each position."""
    out = np.zeros(L, np.int64)
    for n_, (start, ln, _) in enumerate(_segments(L, segs)):
        out[start:start + ln] = n_
    return out


def grouped_positions(L, segs):
    """Modality-grouped order: text positions ascending, then video ascending
    ([MMV] core_discovery: permutation grouping same-modality tokens)."""
    m, _, _ = modality_tables(L, segs)
    return np.concatenate([np.nonzero(m == TEXT)[0], np.nonzero(m == VIDEO)[0]])


def grid_coordinate(L, segs, grouped):
    """Coordinate x(p) on which grid lines are evenly spaced: the original
    position, or the position in the modality-grouped order."""
    if not grouped:
        return np.arange(L, dtype=np.int64)
    x = np.empty(L, np.int64)
    x[grouped_positions(L, segs)] = np.arange(L)
    return x


# ---------------------------------------------------------------------------
# Estimation: last-64-query attention ([MI] "Approach"; [MMV] key_machinery)
# ---------------------------------------------------------------------------
def estimation_rows(query_positions):
    """The last min(64, n) queries of an ascending query set."""
    qp = np.asarray(query_positions, np.int64)
    return qp[-N_EST:]


def last_rows_attention(q_rows, k, row_pos, scale):
    """Exact causal softmax of each estimation row over all keys j <= i_r.

    Returns a[r, j] (0 where j > i_r), and the row max / row sum of exp in the
    natural-log domain (the statistics of the two-pass normalisation)."""
    q_rows = np.asarray(q_rows, np.float64)
    k = np.asarray(k, np.float64)
    L = k.shape[0]
    x = scale * (q_rows @ k.T)                       # (n_R, L)
    causal = np.arange(L)[None, :] <= np.asarray(row_pos)[:, None]
    x = np.where(causal, x, -np.inf)
    mx = x.max(axis=1)
    e = np.exp(x - mx[:, None])
    ssum = e.sum(axis=1)
    return e / ssum[:, None], mx, ssum


def vs_scores_original(a, row_pos, L):
    """Vertical score v[j] = sum_r a_r[j]; slash score s[o] = sum_r a_r[i_r - o]
    for o = i_r - j >= 0 (original coordinates)."""
    v = a.sum(axis=0)
    s = np.zeros(L, np.float64)
    for r, i in enumerate(np.asarray(row_pos)):
        s[:i + 1] += a[r, i::-1]
    return v, s


def vs_candidates_original(row_pos):
    """Candidate index ranges (lo, hi) of v and s: every column and every
    diagonal that meets the causal part of the estimation rows."""
    imax = int(np.max(row_pos))
    return (0, imax + 1), (0, imax + 1)


def vs_scores_pair(a, row_pos, row_rank, key_mod, key_rank, m_k, n_k, n_q):
    """2D-boundary scores of one (query modality, key modality) pair, in
    compacted coordinates: v over key ranks kappa in [0, n_k); s over the
    signed offset o = rho - kappa, stored at index o + n_k - 1."""
    cols = np.nonzero(key_mod == m_k)[0]              # ascending => rank order
    v = a[:, cols].sum(axis=0)
    s = np.zeros(max(n_q + n_k - 1, 0), np.float64)
    for r, rho in enumerate(np.asarray(row_rank)):
        # kappa = 0..n_k-1 lands on index rho + n_k - 1 - kappa
        s[rho:rho + n_k] += a[r, cols][::-1]
    # candidates: keys of m_k visible to some estimation row
    vis = [int(np.searchsorted(cols, i, side='right')) for i in row_pos]   # n'_k(r)
    nk_last = max(vis) if vis else 0
    vc = (0, nk_last)
    rows_with = [(int(rho), nv) for rho, nv in zip(row_rank, vis) if nv >= 1]
    if rows_with:
        hi = max(rho for rho, _ in rows_with)
        lo = min(rho - nv + 1 for rho, nv in rows_with)
        sc = (lo + n_k - 1, hi + n_k)
    else:
        sc = (0, 0)
    return v, s, vc, sc


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------
def topk_select(x_f32, k, lo=0, hi=None):
    """Indices of the k largest float32 scores among [lo, hi): order by value
    descending, ties to the lowest index; +0 and -0 compare equal; returned
    ascending.  k is clamped to the candidate count."""
    x = np.asarray(x_f32, dtype=np.float32)
    if hi is None:
        hi = x.shape[0]
    n = hi - lo
    k = min(int(k), n)
    if k <= 0:
        return np.zeros(0, np.int64)
    xs = x[lo:hi].astype(np.float64) + 0.0
    if np.isnan(xs).any():
        raise ValueError("NaN score")
    idx = np.arange(lo, hi, dtype=np.int64)
    order = np.lexsort((idx, -xs))
    return np.sort(idx[order[:k]])


# ---------------------------------------------------------------------------
# Grid stride / phase rule ([MMV] key_machinery: stride and phase found online
# by scanning the approximate attention of the last 64 queries).  Reading: a
# matched-filter z-score on clipped fixed-point vertical scores, compared in
# exact integers.
# ---------------------------------------------------------------------------
def _grid_key(X, cnt):
    """Exact ordering key of a (stride, phase) line family: sgn(X) X^2 / cnt."""
    X = int(X)
    return Fraction((1 if X > 0 else -1 if X < 0 else 0) * X * X, int(cnt))


def grid_rule(v_f32, D, n_rows, clip, stride_lo, stride_hi, phases):
    """Returns (sigma, sorted phases).

    u[x] = min(floor(v[x] * 2^24), floor(clip * n_rows * 2^24 / D)) for x < D;
    U = sum u; for stride s and phase f < s: F = sum_{x = f mod s} u[x],
    cnt = ceil((D - f) / s), X = D*F - cnt*U.  (s, f) beats (s', f') iff
    sgn(X) X^2 cnt' > sgn(X') X'^2 cnt; ties go to the smaller stride, then the
    smaller phase.  The phases kept are the best `phases` at the winning stride."""
    D = int(D)
    v = np.asarray(v_f32, np.float32)[:D].astype(np.float64)
    u = np.floor(v * Q24).astype(np.int64)
    cap = (int(clip) * int(n_rows) * Q24) // D
    u = np.minimum(u, cap)
    U = int(u.sum())
    s_lo = min(int(stride_lo), D)
    s_hi = min(int(stride_hi), D)
    best = None                                   # (key, -sigma, sigma)
    best_sigma = None
    for sig in range(s_lo, s_hi + 1):
        n_full = -(-D // sig)
        up = np.zeros(n_full * sig, np.int64)
        up[:D] = u
        F = up.reshape(n_full, sig).sum(axis=0)
        phi = np.arange(sig, dtype=np.int64)
        cnt = (D - phi + sig - 1) // sig
        X = D * F - cnt * U
        # float pre-filter, then exact comparison among near-maxima
        approx = np.sign(X) * (X.astype(np.float64) ** 2) / cnt
        amax = approx.max()
        if amax > 0:
            cand = np.nonzero(approx >= amax * (1 - 1e-9))[0]
        else:
            cand = np.nonzero(X == X.max())[0] if X.max() == 0 else np.nonzero(approx >= amax * (1 + 1e-9))[0]
        keys = [(_grid_key(X[f], cnt[f]), -int(f)) for f in cand]
        kbest = max(keys)
        if best is None or kbest[0] > best[0]:
            best = kbest
            best_sigma = (sig, X, cnt)
    sig, X, cnt = best_sigma
    w = min(int(phases), sig)
    allk = sorted(((_grid_key(X[f], cnt[f]), -f) for f in range(sig)), reverse=True)
    ph = sorted(-negf for _, negf in allk[:w])
    return sig, np.array(ph, np.int64)


# ---------------------------------------------------------------------------
# Block-sparse estimation ([MI] "Approach": mean-pooled 64-block attention)
# ---------------------------------------------------------------------------
def pool_blocks(x):
    """Mean of each 64-row block (the last block averages its real rows)."""
    x = np.asarray(x, np.float64)
    L = x.shape[0]
    nB = -(-L // TILE)
    out = np.zeros((nB, x.shape[1]), np.float64)
    for b in range(nB):
        out[b] = x[b * TILE:min(L, (b + 1) * TILE)].mean(axis=0)
    return out


def block_logits(qp, kp, scale):
    """Pooled logits z[b, c] = scale * Qp[b] . Kp[c], rounded to float32."""
    return (scale * (np.asarray(qp, np.float64) @ np.asarray(kp, np.float64).T)).astype(np.float32)


def block_select(z_f32, k_blocks):
    """Per query block b: the top min(k, b+1) key blocks among c <= b."""
    z = np.asarray(z_f32, np.float32)
    return [topk_select(z[b], min(k_blocks, b + 1), 0, b + 1) for b in range(z.shape[0])]


# ---------------------------------------------------------------------------
# Index sets of one head
# ---------------------------------------------------------------------------
@dataclass
class HeadIndex:
    cfg: HeadCfg
    L: int
    segs: list
    # VS family: key -> (V, S) where key is 'all', a query modality m, or (m_q, m_k)
    vs: dict = field(default_factory=dict)
    blocks: list = None                       # BLOCK: list of arrays per query block
    sigma: int = 0                            # GRID
    phases: np.ndarray = None
    x: np.ndarray = None                      # GRID coordinate
    extras: dict = field(default_factory=dict)


def _region_rows_for_modality(mtab, mod):
    return estimation_rows(np.nonzero(mtab == mod)[0])


def estimate_head(cfg, qh, kh, segs, scale, scores_override=None):
    """Online index estimation of one head.

    qh (L, d), kh (L, d): float arrays holding the bf16 input values.
    scores_override: optional dict of float32 score vectors (same keys as the
    `extras` this function records) used instead of the oracle's own scores,
    so that selection can be replayed on scores exported by the GPU."""
    cfg = HeadCfg.of(cfg)
    L = qh.shape[0]
    segs = _segments(L, segs)
    hi = HeadIndex(cfg=cfg, L=L, segs=segs)
    ov = scores_override or {}
    if cfg.pattern in ('ashape', 'parallel') or L == 0:
        return hi
    if cfg.pattern == 'block':
        z = ov['z'] if 'z' in ov else block_logits(pool_blocks(qh), pool_blocks(kh), scale)
        hi.extras['z'] = z
        hi.blocks = block_select(z, cfg.k_blocks)
        return hi
    mtab, rtab, n = modality_tables(L, segs)
    if cfg.pattern == 'grid':
        grouped = cfg.layout == 'modality_grouped'
        x = grid_coordinate(L, segs, grouped)
        order = grouped_positions(L, segs) if grouped else np.arange(L)
        rows = estimation_rows(order)
        rows = np.sort(rows)
        imax = int(rows.max())
        D = int(x[:imax + 1].max()) + 1
        if 'v' in ov:            # selection replayed on given scores: nothing to compute
            v32, mx, ssum = ov['v'], None, None
        else:
            a, mx, ssum = last_rows_attention(qh[rows], kh, rows, scale)
            vx = np.zeros(L, np.float64)
            vx[x] = a.sum(axis=0)
            v32 = vx.astype(np.float32)
        hi.extras.update(v=v32, D=D, n_rows=len(rows), rows=rows, stats=(mx, ssum))
        hi.sigma, hi.phases = grid_rule(v32, D, len(rows), cfg.grid_clip or 8,
                                        cfg.stride_lo, cfg.stride_hi, cfg.grid_phases)
        hi.x = x
        return hi
    assert cfg.pattern == 'vs'
    if cfg.layout == 'plain':
        regions = [('all', estimation_rows(np.arange(L)))]
    elif cfg.layout == 'q_segment':
        # [MMV] core_discovery names estimation from the last 64 queries of
        # each modality segment; this layout takes every segment on its own
        regions = [(('seg', n_), estimation_rows(np.arange(start, start + ln)))
                   for n_, (start, ln, _) in enumerate(segs)]
    else:
        regions = [(mod, _region_rows_for_modality(mtab, mod)) for mod in (TEXT, VIDEO) if n[mod] > 0]
    for key, rows in regions:
        given = cfg.layout != 'boundary_2d' and ('v', key) in ov and ('s', key) in ov
        if given:                # selection replayed on given scores: nothing to compute
            hi.extras[('stats', key)] = (None, None)
        else:
            a, mx, ssum = last_rows_attention(qh[rows], kh, rows, scale)
            hi.extras[('stats', key)] = (mx, ssum)
        if cfg.layout in ('plain', 'q_boundary', 'q_segment'):
            vc, sc = vs_candidates_original(rows)
            if given:
                v32, s32 = ov[('v', key)], ov[('s', key)]
            else:
                v, s = vs_scores_original(a, rows, L)
                v32, s32 = v.astype(np.float32), s.astype(np.float32)
            hi.extras[('v', key)], hi.extras[('s', key)] = v32, s32
            hi.extras[('cand', key)] = (vc, sc)
            hi.vs[key] = (topk_select(v32, cfg.k_vertical, *vc), topk_select(s32, cfg.k_slash, *sc))
        else:  # boundary_2d
            m_q = key
            row_rank = rtab[rows]
            for m_k in (TEXT, VIDEO):
                if n[m_k] == 0:
                    continue
                v, s, vc, sc = vs_scores_pair(a, rows, row_rank, mtab, rtab, m_k, n[m_k], n[m_q])
                pk = (m_q, m_k)
                v32 = ov.get(('v', pk), v.astype(np.float32))
                s32 = ov.get(('s', pk), s.astype(np.float32))
                hi.extras[('v', pk)], hi.extras[('s', pk)] = v32, s32
                hi.extras[('cand', pk)] = (vc, sc)
                hi.vs[pk] = (topk_select(v32, cfg.k_vertical, *vc), topk_select(s32, cfg.k_slash, *sc))
    return hi


# ---------------------------------------------------------------------------
# Masks (which keys a query row attends to), always with causality j <= i
# ---------------------------------------------------------------------------
def _tile_rows(hi, i, mtab, rtab):
    """Rows of the query tile that holds row i, as original positions: 64
    consecutive positions for plain heads, 64 consecutive ranks of one
    modality for boundary heads (rows grouped by modality)."""
    L = hi.L
    if hi.cfg.layout in ('q_boundary', 'boundary_2d'):
        mod = mtab[i]
        t = rtab[i] // TILE
        pos = np.nonzero(mtab == mod)[0]
        return pos[t * TILE:(t + 1) * TILE]
    if hi.cfg.layout == 'q_segment':   # 64 consecutive positions of one segment
        for start, ln, _ in hi.segs:
            if start <= i < start + ln:
                t0 = start + ((i - start) // TILE) * TILE
                return np.arange(t0, min(start + ln, t0 + TILE))
    t = i // TILE
    return np.arange(t * TILE, min(L, (t + 1) * TILE))


def _vs_key(hi, i, mtab):
    """The index set row i uses: the layer's, its modality's or its segment's."""
    if hi.cfg.layout == 'plain':
        return 'all'
    if hi.cfg.layout == 'q_segment':
        if 'segidx' not in hi.extras:
            hi.extras['segidx'] = segment_index(hi.L, hi.segs)
        return ('seg', int(hi.extras['segidx'][i]))
    return int(mtab[i])


def _slash_tiles_original(rows, S):
    """Key tiles crossed by the selected diagonals over the tile's rows:
    {floor((p - o) / 64) : p in rows, o in S, p >= o}."""
    if len(S) == 0:
        return np.zeros(0, np.int64)
    diff = np.asarray(rows)[:, None] - np.asarray(S)[None, :]
    return np.unique(diff[diff >= 0] // TILE)


def parallel_floor(cfg, L, i):
    """[PE] key_machinery, the parallel-encoding mask.  Tokens [0, S) form the
    sink block (S = cfg.sink), the last Q tokens the question block
    (Q = cfg.question), and the tokens between them are cut into context
    blocks of B = cfg.window tokens from S on (the last one may be shorter).
    A context row sees the sink block and its own block; sink and question
    rows see every earlier token.  Returns the first non-sink key row i may
    see: the start of its context block, or 0 for sink and question rows."""
    S, B = cfg.sink, cfg.window
    qs = L - min(cfg.question, L)
    if i < S or i >= qs:
        return 0
    return S + ((i - S) // B) * B


def row_mask(hi, i, cache=None):
    """Boolean mask over keys 0..L-1 of the keys selected for query row i."""
    cfg, L = hi.cfg, hi.L
    j = np.arange(L)
    causal = j <= i
    if cfg.pattern == 'ashape':
        return causal & ((j < cfg.sink) | (i - j < cfg.window))
    if cfg.pattern == 'parallel':
        return causal & ((j < cfg.sink) | (j >= parallel_floor(cfg, L, i)))
    if cfg.pattern == 'block':
        sel = np.zeros(-(-L // TILE), bool)
        sel[hi.blocks[i // TILE]] = True
        return causal & sel[j // TILE]
    if cfg.pattern == 'grid':
        # lines of both kinds, plus an optional sink and local window on the
        # rows (R12 widened: window and sink default to 0, none)
        line = np.isin(hi.x % hi.sigma, hi.phases)
        return causal & (line[i] | line | (j < cfg.sink) | (i - j < cfg.window))
    # VS family
    if cache is None:
        cache = {}
    if 'mr' not in cache:
        cache['mr'] = modality_tables(L, hi.segs)
    mtab, rtab, n = cache['mr']
    rows = _tile_rows(hi, i, mtab, rtab)
    sel = np.zeros(L, bool)
    if cfg.layout in ('plain', 'q_boundary', 'q_segment'):
        key = _vs_key(hi, i, mtab)
        V, S = hi.vs[key]
        tiles = _slash_tiles_original(rows, S)
        tsel = np.zeros(-(-L // TILE), bool)
        tsel[tiles] = True
        sel |= tsel[j // TILE]
        sel[V] = True
        return causal & sel
    m_q = int(mtab[i])
    rho = rtab[rows]
    for m_k in (TEXT, VIDEO):
        if (m_q, m_k) not in hi.vs:
            continue
        V, S = hi.vs[(m_q, m_k)]
        n_k = n[m_k]
        keys = np.nonzero(mtab == m_k)[0]
        o = np.asarray(S) - (n_k - 1)
        kap = (rho[:, None] - o[None, :]).ravel()
        kap = kap[(kap >= 0) & (kap < n_k)]
        tiles = np.unique(kap // TILE)
        ksel = np.zeros(n_k, bool)
        if tiles.size:
            ksel |= np.isin(np.arange(n_k) // TILE, tiles)
        ksel[V] = True
        sel[keys[ksel]] = True
    return causal & sel


def pair_count(hi, rows=None):
    """Number of selected causal (query, key) pairs over the given rows."""
    rows = range(hi.L) if rows is None else rows
    cache = {}
    return int(sum(int(row_mask(hi, int(i), cache).sum()) for i in rows))


# ---------------------------------------------------------------------------
# Attention over a mask (dense masked softmax, float64)
# ---------------------------------------------------------------------------
def attend_rows(q, k, v, rows, mask_fn, scale):
    """For each row i: softmax over the selected keys of scale * q_i . k_j,
    output sum_j p_j v_j and the natural-log LSE.  A row with no selected key
    gives a zero output and LSE = -inf."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    out = np.zeros((len(rows), v.shape[1]), np.float64)
    lse = np.full(len(rows), -np.inf)
    for n_, i in enumerate(rows):
        J = np.nonzero(mask_fn(int(i)))[0]
        if J.size == 0:
            continue
        s = scale * (k[J] @ q[int(i)])
        m = s.max()
        p = np.exp(s - m)
        den = p.sum()
        out[n_] = (p @ v[J]) / den
        lse[n_] = m + math.log(den)
    return out, lse


def head_attention(hi, qh, kh, vh, scale, rows=None):
    """Direct masked attention of one head on the given rows (default: all)."""
    rows = np.arange(hi.L) if rows is None else np.asarray(rows)
    cache = {}
    return attend_rows(qh, kh, vh, rows, lambda i: row_mask(hi, i, cache), scale)


# ---------------------------------------------------------------------------
# Attention recall of a mask ([MI] "Approach": the offline search scores each
# pattern and budget by attention recall at the FLOPs the kernel spends)
# ---------------------------------------------------------------------------
def head_recall(hi, qh, kh, scale, rows=None):
    """Per row: the share of the row's dense causal softmax (keys j <= i) that
    falls on the keys its mask selects.  Float64, straight from the
    definition: normalise over all causal keys, then sum over the mask."""
    rows = np.arange(hi.L) if rows is None else np.asarray(rows)
    q = np.asarray(qh, np.float64)
    k = np.asarray(kh, np.float64)
    out = np.zeros(len(rows), np.float64)
    cache = {}
    for n_, i in enumerate(rows):
        i = int(i)
        s = scale * (k[:i + 1] @ q[i])
        p = np.exp(s - s.max())
        p /= p.sum()
        out[n_] = p[row_mask(hi, i, cache)[:i + 1]].sum()
    return out


# ---------------------------------------------------------------------------
# Permuted mode (self-check only): permute rows, plan tiles in the permuted
# coordinates, attend tile by tile, scatter back.  Shares the definitions of
# the index sets with the direct mode but not its mask construction.
# ---------------------------------------------------------------------------
def _pad_to_tile(arr):
    n = len(arr)
    padn = -(-n // TILE) * TILE
    out = np.full(padn, -1, np.int64)
    out[:n] = arr
    return out


def row_order(hi):
    """Permuted row order (original position per slot, -1 for padding)."""
    cfg, L = hi.cfg, hi.L
    if cfg.pattern == 'grid':
        line = np.isin(hi.x % hi.sigma, hi.phases)
        return np.concatenate([_pad_to_tile(np.nonzero(line)[0]), _pad_to_tile(np.nonzero(~line)[0])])
    if cfg.pattern == 'vs' and cfg.layout in ('q_boundary', 'boundary_2d'):
        mtab, _, _ = modality_tables(L, hi.segs)
        return np.concatenate([_pad_to_tile(np.nonzero(mtab == m)[0]) for m in (TEXT, VIDEO)])
    if cfg.pattern == 'vs' and cfg.layout == 'q_segment':
        return np.concatenate([_pad_to_tile(np.arange(start, start + ln)) for start, ln, _ in hi.segs])
    return _pad_to_tile(np.arange(L))


def tile_plan(hi, tile_rows):
    """For one query tile (original positions of its rows, no padding): the
    key groups to load.  Each group is an array of original key positions:
    whole 64-key tiles of the head's key view, then gathered single columns
    that no listed tile already holds."""
    cfg, L = hi.cfg, hi.L
    pmax = int(tile_rows.max())
    nT = -(-L // TILE)
    tiles_orig = lambda ts: [np.arange(c * TILE, min(L, (c + 1) * TILE)) for c in ts]
    if cfg.pattern == 'ashape':
        t = pmax // TILE
        lo = max(0, int(tile_rows.min()) - cfg.window + 1) // TILE
        ts = sorted(set(range(min(-(-cfg.sink // TILE), t + 1))) | set(range(lo, t + 1)))
        return tiles_orig(ts), []
    if cfg.pattern == 'parallel':
        # the sink tiles, and every tile from the lowest first-visible key of
        # the tile's rows up to its last row
        t = pmax // TILE
        lo = min(parallel_floor(cfg, L, int(r)) for r in tile_rows) // TILE
        ts = sorted(set(range(min(-(-cfg.sink // TILE), t + 1))) | set(range(lo, t + 1)))
        return tiles_orig(ts), []
    if cfg.pattern == 'block':
        return tiles_orig(hi.blocks[pmax // TILE]), []
    if cfg.pattern == 'grid':
        line = np.isin(hi.x % hi.sigma, hi.phases)
        if line[tile_rows].all():
            return tiles_orig(range(pmax // TILE + 1)), []
        keys = np.nonzero(line)[0]
        keys = keys[keys <= pmax]
        # sink and window tiles; line keys inside them are not gathered again
        t = pmax // TILE
        ts = set(range(min(-(-cfg.sink // TILE), t + 1)))
        if cfg.window > 0:
            ts |= set(range(max(0, int(tile_rows.min()) - cfg.window + 1) // TILE, t + 1))
        return tiles_orig(sorted(ts)), [keys[~np.isin(keys // TILE, sorted(ts))]]
    mtab, rtab, n = modality_tables(L, hi.segs)
    if cfg.layout in ('plain', 'q_boundary', 'q_segment'):
        V, S = hi.vs[_vs_key(hi, int(tile_rows[0]), mtab)]
        ts = _slash_tiles_original(tile_rows, S)
        tset = set(int(c) for c in ts)
        gath = np.array([c for c in V if c <= pmax and (c // TILE) not in tset], np.int64)
        return tiles_orig(sorted(tset)), [gath]
    m_q = int(mtab[tile_rows[0]])
    rho = rtab[tile_rows]
    groups, gath = [], []
    for m_k in (TEXT, VIDEO):
        if (m_q, m_k) not in hi.vs:
            continue
        V, S = hi.vs[(m_q, m_k)]
        n_k = n[m_k]
        keys = np.nonzero(mtab == m_k)[0]
        o = np.asarray(S) - (n_k - 1)
        kap = (rho[:, None] - o[None, :]).ravel()
        kap = kap[(kap >= 0) & (kap < n_k)]
        tset = set(int(c) for c in np.unique(kap // TILE))
        for c in sorted(tset):
            groups.append(keys[c * TILE:min(n_k, (c + 1) * TILE)])
        g = np.array([keys[c] for c in V if (c // TILE) not in tset], np.int64)
        gath.append(g[g <= pmax] if g.size else g)
    return groups, gath


def permuted_attention(hi, qh, kh, vh, scale):
    """Attention computed in the permuted coordinates, then unpermuted."""
    cfg, L = hi.cfg, hi.L
    order = row_order(hi)
    out = np.zeros((L, vh.shape[1]), np.float64)
    lse = np.full(L, -np.inf)
    for t0 in range(0, len(order), TILE):
        slot = order[t0:t0 + TILE]
        rows = slot[slot >= 0]
        if rows.size == 0:
            continue
        groups, gath = tile_plan(hi, rows)
        cand = [g for g in groups] + [g for g in gath if len(g)]
        keys = np.concatenate(cand) if cand else np.zeros(0, np.int64)
        line = np.isin(hi.x % hi.sigma, hi.phases) if cfg.pattern == 'grid' else None
        for i in rows:
            kk = keys[keys <= i]
            if cfg.pattern == 'grid' and not line[i]:
                kk = kk[line[kk] | (kk < cfg.sink) | (i - kk < cfg.window)]
            if cfg.pattern == 'ashape':
                kk = kk[(kk < cfg.sink) | (i - kk < cfg.window)]
            if cfg.pattern == 'parallel':
                kk = kk[(kk < cfg.sink) | (kk >= parallel_floor(cfg, L, int(i)))]
            if kk.size == 0:
                continue
            s = scale * (np.asarray(kh, np.float64)[kk] @ np.asarray(qh, np.float64)[i])
            m = s.max()
            p = np.exp(s - m)
            out[i] = (p @ np.asarray(vh, np.float64)[kk]) / p.sum()
            lse[i] = m + math.log(p.sum())
    return out, lse


# ---------------------------------------------------------------------------
# A whole layer
# ---------------------------------------------------------------------------
def kv_head_map(Hq, Hkv, kv_head_of=None):
    if kv_head_of is not None:
        return [int(g) for g in kv_head_of]
    return [h // (Hq // Hkv) for h in range(Hq)]


def estimate_layer(q, k, heads, segs, scale, kv_head_of=None):
    """q: (Hq, L, d), k: (Hkv, L, d) -> list of HeadIndex."""
    Hq = q.shape[0]
    gmap = kv_head_map(Hq, k.shape[0], kv_head_of)
    return [estimate_head(heads[h], q[h], k[gmap[h]], segs, scale) for h in range(Hq)]
