"""Seeded random layers through the whole path against the CPU oracle.

Each case draws a segment layout (1-5 text/video segments of uneven
lengths), a ragged L, d in {64, 128}, a GQA head map and, per head, any
pattern and layout the library supports with random budgets; some cases take
the materialised permutation, and odd seeds walk key tiles lowest first (the
order the library picks by itself only for layers whose K/V pass 256 MB).  The checks are those of the fixed cases
(index sets bit-exact on the GPU's scores, scores within 1e-3, attention
within 2e-2 / 2e-3, exact per-tile pair counts).
"""
import numpy as np
import pytest

from dynamic_sparse_attention_head_amd import mmsa, synth
from parity_util import full_check

pytestmark = pytest.mark.gpu

TEXT, VIDEO = 0, 1


def random_head(rng, L, has_video, scale=1):
    kind = rng.choice(["ashape", "vs", "vs_qb", "vs_2d", "vs_seg", "block", "grid", "grid_grouped", "parallel"])
    kv, ks = int(rng.integers(0, 80 * scale)), int(rng.integers(0, 200 * scale))
    if kind == "ashape":
        return synth.ashape(int(rng.integers(0, 200 * scale)), int(rng.integers(1, 600 * scale)))
    if kind == "vs":
        return synth.vs(kv, ks)
    if kind == "vs_qb":
        return synth.vs(kv, ks, "q_boundary")
    if kind == "vs_2d":
        return synth.vs(kv, ks, "boundary_2d")
    if kind == "vs_seg":
        return synth.vs(kv, ks, "q_segment")
    if kind == "block":
        return synth.block(int(rng.integers(0, 12 * scale)))
    if kind == "parallel":
        return synth.parallel(int(rng.integers(0, 300 * scale)), int(rng.integers(1, 400 * scale)),
                              int(rng.integers(0, 300 * scale)))
    layout = "modality_grouped" if kind == "grid_grouped" else "plain"
    lo = int(rng.integers(16, 60))
    sink, window = 0, 0
    if rng.integers(0, 2):      # half the grid heads add a sink and a local window
        sink, window = int(rng.integers(0, 100 * scale)), int(rng.integers(0, 400 * scale))
    return synth.grid(int(rng.integers(1, 4)), lo, lo + int(rng.integers(0, 120)), layout=layout,
                      sink=sink, window=window)


def random_spec(seed):
    rng = np.random.default_rng(seed)
    n_seg = int(rng.integers(1, 6))
    segs, pos = [], 0
    for _ in range(n_seg):
        n = int(rng.integers(1, 500))
        segs.append((pos, n, int(rng.integers(0, 2))))
        pos += n
    L = pos
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 4))
    has_video = any(m == VIDEO for _, _, m in segs)
    heads = [random_head(rng, L, has_video) for _ in range(Hq)]
    spec = synth.small_spec(f"random{seed}", L, Hq, Hkv, d, heads, seed=1000 + seed, segs=segs,
                            period=49, period_amp=3.0)
    return spec, bool(rng.integers(0, 4) == 0)


@pytest.mark.parametrize("seed", range(160))
def test_random_layer(seed):
    spec, materialize = random_spec(seed)
    full_check(spec, materialize=materialize, flags=mmsa.FLAG_KEYS_ASCENDING if seed % 2 else 0)


def random_medium_spec(seed):
    """4K-30K tokens: key-tile bitmaps of 2-8 words (the small layers above
    fit one), 1-8 segments, budgets scaled up with the length."""
    rng = np.random.default_rng(10_000 + seed)
    L = int(rng.integers(4100, 30_000))
    n_seg = int(rng.integers(1, 9))
    cuts = np.sort(rng.choice(np.arange(1, L), n_seg - 1, replace=False)) if n_seg > 1 else np.array([], int)
    bounds = [0, *[int(c) for c in cuts], L]
    segs = [(bounds[i], bounds[i + 1] - bounds[i], int(rng.integers(0, 2))) for i in range(n_seg)]
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 4))
    has_video = any(m == VIDEO for _, _, m in segs)
    heads = [random_head(rng, L, has_video, scale=4) for _ in range(Hq)]
    spec = synth.small_spec(f"random-medium{seed}", L, Hq, Hkv, d, heads, seed=2000 + seed, segs=segs,
                            period=49, period_amp=3.0)
    return spec


@pytest.mark.parametrize("seed", range(8))
def test_random_medium_layer(seed):
    spec = random_medium_spec(seed)
    rng = np.random.default_rng(seed)
    n_tiles = -(-spec.L // 64)
    tiles = sorted({0, n_tiles - 1} | set(int(t) for t in rng.integers(0, n_tiles, 40)))
    full_check(spec, rows_per_head=256, pair_tiles=tiles, seed=seed,
               flags=mmsa.FLAG_KEYS_ASCENDING if seed % 2 else 0)
