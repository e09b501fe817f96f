"""GPU parity of the whole path (estimation, permutation, plan, attention,
inverse permutation) against the CPU oracle, through the C ABI, with the
permutation index-based inside the attention call (the default) and
materialised by explicit gathers and an output scatter.

Sizes are small enough for the oracle to finish in seconds and still span
several 64-tiles with a ragged tail; every pattern and layout is covered.
"""
import numpy as np
import pytest
import torch

from dynamic_sparse_attention_head_amd import mmsa, synth
from parity_util import full_check, run_gpu

pytestmark = pytest.mark.gpu

TEXT, VIDEO = 0, 1


def test_tiny_config_all_rows():
    # 4K tokens, d = 64: head 0 A-shape (64, 512), head 1 vertical-slash (128, 256)
    full_check(synth.config(1))


def test_mixed_heads_ragged():
    heads = [synth.vs(40, 90), synth.vs(7, 300), synth.block(5), synth.ashape(64, 256),
             synth.block(1000), synth.ashape(0, 1), synth.vs(0, 3), synth.block(1)]
    spec = synth.small_spec("mixed", 1000, 8, 2, 128, heads, seed=11, rope_base=1e4, strong_cols=16)
    full_check(spec)


def test_block_heads_clustered():
    spec = synth.small_spec("blocks", 3000 + 17, 4, 2, 128, [synth.block(12)] * 4, seed=3, cluster_blocks=8)
    full_check(spec, rows_per_head=256)


def test_grid_plain_ragged():
    frames = 9
    L = 70 + 196 * frames + 23
    segs = [(0, 70, TEXT), (70, 196 * frames, VIDEO), (70 + 196 * frames, 23, TEXT)]
    heads = [synth.grid(1, 16, 400), synth.grid(2, 64, 512), synth.vs(30, 60), synth.grid(3, 100, 300)]
    spec = synth.small_spec("grid", L, 4, 2, 128, heads, seed=5, segs=segs, period=196, period_amp=3.0)
    full_check(spec, rows_per_head=200)


def test_grid_with_sink_and_window_ragged():
    # grid heads whose rows off the lines also keep a sink and a local window
    # (line keys inside the window come once), plain and modality-grouped
    frames = 9
    L = 70 + 196 * frames + 23
    segs = [(0, 70, TEXT), (70, 196 * frames, VIDEO), (70 + 196 * frames, 23, TEXT)]
    heads = [synth.grid(1, 16, 400, sink=64, window=300), synth.grid(2, 64, 512, window=1),
             synth.grid(3, 100, 300, sink=100), synth.grid(1, 16, 128, layout="modality_grouped", sink=30, window=500),
             synth.grid(1, 16, 400, window=5000)]
    spec = synth.small_spec("grid-window", L, 5, 1, 128, heads, seed=7, segs=segs, period=196, period_amp=3.0)
    full_check(spec, rows_per_head=300)


def test_grid_with_window_d64_materialized():
    segs, L = synth.interleaved_segments(3, 4, 49, 77)
    heads = [synth.grid(2, 16, 200, layout="modality_grouped", sink=13, window=130),
             synth.grid(1, 16, 100, window=64)]
    spec = synth.small_spec("grid-window-mat", L, 2, 1, 64, heads, seed=17, segs=segs, period=49, period_amp=3.0)
    full_check(spec, materialize=True)


def test_boundary_layouts_on_tile_aligned_segments():
    # segments on 64-token boundaries: the full tiles of Q-boundary and
    # per-segment heads take the shifted-bitmap plan, as plain heads do
    segs = [(0, 128, TEXT), (128, 640, VIDEO), (768, 192, TEXT), (960, 576, VIDEO), (1536, 37, TEXT)]
    heads = [synth.vs(20, 60, "q_boundary"), synth.vs(12, 90, "q_segment"), synth.vs(15, 80),
             synth.vs(25, 33, "boundary_2d")]
    full_check(synth.small_spec("aligned", 1573, 4, 2, 128, heads, seed=71, segs=segs, period=64, period_amp=3.0))


def test_boundary_long_single_modality_runs():
    # a 7K-token video run: same-modality 2D pairs reach more query plus key
    # tiles than the head's tile bitmap has bits (the plan's shift bitmaps
    # must cover both)
    segs = [(0, 640, TEXT), (640, 7040, VIDEO), (7680, 93, TEXT)]
    heads = [synth.vs(30, 200, "boundary_2d"), synth.vs(30, 200, "q_boundary"), synth.vs(9, 700, "boundary_2d"),
             synth.vs(9, 700)]
    full_check(synth.small_spec("long-runs", 7773, 4, 2, 128, heads, seed=73, segs=segs, period=64,
                                period_amp=3.0), rows_per_head=400)


def test_boundary_layouts():
    full_check(boundary_spec())


def test_boundary_text_first_and_single_modality():
    segs = [(0, 130, TEXT), (130, 300, VIDEO), (430, 90, TEXT)]
    heads = [synth.vs(20, 40, "q_boundary"), synth.vs(25, 33, "boundary_2d"),
             synth.grid(1, 16, 100, layout="modality_grouped"), synth.vs(9, 9, "boundary_2d")]
    full_check(synth.small_spec("tv", 520, 4, 2, 64, heads, seed=2, segs=segs, period=49))
    # a video-only layer: every boundary layout reduces to its plain form
    full_check(synth.small_spec("v", 333, 2, 1, 128, [synth.vs(10, 20, "boundary_2d"),
                                                      synth.vs(10, 20, "q_boundary")],
                                seed=4, segs=[(0, 333, VIDEO)]))


def boundary_spec():
    segs, L = synth.interleaved_segments(3, 4, 49, 77)
    heads = [synth.grid(2, 16, 200, layout="modality_grouped"), synth.vs(20, 40, "q_boundary"),
             synth.vs(25, 33, "boundary_2d"), synth.vs(15, 80, "plain")]
    return synth.small_spec("boundary", L, 4, 1, 128, heads, seed=9, segs=segs, period=49, period_amp=3.0)


def test_boundary_layouts_materialized():
    # explicit gathers of permuted Q and grouped K/V, output scattered by unpermute
    full_check(boundary_spec(), materialize=True)


@pytest.mark.parametrize("which", ["boundary", "grid"])
def test_index_based_equals_materialized(which):
    if which == "boundary":
        spec = boundary_spec()
    else:
        frames = 9
        L = 70 + 196 * frames + 23
        segs = [(0, 70, TEXT), (70, 196 * frames, VIDEO), (70 + 196 * frames, 23, TEXT)]
        heads = [synth.grid(1, 16, 400), synth.grid(2, 64, 512, layout="modality_grouped"), synth.vs(30, 60, "boundary_2d")]
        spec = synth.small_spec("grid", L, 3, 1, 64, heads, seed=5, segs=segs, period=196, period_amp=3.0)
    _, q, k, v, o_idx, lse_idx = run_gpu(spec)
    L2, _, _, _, o_mat, lse_mat = run_gpu(spec, q=q, k=k, v=v, materialize=True)
    # the same values in the same arithmetic order: bit-identical
    assert torch.equal(o_idx.view(torch.int16), o_mat.view(torch.int16))
    assert torch.equal(lse_idx.view(torch.int32), lse_mat.view(torch.int32))
    assert L2.workspace_bytes() > mmsa_layer_bytes(spec, q, k, v)


def mmsa_layer_bytes(spec, q, k, v):
    from dynamic_sparse_attention_head_amd import mmsa
    return mmsa.Layer(q, k, v, spec.heads, segs=spec.segs).workspace_bytes()


@pytest.mark.parametrize("L", [1, 63, 64, 65, 130])
def test_edge_lengths(L):
    heads = [synth.vs(3, 5), synth.block(2), synth.ashape(4, 16), synth.grid(1, 16, 64)]
    full_check(synth.small_spec("edge", L, 4, 4, 64, heads, seed=L))


def segment_spec(d=128, seed=31):
    # text and video segments of uneven, untiled lengths, one of them shorter
    # than the 64 estimation rows
    segs = [(0, 100, TEXT), (100, 49 * 9, VIDEO), (541, 37, TEXT), (578, 49 * 11, VIDEO), (1117, 130, TEXT)]
    heads = [synth.vs(20, 40, "q_segment"), synth.vs(7, 90, "q_segment"), synth.vs(20, 40, "q_boundary"),
             synth.vs(15, 30)]
    return synth.small_spec("segment", 1247, 4, 2, d, heads, seed=seed, segs=segs, period=49, period_amp=3.0)


def test_segment_layout():
    full_check(segment_spec())


def test_segment_layout_d64_materialized():
    full_check(segment_spec(d=64, seed=32), materialize=True)


def test_segment_layout_single_segment():
    full_check(synth.small_spec("seg1", 333, 2, 1, 128, [synth.vs(10, 20, "q_segment"), synth.vs(10, 20)],
                                seed=33, segs=[(0, 333, VIDEO)]))


def many_segments_spec(n_seg=640, seed=41):
    # 640 segments of 1-40 tokens with modalities drawn at random (an
    # interleaved image-text document): hundreds of per-segment estimates per
    # head, more estimation batches than one wave of workgroups, hundreds of
    # segment-padded query tiles, and modality parts split into many runs
    rng = np.random.default_rng(seed)
    segs, pos = [], 0
    for _ in range(n_seg):
        n = int(rng.integers(1, 41))
        segs.append((pos, n, int(rng.integers(0, 2))))
        pos += n
    heads = [synth.vs(20, 40, "q_segment"), synth.vs(12, 60, "q_segment"), synth.vs(20, 40, "boundary_2d"),
             synth.vs(10, 30, "q_boundary"), synth.grid(1, 16, 64, layout="modality_grouped"), synth.block(6),
             synth.vs(9, 50, "q_segment"), synth.grid(2, 16, 80, sink=30, window=200)]
    return synth.small_spec("many-segments", pos, 8, 2, 64, heads, seed=seed, segs=segs, period=49, period_amp=3.0)


def test_many_short_segments():
    # every tile's pair count, attention on 400 sampled rows per head
    full_check(many_segments_spec(), rows_per_head=400)


def test_uneven_kv_head_map():
    # a GQA map that is neither contiguous nor even: KV head 2 serves three q
    # heads, KV head 0 two, KV head 1 one and KV head 3 none
    segs = [(0, 300, TEXT), (300, 49 * 14, VIDEO), (986, 77, TEXT), (1063, 49 * 9, VIDEO)]
    heads = [synth.vs(20, 40, "boundary_2d"), synth.block(5), synth.grid(1, 16, 64, layout="modality_grouped"),
             synth.vs(15, 60), synth.ashape(32, 200), synth.vs(10, 30, "q_segment")]
    spec = synth.small_spec("kv-map", 1504, 6, 4, 128, heads, seed=43, segs=segs, period=49, period_amp=3.0)
    full_check(spec, kv_head_of=[2, 0, 2, 1, 0, 2])


@pytest.mark.parametrize("scale", [0.03, 0.25])
def test_custom_softmax_scale(scale):
    # a scale given in the descriptor (flatter and sharper than 1/sqrt(d)):
    # estimation scores, index sets, attention and LSE all use it
    segs = [(0, 150, TEXT), (150, 49 * 12, VIDEO), (738, 90, TEXT)]
    heads = [synth.vs(20, 40), synth.vs(15, 30, "q_boundary"), synth.block(5),
             synth.grid(1, 16, 64, layout="modality_grouped"), synth.ashape(16, 100), synth.vs(10, 20, "boundary_2d")]
    spec = synth.small_spec("scale", 828, 6, 2, 128, heads, seed=49, segs=segs, period=49, period_amp=3.0,
                            rope_base=1e4, strong_cols=16)
    full_check(spec, scale=scale)


def test_saturated_budgets_select_every_causal_pair():
    # budgets at or above the candidate counts (clamped, not errors): vertical
    # and slash sets of L on every layout, more blocks than there are, a grid
    # of stride 16 with all 16 phases (every key a line key) and a window of L.
    # Every head then keeps every causal pair and equals dense attention.
    L = 1500
    segs = [(0, 300, TEXT), (300, 49 * 20, VIDEO), (1280, 220, TEXT)]
    heads = [synth.vs(L, L), synth.vs(L, L, "q_boundary"), synth.vs(L, L, "boundary_2d"), synth.vs(L, L, "q_segment"),
             synth.block(L // 64 + 5), synth.grid(16, 16, 16), synth.grid(16, 16, 16, layout="modality_grouped"),
             synth.ashape(0, L)]
    spec = synth.small_spec("saturated", L, 8, 2, 64, heads, seed=53, segs=segs, period=49, period_amp=3.0)
    lay = full_check(spec, rows_per_head=300)
    for h in range(spec.Hq):
        assert int(lay.view("tile_pairs", h).sum().item()) == L * (L + 1) // 2, f"head {h}"


def test_maximum_head_count():
    # B*Hq at its limit (4096 q heads over 512 KV heads) on a short ragged
    # layer, every pattern and layout in turn: host tables, launch grids and the
    # head field of the work items at their largest
    kinds = [synth.vs(5, 9), synth.vs(4, 8, "q_boundary"), synth.vs(3, 7, "boundary_2d"),
             synth.vs(4, 6, "q_segment"), synth.block(2), synth.grid(1, 16, 32),
             synth.grid(1, 16, 32, layout="modality_grouped"), synth.ashape(8, 40), synth.parallel(10, 30, 20)]
    heads = [kinds[h % len(kinds)] for h in range(4096)]
    segs = [(0, 70, TEXT), (70, 98, VIDEO), (168, 29, TEXT)]
    spec = synth.small_spec("max-heads", 197, 4096, 512, 64, heads, seed=61, segs=segs, period=49, period_amp=3.0)
    from parity_util import check_attention, check_head_indices, check_tile_pairs, f64
    import oracle.mmsa_oracle as O
    L, q, k, v, o, lse = run_gpu(spec)
    assert torch.isfinite(o.float()).all().item()
    causal = spec.L * (spec.L + 1) // 2   # every head's plan: selected pairs bounded by the causal count
    for h in range(spec.Hq):
        assert 0 <= int(L.view("tile_pairs", h).sum().item()) <= causal
    gmap = O.kv_head_map(spec.Hq, spec.Hkv)
    scale = 1 / np.sqrt(spec.d)
    rows = np.arange(0, spec.L, 7)
    for h in list(range(9)) + list(range(spec.Hq - 9, spec.Hq)):   # every kind, and the largest head indices
        qn, kn, vn = f64(q[0, h]), f64(k[0, gmap[h]]), f64(v[0, gmap[h]])
        hi = check_head_indices(L, h, spec.heads[h], qn, kn, spec.segs, scale)
        check_attention(hi, qn, kn, vn, f64(o[0, h]), lse[0, h].cpu().numpy().astype(np.float64), scale, rows,
                        name=f"head {h}")
        check_tile_pairs(L, h, hi)


def test_grid_at_its_parameter_limits():
    # strides up to the largest searched (1024), all 16 phases, the widest and
    # the narrowest clip, plain and modality-grouped, with a sink and window
    segs = [(0, 1000, TEXT), (1000, 700 * 26, VIDEO), (19200, 800, TEXT)]
    heads = [synth.grid(16, 512, 1024, clip=64), synth.grid(16, 512, 1024, clip=64, layout="modality_grouped"),
             synth.grid(4, 1000, 1024, clip=1, layout="modality_grouped"),
             synth.grid(16, 16, 1024, clip=64, sink=64, window=700)]
    spec = synth.small_spec("grid-limits", 20000, 4, 1, 128, heads, seed=67, segs=segs, period=700, period_amp=3.0)
    rng = np.random.default_rng(67)
    full_check(spec, rows_per_head=200, pair_tiles=sorted({0, 312} | set(int(t) for t in rng.integers(0, 313, 40))))


def test_parallel_encoding_ragged():
    # sink, context and question blocks off the 64-token tiles, a partial last
    # context block, a head with no sink or question, and 5-token blocks
    heads = [synth.parallel(300, 517, 129), synth.parallel(0, 64, 0), synth.parallel(236, 392, 64),
             synth.parallel(37, 5, 100)]
    full_check(synth.small_spec("parallel", 3017, 4, 2, 128, heads, seed=21))


@pytest.mark.parametrize("L", [1, 63, 65, 130])
def test_parallel_encoding_edges(L):
    # sink or question covering the whole layer, and one block per token
    heads = [synth.parallel(40, 30, 20), synth.parallel(L + 5, 3, 0), synth.parallel(0, 1, 0),
             synth.parallel(10, 7, L + 9)]
    full_check(synth.small_spec("parallel-edge", L, 4, 4, 64, heads, seed=L + 100))


def test_parallel_encoding_mixed_with_estimated_heads():
    heads = [synth.parallel(128, 196, 64), synth.vs(30, 60), synth.ashape(16, 100), synth.block(4)]
    full_check(synth.small_spec("parallel-mixed", 1500, 4, 1, 128, heads, seed=23))


def test_parallel_encoding_video_layer_shortened():
    # the 101K parallel-encoding workload's structure at 3K tokens
    full_check(synth.config(6, L=3000), rows_per_head=300)


def test_sparse_prefill_can_be_repeated_on_one_plan():
    # the attention call resets its own work queue: a second call on the same
    # plan writes the same output bits into a fresh buffer
    spec = synth.config(1)
    L, q, k, v, o, lse = run_gpu(spec)
    o2 = torch.full_like(o, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    L.sparse_prefill(q, k, v, o2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


def test_block_topk_breaks_exact_ties_to_the_lower_block():
    # key blocks 3, 5, 8, 9, 12 are copies of block 1, so their pooled logits
    # tie exactly with block 1's in every row: the selection must keep the
    # lower block indices among equal logits
    import math
    import oracle.mmsa_oracle as O
    from parity_util import check_attention, check_head_indices, f64
    spec = synth.small_spec("ties", 64 * 16, 2, 1, 128, [synth.block(4), synth.block(7)], seed=41)
    lay = synth.make_layer(spec, "cuda")
    q, k, v = lay["q"], lay["k"].clone(), lay["v"]
    for c in (3, 5, 8, 9, 12):
        k[0, 0, 64 * c:64 * c + 64] = k[0, 0, 64:128]
    L, q, k, v, o, lse = run_gpu(spec, q=q, k=k, v=v)
    scale = 1.0 / math.sqrt(spec.d)
    qn, kn, vn, on = f64(q[0]), f64(k[0]), f64(v[0]), f64(o[0])
    ln = lse[0].cpu().numpy().astype(np.float64)
    for h in range(spec.Hq):
        z = L.view("block_scores", h).cpu().numpy().reshape(16, 16)
        assert (z[12:, [1, 3, 5, 8, 9, 12]] == z[12:, [1]]).all()   # the ties are exact
        hi = check_head_indices(L, h, spec.heads[h], qn[h], kn[0], spec.segs, scale)
        check_attention(hi, qn[h], kn[0], vn[0], on[h], ln[h], scale, np.arange(spec.L), name=f"ties head {h}")


def test_vertical_topk_breaks_exact_ties_to_the_lower_key():
    # key rows 300..420 are copies of row 100, made the strongest key of the
    # estimation rows: their vertical scores tie exactly.  Head 0 keeps 40 of
    # the 122 tied keys (the threshold inside the group: the lowest positions
    # are kept), head 1 keeps 150 (the whole group and the next largest)
    import math
    from parity_util import check_attention, check_head_indices, f64
    L_ = 64 * 20
    spec = synth.small_spec("vties", L_, 2, 1, 128, [synth.vs(40, 64), synth.vs(150, 64)], seed=43)
    lay = synth.make_layer(spec, "cuda")
    q, k, v = lay["q"], lay["k"].clone(), lay["v"]
    rows = q[0, :, L_ - 64:].float().sum(dim=(0, 1))
    k[0, 0, 100] = (4.0 * rows / rows.norm() * math.sqrt(spec.d)).to(torch.bfloat16)
    k[0, 0, 300:421] = k[0, 0, 100]
    L, q, k, v, o, lse = run_gpu(spec, q=q, k=k, v=v)
    scale = 1.0 / math.sqrt(spec.d)
    qn, kn, vn, on = f64(q[0]), f64(k[0]), f64(v[0]), f64(o[0])
    ln = lse[0].cpu().numpy().astype(np.float64)
    tied = [100] + list(range(300, 421))
    for h in range(spec.Hq):
        vsc = L.view("v_scores", h, 0).cpu().numpy()
        assert (vsc[tied] == vsc[100]).all()                    # the ties are exact
        assert (vsc[tied[0]] >= np.delete(vsc, tied)).all()     # and they are the largest scores
        hi = check_head_indices(L, h, spec.heads[h], qn[h], kn[0], spec.segs, scale)
        V = hi.vs["all"][0]
        kv = spec.heads[h]["k_vertical"]
        if kv <= len(tied):   # the threshold inside the tied group: its lowest positions
            assert list(V) == tied[:kv], f"head {h}: {list(V)[:8]}"
        else:                 # the whole group, then the next largest scores
            assert len(V) == kv and set(tied) <= set(V.tolist()), f"head {h}"
        check_attention(hi, qn[h], kn[0], vn[0], on[h], ln[h], scale, np.arange(spec.L), name=f"vties head {h}")


def test_empty_layer_is_noop():
    spec = synth.small_spec("empty", 0, 2, 1, 128, [synth.vs(3, 5), synth.ashape(4, 8)], seed=0)
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 1, 0, 128), dtype=torch.bfloat16, device="cuda")
    L, *_ = run_gpu(spec, q=q, k=k, v=k.clone())


def test_strided_inputs_and_batch():
    # B = 2, heads interleaved in memory ([B, L, H, d] storage), GQA 4:1
    spec = synth.small_spec("strided", 300, 4, 1, 128, [synth.vs(10, 20), synth.block(3), synth.ashape(8, 40),
                                                        synth.grid(1, 16, 64)], seed=6)
    lay = synth.make_layer(spec, "cuda")
    from dynamic_sparse_attention_head_amd import mmsa
    import oracle.mmsa_oracle as O
    from parity_util import check_head_indices, check_attention, f64
    qs = torch.stack([lay["q"][0], lay["q"][0].flip(1)]).transpose(1, 2).contiguous().transpose(1, 2)
    ks = torch.stack([lay["k"][0], lay["k"][0].flip(1)]).transpose(1, 2).contiguous().transpose(1, 2)
    vs_ = torch.stack([lay["v"][0], lay["v"][0].flip(1)]).transpose(1, 2).contiguous().transpose(1, 2)
    assert not qs.is_contiguous()
    Lh = mmsa.Layer(qs, ks, vs_, spec.heads)
    o = torch.full((2, 4, 300, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    Lh.forward(qs, ks, vs_, o)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(4):
            qn, kn, vn = f64(qs[b, h]), f64(ks[b, 0]), f64(vs_[b, 0])
            hi = check_head_indices(Lh, b * 4 + h, spec.heads[h], qn, kn, None, 1 / np.sqrt(128))
            check_attention(hi, qn, kn, vn, f64(o[b, h]), None, 1 / np.sqrt(128), np.arange(300),
                            name=f"b{b} h{h}")


def test_batch_of_two_with_segments_and_every_layout():
    # B = 2 with modality segments: two independent layers (different seeds)
    # in one call, every pattern and layout, each batch element with its own
    # estimates, plans, LSE and exact per-tile pair counts
    from dataclasses import replace
    from parity_util import check_attention, check_head_indices, check_tile_pairs, f64
    import oracle.mmsa_oracle as O
    segs = [(0, 200, TEXT), (200, 49 * 10, VIDEO), (690, 60, TEXT), (750, 49 * 8, VIDEO)]
    heads = [synth.vs(20, 40, "q_boundary"), synth.vs(15, 50, "boundary_2d"), synth.vs(10, 30, "q_segment"),
             synth.grid(1, 16, 64, layout="modality_grouped"), synth.grid(1, 16, 64, sink=20, window=100),
             synth.block(4), synth.parallel(100, 98, 50), synth.ashape(16, 128)]
    spec = synth.small_spec("batch-segs", 1142, 8, 2, 128, heads, seed=47, segs=segs, period=49, period_amp=3.0)
    lays = [synth.make_layer(spec, "cuda"), synth.make_layer(replace(spec, seed=48), "cuda")]
    q, k, v = (torch.cat([lay[n] for lay in lays]).contiguous() for n in ("q", "k", "v"))
    Lh = mmsa.Layer(q, k, v, spec.heads, segs=spec.segs)
    o = torch.full((2, spec.Hq, spec.L, spec.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((2, spec.Hq, spec.L), float("nan"), dtype=torch.float32, device="cuda")
    Lh.forward(q, k, v, o, lse)
    torch.cuda.synchronize()
    gmap = O.kv_head_map(spec.Hq, spec.Hkv)
    scale = 1 / np.sqrt(spec.d)
    for b in range(2):
        for h in range(spec.Hq):
            qn, kn, vn = f64(q[b, h]), f64(k[b, gmap[h]]), f64(v[b, gmap[h]])
            hi = check_head_indices(Lh, b * spec.Hq + h, spec.heads[h], qn, kn, spec.segs, scale)
            check_attention(hi, qn, kn, vn, f64(o[b, h]), lse[b, h].cpu().numpy().astype(np.float64), scale,
                            np.arange(spec.L), name=f"b{b} h{h}")
            check_tile_pairs(Lh, b * spec.Hq + h, hi)
