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

from dynamic_sparse_attention_head_amd import synth
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
