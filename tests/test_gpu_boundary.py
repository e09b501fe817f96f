"""GPU checks of the boundary's options (include/mmsa.h): the debug word of
MMSA_FLAG_DEBUG, the forced key-tile walk orders, and tensors that are views
into larger allocations whose bytes past the layer are NaN.  Parity against the
CPU oracle uses the same bars as the other GPU tests."""
import numpy as np
import pytest
import torch

from dynamic_sparse_attention_head_amd import mmsa, synth
from parity_util import full_check, run_gpu

pytestmark = pytest.mark.gpu

TEXT, VIDEO = 0, 1


def debug_word(L):
    return int(L.view("debug_flags", 0).cpu().item())


def mixed_spec(L=1000, d=128, seed=51):
    heads = [synth.vs(40, 90), synth.block(5), synth.ashape(64, 256), synth.grid(1, 16, 64)]
    return synth.small_spec("dbg", L, 4, 2, d, heads, seed=seed, rope_base=1e4, strong_cols=16)


def test_debug_word_is_zero_on_finite_inputs_and_changes_no_output_bit():
    spec = mixed_spec()
    L0, q, k, v, o0, lse0 = run_gpu(spec)
    L1, _, _, _, o1, lse1 = run_gpu(spec, q=q, k=k, v=v, flags=mmsa.FLAG_DEBUG)
    assert debug_word(L1) == 0
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(lse0.view(torch.int32), lse1.view(torch.int32))


@pytest.mark.parametrize("which,value,bit", [("q", float("nan"), 1), ("k", float("inf"), 2), ("v", float("nan"), 4),
                                             ("v", float("-inf"), 4)])
def test_debug_word_records_a_non_finite_input(which, value, bit):
    # A-shape and parallel-encoding heads only: no estimation reads the bad value
    heads = [synth.ashape(16, 100), synth.parallel(64, 50, 30)]
    spec = synth.small_spec("dbg-nf", 700, 2, 1, 64, heads, seed=52)
    lay = synth.make_layer(spec, "cuda")
    t = {"q": lay["q"], "k": lay["k"], "v": lay["v"]}
    t[which] = t[which].clone()
    t[which][0, 0, 70, 5] = value      # row 70: every head's row 70 and its window see it
    L, *_ = run_gpu(spec, q=t["q"], k=t["k"], v=t["v"], flags=mmsa.FLAG_DEBUG)
    w = debug_word(L)
    assert w & 7 == bit, hex(w)
    assert w & 8, f"a non-finite output must set bit 3: {hex(w)}"


def nan_padded(t, extra_rows, bl_layout=False):
    """A copy of t [B, H, L, d] stored as a view at the front of a NaN-filled
    allocation with `extra_rows` more rows per head ([B, H, L + extra, d]), or
    with bl_layout as a [B, L + extra, H, d] allocation viewed as [B, H, L, d]."""
    B, H, Lq, d = t.shape
    if bl_layout:
        buf = torch.full((B, Lq + extra_rows, H, d), float("nan"), dtype=t.dtype, device=t.device)
        view = buf[:, :Lq].transpose(1, 2)
    else:
        buf = torch.full((B, H, Lq + extra_rows, d), float("nan"), dtype=t.dtype, device=t.device)
        view = buf[:, :, :Lq]
    view.copy_(t)
    return view


@pytest.mark.parametrize("bl_layout", [False, True])
@pytest.mark.parametrize("Lq", [65, 1000, 3017])
def test_ragged_layers_never_read_past_the_last_row(Lq, bl_layout):
    # the rows after the layer's last one are NaN in every head's slice: a
    # partial last key tile that read them would put NaN into the outputs
    heads = [synth.vs(20, 40), synth.block(3), synth.ashape(8, 100), synth.grid(1, 16, 64),
             synth.vs(10, 30, "boundary_2d"), synth.parallel(100, 64, 40)]
    segs = [(0, Lq // 3, TEXT), (Lq // 3, Lq - Lq // 3, VIDEO)]
    spec = synth.small_spec("nan-tail", Lq, 6, 2, 128, heads, seed=Lq, segs=segs, period=49)
    lay = synth.make_layer(spec, "cuda")
    q = nan_padded(lay["q"], 64, bl_layout)
    k = nan_padded(lay["k"], 64, bl_layout)
    v = nan_padded(lay["v"], 64, bl_layout)
    L = full_check(spec, q=q, k=k, v=v, flags=mmsa.FLAG_DEBUG, rows_per_head=None if Lq < 2000 else 300)
    assert debug_word(L) == 0


def order_specs():
    segs, Lb = synth.interleaved_segments(3, 4, 49, 77)
    return {
        "edge-65": synth.small_spec("edge", 65, 4, 4, 64, [synth.vs(3, 5), synth.block(2), synth.ashape(4, 16),
                                                           synth.grid(1, 16, 64)], seed=65),
        "edge-130": synth.small_spec("edge", 130, 4, 4, 64, [synth.vs(3, 5), synth.block(2), synth.ashape(4, 16),
                                                             synth.grid(1, 16, 64)], seed=130),
        "mixed": synth.small_spec("mixed", 1000, 8, 2, 128,
                                  [synth.vs(40, 90), synth.vs(7, 300), synth.block(5), synth.ashape(64, 256),
                                   synth.block(1000), synth.ashape(0, 1), synth.vs(0, 3), synth.block(1)],
                                  seed=11, rope_base=1e4, strong_cols=16),
        "boundary": synth.small_spec("boundary", Lb, 4, 1, 128,
                                     [synth.grid(2, 16, 200, layout="modality_grouped"), synth.vs(20, 40, "q_boundary"),
                                      synth.vs(25, 33, "boundary_2d"), synth.vs(15, 80, "plain")],
                                     seed=9, segs=segs, period=49, period_amp=3.0),
        "parallel": synth.small_spec("parallel", 3017, 4, 2, 128,
                                     [synth.parallel(300, 517, 129), synth.parallel(0, 64, 0),
                                      synth.parallel(236, 392, 64), synth.parallel(37, 5, 100)], seed=21),
        "parallel-edge": synth.small_spec("parallel-edge", 130, 4, 4, 64,
                                          [synth.parallel(40, 30, 20), synth.parallel(135, 3, 0),
                                           synth.parallel(0, 1, 0), synth.parallel(10, 7, 139)], seed=230),
    }


@pytest.mark.parametrize("name", list(order_specs()))
def test_both_key_walk_orders_match_the_oracle(name):
    spec = order_specs()[name]
    rows = None if spec.L <= 1000 else 300
    La = full_check(spec, flags=mmsa.FLAG_KEYS_ASCENDING, rows_per_head=rows)
    Ld = full_check(spec, flags=mmsa.FLAG_KEYS_DESCENDING, rows_per_head=rows)
    # the plans are the same bits; only the summation order differs
    for h in range(spec.Hq):
        for buf in ("tile_bitmap", "tile_pairs", "tile_info"):
            assert torch.equal(La.view(buf, h), Ld.view(buf, h)), (h, buf)


def test_layers_interleaved_on_one_stream_keep_their_own_tables():
    # The host tables are cached by descriptor contents and uploaded by every
    # call: two layers of different shape and patterns whose calls alternate
    # on one stream (each with its own workspace), and a third layer that
    # differs from the first only in one head's slash budget, must each produce the
    # output they produce alone, bit for bit.
    specs = [mixed_spec(L=1000, seed=61),
             synth.small_spec("other", 777, 2, 1, 64, [synth.vs(20, 40), synth.ashape(32, 128)], seed=62)]
    alone = []
    for sp in specs:
        L_, q, k, v, o, lse = run_gpu(sp)
        alone.append((q, k, v, o))
    heads3 = [dict(h) for h in specs[0].heads]
    heads3[0]["k_slash"] = 3          # few slashes: head 0 keeps far fewer tiles
    spec3 = synth.with_heads(specs[0], heads3)
    q0, k0, v0, _ = alone[0]
    _, _, _, _, o3_alone, _ = run_gpu(spec3, q=q0, k=k0, v=v0)
    lay = [mmsa.Layer(alone[i][0], alone[i][1], alone[i][2], specs[i].heads, segs=specs[i].segs) for i in range(2)]
    lay.append(mmsa.Layer(q0, k0, v0, spec3.heads, segs=spec3.segs))
    ins = [alone[0][:3], alone[1][:3], (q0, k0, v0)]
    outs = [torch.full_like(alone[0][3], float("nan")), torch.full_like(alone[1][3], float("nan")),
            torch.full_like(o3_alone, float("nan"))]
    for L_ in lay:
        L_.alloc_workspace()
    for _ in range(2):
        for call in ("estimate_vs", "estimate_blocks", "permute"):
            for i in (0, 1, 2):
                q, k, v = ins[i]
                if call == "permute":
                    lay[i].permute(q, k, v)
                else:
                    getattr(lay[i], call)(q, k)
        for i in (2, 0, 1):
            q, k, v = ins[i]
            lay[i].sparse_prefill(q, k, v, outs[i], None)
            lay[i].unpermute(outs[i])
    torch.cuda.synchronize()
    want = [alone[0][3], alone[1][3], o3_alone]
    for i in range(3):
        assert torch.equal(outs[i].view(torch.int16), want[i].view(torch.int16)), f"layer {i}"
    assert not torch.equal(outs[2].view(torch.int16), outs[0].view(torch.int16))   # the budget matters


def test_graph_capture_replays_match_eager():
    # The five calls, and the allocation-free call, captured into graphs.
    # Every replay gives the eager output bit for bit, with other layers run
    # eagerly in between (the allocation-free one through the same static
    # scratch) and the host layout cache cycled past its 16 entries, which
    # frees the captured layer's own copy of its tables.
    spec = mixed_spec()
    lay = synth.make_layer(spec, "cuda")
    q, k, v = lay["q"], lay["k"], lay["v"]
    L = mmsa.Layer(q, k, v, spec.heads, segs=spec.segs)
    shape = (1, spec.Hq, spec.L, spec.d)
    o_e = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    l_e = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
    L.forward(q, k, v, o_e, l_e)
    torch.cuda.synchronize()
    outs = {}
    graphs = {}
    for name in ("five", "noalloc"):
        o = torch.zeros_like(o_e)
        lse = torch.zeros_like(l_e)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            if name == "five":
                L.forward(q, k, v, o, lse)
            else:
                L.forward_noalloc(q, k, v, o, lse)
        outs[name], graphs[name] = (o, lse), g
    spec2 = synth.config(2, L=8192)
    lay2 = synth.make_layer(spec2, "cuda")
    L2 = mmsa.Layer(lay2["q"], lay2["k"], lay2["v"], spec2.heads)
    o2 = torch.zeros((1, spec2.Hq, spec2.L, spec2.d), dtype=torch.bfloat16, device="cuda")
    for r in range(3):
        for name in ("five", "noalloc"):
            o, lse = outs[name]
            o.zero_()
            lse.zero_()
            graphs[name].replay()
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), o_e.view(torch.int16)), f"{name} replay {r}: output"
            assert torch.equal(lse, l_e), f"{name} replay {r}: lse"
        L2.forward_noalloc(lay2["q"], lay2["k"], lay2["v"], o2)
        L2.forward(lay2["q"], lay2["k"], lay2["v"], o2)
        for i in range(20):   # 20 other layouts through the host-only size query
            mmsa.Layer(None, None, None, [synth.vs(1 + i + 20 * r, 2)], shape=(1, 1, 1, 4096, 64),
                       device="cuda").workspace_bytes()
        torch.cuda.synchronize()
