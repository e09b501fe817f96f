"""mmsa_prefill_noalloc (the allocation-free form of the five calls, on the
library's static scratch) against the five calls on a caller workspace,
through the C ABI: the outputs must agree bit for bit.  Two calls in a row,
the second on a smaller layer, so whatever the first left in the scratch is
in place when the second runs."""
import ctypes

import pytest
import torch

from dynamic_sparse_attention_head_amd import mmsa, synth

pytestmark = pytest.mark.gpu


def _same_as_five_calls(spec):
    lay = synth.make_layer(spec, "cuda")
    q, k, v = lay["q"], lay["k"], lay["v"]
    L = mmsa.Layer(q, k, v, spec.heads, segs=spec.segs)
    assert L.workspace_bytes() <= mmsa.NOALLOC_SCRATCH_BYTES
    shape = (1, spec.Hq, spec.L, spec.d)
    o_ref = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_ref = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    L.forward(q, k, v, o_ref, lse_ref)
    o = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    L.forward_noalloc(q, k, v, o, lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all().item()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))


def test_noalloc_equals_the_five_calls_twice_the_second_smaller():
    # 32K tokens of the LLaMA-3-8B-shaped layer (vertical-slash, block and
    # A-shape heads; about 56 MiB of workspace), then a 4K mixed-modality
    # layer (grid, Q-boundary, 2D-boundary and plain vertical-slash heads)
    _same_as_five_calls(synth.config(2, L=32768))
    _same_as_five_calls(synth.config(5, L=4022))


def test_noalloc_refuses_a_layer_beyond_its_scratch():
    spec = synth.config(2, L=65536)
    L = mmsa.Layer(None, None, None, spec.heads, shape=(1, spec.Hq, spec.Hkv, spec.L, spec.d), device="cuda")
    assert L.workspace_bytes() > mmsa.NOALLOC_SCRATCH_BYTES
    p = 1 << 20    # never dereferenced: the size check comes before anything is enqueued
    st = mmsa.lib().mmsa_prefill_noalloc(ctypes.byref(L.desc), p, p, p, p, None, None)
    assert st == mmsa.WORKSPACE_TOO_SMALL
    assert "static scratch" in mmsa.lib().mmsa_last_error().decode()
