"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/mmsa.h declares, and rejects invalid descriptors,
pointers and workspaces with the documented status before anything touches
the device (an attempted HIP call on a host without a GPU would come back as
MMSA_HIP_ERROR instead)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

from dynamic_sparse_attention_head_amd import mmsa, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmsa.h")

OK, INVALID, UNSUPPORTED, TOO_SMALL, HIP_ERROR = range(5)


def header_text():
    with open(HEADER) as f:
        return f.read()


def declared_functions():
    """Names of the functions include/mmsa.h declares (prototypes ending in ';')."""
    txt = re.sub(r"/\*.*?\*/", "", header_text(), flags=re.S)
    txt = re.sub(r"//[^\n]*", "", txt)
    names = set()
    for m in re.finditer(r"\b(mmsa_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", txt):
        names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    try:
        return mmsa.lib()
    except RuntimeError as e:  # pragma: no cover
        pytest.skip(str(e))


def test_header_declares_the_five_path_calls():
    names = declared_functions()
    for n in ("mmsa_estimate_vs", "mmsa_estimate_blocks", "mmsa_permute", "mmsa_sparse_prefill",
              "mmsa_unpermute", "mmsa_workspace_bytes", "mmsa_status_string", "mmsa_last_error",
              "mmsa_abi_version"):
        assert n in names, n


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert names
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, f"not exported: {missing}"
    assert set(mmsa._SYMBOLS) <= set(names)


def test_abi_version_matches_header(L):
    m = re.search(r"#define\s+MMSA_ABI_VERSION\s+(\d+)", header_text())
    assert m and L.mmsa_abi_version() == int(m.group(1))


def test_status_strings(L):
    L.mmsa_status_string.restype = ctypes.c_char_p
    want = {OK: "ok", INVALID: "invalid argument", UNSUPPORTED: "unsupported", TOO_SMALL: "workspace too small",
            HIP_ERROR: "HIP error", 99: "unknown status"}
    for s, txt in want.items():
        assert L.mmsa_status_string(s).decode() == txt


def host_layer(heads, Lq=4096, Hq=None, Hkv=1, d=128, B=1, segs=None, **kw):
    Hq = len(heads) if Hq is None else Hq
    return mmsa.Layer(None, None, None, heads, segs=segs, shape=(B, Hq, Hkv, Lq, d), device="cpu", **kw)


def status_of(layer):
    n = mmsa.lib().mmsa_workspace_bytes(ctypes.byref(layer.desc))
    if n:
        return OK
    return -1


def ws_status(layer):
    """Status of mmsa_workspace_view (host only), which validates the descriptor."""
    off, cnt = ctypes.c_int64(), ctypes.c_int64()
    return mmsa.lib().mmsa_workspace_view(ctypes.byref(layer.desc), 9, 0, 0, ctypes.byref(off), ctypes.byref(cnt))


def last_error():
    return mmsa.lib().mmsa_last_error().decode()


@pytest.mark.parametrize("mutate,code,needle", [
    (lambda D: setattr(D, "d", 96), UNSUPPORTED, "head dimension"),
    (lambda D: setattr(D, "L", -1), INVALID, "negative shape"),
    (lambda D: setattr(D, "flags", 2), INVALID, "flags"),
    (lambda D: setattr(D, "L", 1 << 22), UNSUPPORTED, "2^22"),
    (lambda D: setattr(D, "Hkv", 3), INVALID, "multiple"),
    (lambda D: setattr(D, "scale", float("nan")), INVALID, "scale"),
    (lambda D: setattr(D, "scale", -1.0), INVALID, "scale"),
    (lambda D: D.q_strides.__setitem__(2, 100), INVALID, "strides"),
    (lambda D: D.k_strides.__setitem__(2, 64), INVALID, "strides"),
    (lambda D: D.k_strides.__setitem__(2, 1 << 19), UNSUPPORTED, "2 GiB"),
    (lambda D: D.v_strides.__setitem__(2, 1 << 19), UNSUPPORTED, "2 GiB"),
    (lambda D: setattr(D, "heads", None), INVALID, "heads is NULL"),
])
def test_descriptor_validation(L, mutate, code, needle):
    lay = host_layer([synth.vs(10, 20), synth.ashape(4, 64)], Hkv=1)
    assert ws_status(lay) == OK
    mutate(lay.desc)
    assert ws_status(lay) == code
    assert needle in last_error()
    assert L.mmsa_workspace_bytes(ctypes.byref(lay.desc)) == 0


@pytest.mark.parametrize("head,needle", [
    (dict(pattern="ashape", layout="q_boundary", sink=4, window=64), "valid combination"),
    (dict(pattern="block", layout="boundary_2d", k_blocks=4), "valid combination"),
    (dict(pattern="grid", layout="q_boundary"), "valid combination"),
    (dict(pattern="ashape", sink=-1, window=64), "A-shape"),
    (dict(pattern="ashape", sink=0, window=0), "A-shape"),
    (dict(pattern="vs", k_vertical=-1, k_slash=3), "budget"),
    (dict(pattern="block", k_blocks=-2), "block budget"),
    (dict(pattern="grid", grid_phases=0), "grid needs"),
    (dict(pattern="grid", stride_lo=8, stride_hi=64), "grid needs"),
    (dict(pattern="grid", stride_lo=64, stride_hi=2048), "grid needs"),
    (dict(pattern="grid", stride_lo=200, stride_hi=100), "grid needs"),
    (dict(pattern="parallel", layout="q_boundary", sink=4, window=64), "valid combination"),
    (dict(pattern="block", layout="q_segment", k_blocks=4), "valid combination"),
    (dict(pattern="grid", layout="q_segment"), "valid combination"),
    (dict(pattern="parallel", sink=-1, window=64), "parallel encoding"),
    (dict(pattern="parallel", sink=64, window=0), "parallel encoding"),
    (dict(pattern="parallel", sink=64, window=64, question=-3), "parallel encoding"),
])
def test_head_validation(L, head, needle):
    lay = host_layer([head], Hkv=1)
    assert ws_status(lay) == INVALID
    assert needle in last_error()


@pytest.mark.parametrize("segs", [
    [(0, 100, 0), (100, 100, 1)],                 # does not reach L
    [(0, 3000, 0), (2000, 2096, 1)],              # overlap
    [(0, 4096, 2)],                               # unknown modality
    [(10, 4086, 0)],                              # does not start at 0
])
def test_segment_validation(L, segs):
    lay = host_layer([synth.vs(10, 20, layout="q_boundary")], segs=segs)
    assert ws_status(lay) == INVALID


def test_segment_parts_span_every_segment(L):
    """A per-segment head has one index set per segment (more than the four
    parts other layouts use): each covers the causal keys up to its segment's
    end with the last min(64, len) rows, and the part after the last is rejected."""
    segs = [(0, 700, 0), (700, 30, 1), (730, 900, 0), (1630, 64, 1), (1694, 1200, 0), (2894, 1202, 1)]
    lay = host_layer([synth.vs(40, 100, layout="q_segment")], segs=segs)
    n, spans = lay.workspace_bytes(), []
    for part, (s0, ln, _) in enumerate(segs):
        m = lay.meta(0, part)
        assert m[:4] == [0, s0 + ln, 0, s0 + ln]
        assert m[4:8] == [min(40, s0 + ln), min(100, s0 + ln), 0, min(64, ln)]
        off, cnt = lay.view_offset("v_index", 0, part)
        assert cnt == min(40, s0 + ln) and off % 4 == 0 and off + 4 * cnt <= n
        spans.append((off, off + 4 * cnt))
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))    # disjoint index sets
    with pytest.raises(mmsa.MMSAError):
        lay.meta(0, len(segs))
    with pytest.raises(mmsa.MMSAError):
        lay.view_offset("v_index", 0, len(segs))


def test_kv_head_map_validation(L):
    lay = host_layer([synth.vs(1, 2)] * 3, Hkv=2, kv_head_of=[0, 1, 2])
    assert ws_status(lay) == INVALID and "kv_head_of" in last_error()
    lay = host_layer([synth.vs(1, 2)] * 3, Hkv=2, kv_head_of=[0, 1, 1])
    assert ws_status(lay) == OK


def test_workspace_sizes_and_views(L):
    small = host_layer([synth.vs(10, 20), synth.block(4), synth.ashape(4, 64)], Lq=1000, Hkv=1)
    big = host_layer([synth.vs(10, 20), synth.block(4), synth.ashape(4, 64)], Lq=8000, Hkv=1)
    n_small, n_big = small.workspace_bytes(), big.workspace_bytes()
    assert 0 < n_small < n_big
    for lay, n in ((small, n_small), (big, n_big)):
        nT = -(-lay.L // 64)
        for h in range(3):
            off, cnt = lay.view_offset("tile_pairs", h)
            assert cnt == nT and off % 8 == 0 and off + 8 * cnt <= n
            off, cnt = lay.view_offset("tile_info", h)
            assert cnt == 4 * nT and off + 4 * cnt <= n
        off, cnt = lay.view_offset("v_index", 0)
        assert cnt == 10 and off + 4 * cnt <= n
        off, cnt = lay.view_offset("block_index", 1)
        assert cnt == nT * 4 and off + 4 * cnt <= n
        assert lay.view_offset("block_index", 0)[1] == 0      # not a block head
        assert lay.view_offset("v_scores", 2)[1] == 0         # A-shape has no scores
    with pytest.raises(mmsa.MMSAError):
        small.view_offset("v_scores", 3)                      # head out of range


def test_materialize_flag_only_grows_workspace_of_permuted_layers(L):
    segs = [(0, 500, 0), (500, 1500, 1), (2000, 96, 0)]
    permuted = [synth.vs(10, 20, layout="boundary_2d"), synth.vs(10, 20, layout="q_boundary"),
                synth.grid(1, 16, 100, layout="modality_grouped")]
    plain = [synth.vs(10, 20), synth.block(4), synth.ashape(4, 64)]
    for heads, grows in ((permuted, True), (plain, False)):
        a = host_layer(heads, Lq=2096, Hkv=1, segs=segs)
        b = host_layer(heads, Lq=2096, Hkv=1, segs=segs, materialize=True)
        assert ws_status(b) == OK
        na, nb = a.workspace_bytes(), b.workspace_bytes()
        assert (nb > na) if grows else (nb == na), (na, nb)


def _call(name, lay, ws, nbytes, ptr=16 * 1024):
    lib = mmsa.lib()
    D = ctypes.byref(lay.desc)
    s = None
    if name == "estimate_vs":
        return lib.mmsa_estimate_vs(D, ptr, ptr, ws, nbytes, s)
    if name == "estimate_blocks":
        return lib.mmsa_estimate_blocks(D, ptr, ptr, ws, nbytes, s)
    if name == "permute":
        return lib.mmsa_permute(D, ptr, ptr, ptr, ws, nbytes, s)
    if name == "sparse_prefill":
        return lib.mmsa_sparse_prefill(D, ptr, ptr, ptr, ws, nbytes, ptr, None, s)
    return lib.mmsa_unpermute(D, ws, nbytes, ptr, s)


CALLS = ["estimate_vs", "estimate_blocks", "permute", "sparse_prefill", "unpermute"]


@pytest.mark.parametrize("name", CALLS)
def test_workspace_errors_before_any_launch(L, name):
    lay = host_layer([synth.vs(10, 20), synth.block(4)], Lq=1000, Hkv=1)
    n = lay.workspace_bytes()
    aligned = 1 << 20   # a host address: never dereferenced, the checks come first
    assert _call(name, lay, None, n) == INVALID and "workspace is NULL" in last_error()
    assert _call(name, lay, aligned + 16, n) == UNSUPPORTED and "256-byte" in last_error()
    assert _call(name, lay, aligned, n - 1) == TOO_SMALL and "needed" in last_error()


@pytest.mark.parametrize("name", CALLS)
def test_tensor_pointer_errors_before_any_launch(L, name):
    lay = host_layer([synth.vs(10, 20), synth.block(4)], Lq=1000, Hkv=1)
    n = lay.workspace_bytes()
    ws = 1 << 20
    assert _call(name, lay, ws, n, ptr=None) == INVALID and "NULL" in last_error()
    assert _call(name, lay, ws, n, ptr=(1 << 16) + 8) == UNSUPPORTED and "aligned" in last_error()


@pytest.mark.parametrize("shape", [(0, 2, 1, 100, 64), (1, 2, 1, 0, 64), (1, 0, 1, 100, 128)])
def test_empty_layers_are_noops(L, shape):
    B, Hq, Hkv, Lq, d = shape
    lay = mmsa.Layer(None, None, None, [synth.vs(1, 2)] * Hq, shape=shape, device="cpu")
    for name in CALLS:
        assert _call(name, lay, None, 0, ptr=None) == OK, name


def test_invalid_desc_pointer(L):
    off, cnt = ctypes.c_int64(), ctypes.c_int64()
    assert L.mmsa_workspace_view(None, 0, 0, 0, ctypes.byref(off), ctypes.byref(cnt)) == INVALID
    assert L.mmsa_workspace_bytes(None) == 0
    for name in ("mmsa_estimate_vs", "mmsa_estimate_blocks"):
        assert getattr(L, name)(None, None, None, None, 0, None) == INVALID
    assert L.mmsa_unpermute(None, None, 0, None, None) == INVALID


def test_product_path_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mmsa, "_lib", None)
    monkeypatch.setattr(mmsa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        mmsa.lib()
    lay = host_layer([synth.vs(1, 2)], Lq=100)
    with pytest.raises(RuntimeError, match="missing"):
        lay.workspace_bytes()
