"""ctypes binding of libmmsa (include/mmsa.h).

Argument marshalling only: every step of the sparse prefill runs in the HIP
library.  PyTorch supplies device memory (the workspace is a uint8 tensor) and
the current stream.  If the library has not been built, `lib()` raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MMSA_LIB names another build of the same library (the host-AddressSanitizer
# build the ABI tests run under); by default the in-tree libmmsa.so
LIB_PATH = os.environ.get("MMSA_LIB") or os.path.join(_HERE, "libmmsa.so")

TILE = 64
OK, INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP_ERROR = range(5)
PATTERNS = {"ashape": 0, "vs": 1, "block": 2, "grid": 3, "parallel": 4}
LAYOUTS = {"plain": 0, "q_boundary": 1, "boundary_2d": 2, "modality_grouped": 3, "q_segment": 4}
BUF = dict(v_scores=0, s_scores=1, v_index=2, s_index=3, nsel=4, grid=5, block_index=6, block_scores=7,
           row_order=8, tile_pairs=9, tile_info=10, est_stats=11, tile_bitmap=12, debug_flags=13)
BUF_DTYPE = dict(v_scores=torch.float32, s_scores=torch.float32, v_index=torch.int32, s_index=torch.int32,
                 nsel=torch.int32, grid=torch.int32, block_index=torch.int32, block_scores=torch.float32,
                 row_order=torch.int32, tile_pairs=torch.int64, tile_info=torch.int32, est_stats=torch.float32,
                 tile_bitmap=torch.int64, debug_flags=torch.int32)


class HeadCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "pattern", "layout", "sink", "window", "k_vertical", "k_slash", "k_blocks",
        "grid_phases", "stride_lo", "stride_hi", "grid_clip", "question")]


class Segment(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("len", ctypes.c_int64), ("modality", ctypes.c_int32),
                ("_pad", ctypes.c_int32)]


# mmsa_layer_desc.flags
FLAG_MATERIALIZE = 1        # explicit gathers and output scatter
FLAG_DEBUG = 2              # record non-finite inputs / outputs in the debug word
FLAG_KEYS_ASCENDING = 4     # attention walks key tiles lowest first
FLAG_KEYS_DESCENDING = 8    # attention walks key tiles highest (diagonal) first


class LayerDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("L", ctypes.c_int32),
                ("d", ctypes.c_int32), ("_pad0", ctypes.c_int32),
                ("q_strides", ctypes.c_int64 * 3), ("k_strides", ctypes.c_int64 * 3),
                ("v_strides", ctypes.c_int64 * 3), ("o_strides", ctypes.c_int64 * 3),
                ("scale", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("kv_head_of", ctypes.POINTER(ctypes.c_int32)), ("heads", ctypes.POINTER(HeadCfg)),
                ("segs", ctypes.POINTER(Segment)), ("n_segs", ctypes.c_int32), ("_pad1", ctypes.c_int32)]


class MMSAError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"mmsa status {status}: {msg}")
        self.status = status


_lib = None
_SYMBOLS = ("mmsa_workspace_bytes", "mmsa_workspace_view", "mmsa_index_meta", "mmsa_estimate_vs",
            "mmsa_estimate_blocks", "mmsa_permute", "mmsa_sparse_prefill", "mmsa_unpermute",
            "mmsa_prefill_noalloc", "mmsa_status_string", "mmsa_last_error", "mmsa_abi_version")
NOALLOC_SCRATCH_BYTES = 64 << 20   # MMSA_NOALLOC_SCRATCH_BYTES


def lib():
    """Load libmmsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m dynamic_sparse_attention_head_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(LayerDesc)
    vp, sz, i32, i64p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)
    L.mmsa_workspace_bytes.argtypes = [P]
    L.mmsa_workspace_bytes.restype = sz
    L.mmsa_workspace_view.argtypes = [P, i32, i32, i32, i64p, i64p]
    L.mmsa_workspace_view.restype = i32
    L.mmsa_index_meta.argtypes = [P, i32, i32, ctypes.POINTER(ctypes.c_int32)]
    L.mmsa_index_meta.restype = i32
    for fn in ("mmsa_estimate_vs", "mmsa_estimate_blocks"):
        getattr(L, fn).argtypes = [P, vp, vp, vp, sz, vp]
        getattr(L, fn).restype = i32
    L.mmsa_permute.argtypes = [P, vp, vp, vp, vp, sz, vp]
    L.mmsa_permute.restype = i32
    L.mmsa_sparse_prefill.argtypes = [P, vp, vp, vp, vp, sz, vp, vp, vp]
    L.mmsa_sparse_prefill.restype = i32
    L.mmsa_unpermute.argtypes = [P, vp, sz, vp, vp]
    L.mmsa_unpermute.restype = i32
    L.mmsa_prefill_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.mmsa_prefill_noalloc.restype = i32
    L.mmsa_status_string.argtypes = [i32]
    L.mmsa_status_string.restype = ctypes.c_char_p
    L.mmsa_last_error.argtypes = []
    L.mmsa_last_error.restype = ctypes.c_char_p
    L.mmsa_abi_version.argtypes = []
    L.mmsa_abi_version.restype = i32
    _lib = L
    return L


def _check(status):
    if status != OK:
        raise MMSAError(status, lib().mmsa_last_error().decode())


def head_cfg(d):
    """dict (the generator's / oracle's head description) -> HeadCfg."""
    c = HeadCfg()
    c.pattern = PATTERNS[d["pattern"]]
    c.layout = LAYOUTS[d.get("layout", "plain")]
    c.sink = int(d.get("sink", 0))
    c.window = int(d.get("window", 0 if d["pattern"] == "grid" else 1))
    c.k_vertical = int(d.get("k_vertical", 0))
    c.k_slash = int(d.get("k_slash", 0))
    c.k_blocks = int(d.get("k_blocks", 0))
    c.grid_phases = int(d.get("grid_phases", 1))
    c.stride_lo = int(d.get("stride_lo", 64))
    c.stride_hi = int(d.get("stride_hi", 512))
    c.grid_clip = int(d.get("grid_clip", 8))
    c.question = int(d.get("question", 0))
    return c


def _strides(t, B, H, L, d):
    if t is None:
        return (H * L * d, L * d, d)
    s = t.stride()
    assert s[3] == 1, "last dimension must be contiguous"
    return (s[0], s[1], s[2])


class Layer:
    """One layer's descriptor plus its workspace.

    q: [B, Hq, L, d] bf16, k / v: [B, Hkv, L, d] bf16 (any strides with the
    last dimension contiguous).  heads: list of dicts (pattern, layout and
    budgets per q head); segs: list of (start, len, modality) or None.
    materialize: copy permuted Q / grouped K,V into the workspace and scatter
    O back in unpermute (MMSA_FLAG_MATERIALIZE) instead of index-based loads
    and stores inside the attention call.  flags: further MMSA_FLAG_* bits
    (FLAG_DEBUG, FLAG_KEYS_ASCENDING, FLAG_KEYS_DESCENDING)."""

    def __init__(self, q, k, v, heads, segs=None, scale=None, kv_head_of=None, o_strides=None,
                 shape=None, device=None, materialize=False, flags=0):
        if q is not None:
            B, Hq, L, d = q.shape
            Hkv = k.shape[1]
            device = q.device
        else:
            B, Hq, Hkv, L, d = shape
        self.B, self.Hq, self.Hkv, self.L, self.d = B, Hq, Hkv, L, d
        self.device = device
        self.heads = list(heads)
        self._cfg = (HeadCfg * max(1, Hq))(*[head_cfg(h) for h in self.heads])
        self._segs = None
        n_segs = 0
        if segs:
            self._segs = (Segment * len(segs))(*[Segment(int(s), int(n), int(m), 0) for s, n, m in segs])
            n_segs = len(segs)
        self._kvmap = None
        if kv_head_of is not None:
            self._kvmap = (ctypes.c_int32 * Hq)(*[int(g) for g in kv_head_of])
        desc = LayerDesc()
        desc.B, desc.Hq, desc.Hkv, desc.L, desc.d = B, Hq, Hkv, L, d
        desc.q_strides[:] = _strides(q, B, Hq, L, d)
        desc.k_strides[:] = _strides(k, B, Hkv, L, d)
        desc.v_strides[:] = _strides(v, B, Hkv, L, d)
        desc.o_strides[:] = o_strides if o_strides is not None else (Hq * L * d, L * d, d)
        desc.scale = float(scale) if scale is not None else 0.0
        desc.flags = (FLAG_MATERIALIZE if materialize else 0) | int(flags)
        desc.kv_head_of = self._kvmap
        desc.heads = self._cfg
        desc.segs = self._segs
        desc.n_segs = n_segs
        self.desc = desc
        self.scale = float(scale) if scale is not None else 1.0 / math.sqrt(d)
        self.ws = None

    # ---- host-only queries ----
    def workspace_bytes(self):
        n = lib().mmsa_workspace_bytes(ctypes.byref(self.desc))
        if n == 0:
            raise MMSAError(INVALID_ARGUMENT, lib().mmsa_last_error().decode())
        return n

    def view_offset(self, buf, bh, part=0):
        off, cnt = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().mmsa_workspace_view(ctypes.byref(self.desc), BUF[buf], bh, part, ctypes.byref(off),
                                         ctypes.byref(cnt)))
        return off.value, cnt.value

    def meta(self, bh, part=0):
        out = (ctypes.c_int32 * 8)()
        _check(lib().mmsa_index_meta(ctypes.byref(self.desc), bh, part, out))
        return list(out)

    # ---- device ----
    def alloc_workspace(self):
        n = self.workspace_bytes()
        if self.ws is None or self.ws.numel() < n:
            self.ws = torch.empty(n + 256, dtype=torch.uint8, device=self.device)
        return self.ws

    def _ws_ptr(self):
        base = self.ws.data_ptr()
        return (base + 255) // 256 * 256

    def view(self, buf, bh, part=0):
        """torch view (on the device) of a workspace buffer; count 0 -> empty."""
        off, cnt = self.view_offset(buf, bh, part)
        dt = BUF_DTYPE[buf]
        if cnt == 0:
            return torch.empty(0, dtype=dt, device=self.device)
        start = self._ws_ptr() - self.ws.data_ptr() + off
        es = torch.tensor([], dtype=dt).element_size()
        return self.ws[start:start + cnt * es].view(dt)

    @staticmethod
    def _stream():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def _on_device(self, t):
        dev = torch.device(self.device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        return t.device == dev

    def _arg(self, t, name, heads, strides):
        """A tensor handed to the library as a raw pointer must be what the
        descriptor says it is: bf16 on the layer's device, [B, heads, L, d]
        with the descriptor's strides (the library reads it through those)."""
        shape = (self.B, heads, self.L, self.d)
        if t.dtype != torch.bfloat16 or not self._on_device(t) or tuple(t.shape) != shape:
            raise ValueError(f"{name}: expected bf16 {shape} on {self.device}, got {t.dtype} "
                             f"{tuple(t.shape)} on {t.device}")
        if t.numel() and (t.stride(3) != 1 or tuple(t.stride()[:3]) != tuple(strides)):
            raise ValueError(f"{name}: strides {tuple(t.stride())} differ from the descriptor's "
                             f"{tuple(strides)} (+1); build the Layer from tensors of this layout")
        return t.data_ptr()

    def _q(self, q):
        return self._arg(q, "q", self.Hq, self.desc.q_strides)

    def _k(self, k):
        return self._arg(k, "k", self.Hkv, self.desc.k_strides)

    def _v(self, v):
        return self._arg(v, "v", self.Hkv, self.desc.v_strides)

    def _o(self, o):
        return self._arg(o, "o", self.Hq, self.desc.o_strides)

    def _lse(self, lse):
        if lse is None:
            return None
        shape = (self.B, self.Hq, self.L)
        if (lse.dtype != torch.float32 or not self._on_device(lse) or tuple(lse.shape) != shape
                or not lse.is_contiguous()):
            raise ValueError(f"lse: expected contiguous float32 {shape} on {self.device}, got {lse.dtype} "
                             f"{tuple(lse.shape)} on {lse.device}")
        return lse.data_ptr()

    def estimate_vs(self, q, k):
        self.alloc_workspace()
        _check(lib().mmsa_estimate_vs(ctypes.byref(self.desc), self._q(q), self._k(k), self._ws_ptr(),
                                      self.workspace_bytes(), self._stream()))

    def estimate_blocks(self, q, k):
        self.alloc_workspace()
        _check(lib().mmsa_estimate_blocks(ctypes.byref(self.desc), self._q(q), self._k(k), self._ws_ptr(),
                                          self.workspace_bytes(), self._stream()))

    def permute(self, q, k, v):
        self.alloc_workspace()
        _check(lib().mmsa_permute(ctypes.byref(self.desc), self._q(q), self._k(k), self._v(v),
                                  self._ws_ptr(), self.workspace_bytes(), self._stream()))

    def sparse_prefill(self, q, k, v, o, lse=None):
        _check(lib().mmsa_sparse_prefill(ctypes.byref(self.desc), self._q(q), self._k(k), self._v(v),
                                         self._ws_ptr(), self.workspace_bytes(), self._o(o), self._lse(lse),
                                         self._stream()))

    def unpermute(self, o):
        _check(lib().mmsa_unpermute(ctypes.byref(self.desc), self._ws_ptr(), self.workspace_bytes(), self._o(o),
                                    self._stream()))

    def forward_noalloc(self, q, k, v, o, lse=None):
        """The whole path through mmsa_prefill_noalloc (the library's static
        scratch instead of this layer's workspace, which is left untouched)."""
        _check(lib().mmsa_prefill_noalloc(ctypes.byref(self.desc), self._q(q), self._k(k), self._v(v),
                                          self._o(o), self._lse(lse), self._stream()))
        return o

    def forward(self, q, k, v, o=None, lse=None):
        """All five calls in order; returns O [B, Hq, L, d] bf16."""
        if o is None:
            o = torch.empty((self.B, self.Hq, self.L, self.d), dtype=torch.bfloat16, device=self.device)
        self.estimate_vs(q, k)
        self.estimate_blocks(q, k)
        self.permute(q, k, v)
        self.sparse_prefill(q, k, v, o, lse)
        self.unpermute(o)
        return o
