"""Seeded synthetic inputs for one prefill attention layer.

This module only builds inputs (Q, K, V, the per-head pattern table and the
modality segments).  It holds none of the method's arithmetic and is shared by
the tests, the smoke check and the benchmark; both the GPU library and the CPU
oracle consume what it returns.

The workloads stand in for the pages' settings (no model weights or datasets
are used): a 4K two-head layer; a LLaMA-3-8B-shaped layer at 128K tokens with
mixed vertical-slash / block / A-shape heads; a 256K block-sparse stress layer;
a Qwen2-7B-shaped video layer (512 text tokens + 1600 frames of 196 tokens);
and a 1M-token interleaved video/text layer.  Structure planted in the keys
(strong columns, clustered blocks, a period-196 component) is what the online
estimators are meant to find.

All randomness comes from torch generators seeded per (config seed, stream),
so a spec regenerates bit-identically on the same device type.  Values are
generated in float32 and rounded to bfloat16 (round to nearest even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

TEXT, VIDEO = 0, 1


@dataclass
class LayerSpec:
    name: str
    L: int
    Hq: int
    Hkv: int
    d: int
    seed: int
    heads: list                       # per q head: dict for oracle.HeadCfg / the C descriptor
    segs: list = None                 # [(start, len, modality)] or None (all text)
    rope_base: float = 0.0            # 0 -> no RoPE
    strong_cols: int = 0              # number of strong key positions (+3u)
    strong_shared: bool = True        # one u for all KV heads, else one per KV head
    strong_amp: float = 3.0
    cluster_blocks: int = 0           # number of 64-blocks sharing a mean vector
    cluster_norm: float = 4.0
    period: int = 0                   # video period (tokens per frame); 0 -> none
    period_amp: float = 2.0
    frame_amp: float = 0.5
    q_periodic: bool = True
    # planted attention targets with a scene cut: query rows [r0, cut) aim at
    # `targets` keys A and rows [cut, r1) at `targets` other keys B, both
    # drawn from [r0, (r0 + cut) // 2); cut == r1 means no cut
    targets: int = 0
    target_amp: float = 10.0
    target_rows: tuple = None         # (r0, cut, r1)
    meta: dict = field(default_factory=dict)


def _gen(seed, stream, device):
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream) * 7919) % (2 ** 63 - 1))
    return g


def _rope(x, base):
    """Rotate-half rotary embedding at positions 0..L-1, theta_k = base^(-2k/d)."""
    L, d = x.shape[-2], x.shape[-1]
    half = d // 2
    inv = base ** (-torch.arange(0, half, device=x.device, dtype=torch.float64) * 2.0 / d)
    ang = torch.arange(L, device=x.device, dtype=torch.float64)[:, None] * inv[None, :]
    cos = torch.cos(ang).to(torch.float32)
    sin = torch.sin(ang).to(torch.float32)
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


def _video_slots(spec, device):
    """(is_video mask, slot index in frame, frame index) per position, where
    slot and frame count video tokens only (video rank)."""
    L = spec.L
    isv = torch.zeros(L, dtype=torch.bool, device=device)
    for s, n, m in (spec.segs or []):
        if m == VIDEO:
            isv[s:s + n] = True
    vr = torch.cumsum(isv.to(torch.int64), 0) - 1
    slot = torch.remainder(vr, spec.period) if spec.period else vr
    frame = torch.div(vr, spec.period, rounding_mode='floor') if spec.period else vr
    return isv, slot, frame


def make_layer(spec: LayerSpec, device='cpu'):
    """Returns dict(q, k, v) bf16 tensors [1, H, L, d] plus the spec fields."""
    dev = torch.device(device)
    L, d = spec.L, spec.d
    q = torch.empty((1, spec.Hq, L, d), dtype=torch.bfloat16, device=dev)
    k = torch.empty((1, spec.Hkv, L, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty((1, spec.Hkv, L, d), dtype=torch.bfloat16, device=dev)
    # structure shared across heads
    strong_pos = None
    if spec.strong_cols:
        gp = _gen(spec.seed, 4, dev)
        strong_pos = torch.randperm(L, generator=gp, device=dev)[:spec.strong_cols]
    if spec.period:
        isv, slot, frame = _video_slots(spec, dev)
        n_frames = int(frame[isv].max().item()) + 1 if bool(isv.any()) else 0
        ang = 2 * math.pi * slot.to(torch.float64) / spec.period
        sin_t = torch.sin(ang).to(torch.float32)
        cos_t = torch.cos(ang).to(torch.float32)
    gs = _gen(spec.seed, 3, dev)
    u_shared = torch.randn(d, generator=gs, device=dev)
    u_shared = u_shared / u_shared.norm()
    group = spec.Hq // spec.Hkv
    for g in range(spec.Hkv):
        gk = _gen(spec.seed, 100 + g, dev)
        kg = torch.randn((L, d), generator=gk, device=dev)
        if spec.rope_base:
            kg = _rope(kg, spec.rope_base)
        if strong_pos is not None:
            if spec.strong_shared:
                u = u_shared
            else:
                u = torch.randn(d, generator=gk, device=dev)
                u = u / u.norm()
            kg[strong_pos] += spec.strong_amp * u
        if spec.cluster_blocks:
            nB = L // 64
            blocks = torch.randperm(nB, generator=gk, device=dev)[:spec.cluster_blocks]
            mu = torch.randn(d, generator=gk, device=dev)
            mu = spec.cluster_norm * mu / mu.norm()
            rows = (blocks[:, None] * 64 + torch.arange(64, device=dev)[None, :]).reshape(-1)
            kg[rows] += mu
        if spec.period:
            ab = torch.randn((d, 2), generator=gk, device=dev)
            qmat, _ = torch.linalg.qr(ab.cpu())
            a_vec, b_vec = qmat[:, 0].to(dev), qmat[:, 1].to(dev)
            pi = spec.period_amp * (sin_t[:, None] * a_vec[None, :] + cos_t[:, None] * b_vec[None, :])
            pi = pi * isv[:, None]
            delta = torch.randn((max(n_frames, 1), d), generator=gk, device=dev)
            delta = delta / delta.norm(dim=1, keepdim=True)
            fr = torch.clamp(frame, min=0)
            kg += pi + spec.frame_amp * delta[fr] * isv[:, None]
        if spec.targets:
            r0, cut, r1 = spec.target_rows
            gt = _gen(spec.seed, 400 + g, dev)
            span = max((r0 + cut) // 2 - r0, 2 * spec.targets)
            pos = r0 + torch.randperm(span, generator=gt, device=dev)[:2 * spec.targets]
            uab, _ = torch.linalg.qr(torch.randn((d, 2), generator=gt, device=dev).cpu())
            u_a, u_b = uab[:, 0].to(dev), uab[:, 1].to(dev)
            kg[pos[:spec.targets]] += spec.target_amp * u_a
            kg[pos[spec.targets:]] += spec.target_amp * u_b
        k[0, g] = kg.to(torch.bfloat16)
        del kg
        gv = _gen(spec.seed, 200 + g, dev)
        v[0, g] = torch.randn((L, d), generator=gv, device=dev).to(torch.bfloat16)
        for hh in range(group):
            h = g * group + hh
            gq = _gen(spec.seed, 300 + h, dev)
            qh = torch.randn((L, d), generator=gq, device=dev)
            if spec.rope_base:
                qh = _rope(qh, spec.rope_base)
            if spec.period and spec.q_periodic:
                qh += pi
            if spec.targets:
                qh[r0:cut] += spec.target_amp * u_a
                qh[cut:r1] += spec.target_amp * u_b
            q[0, h] = qh.to(torch.bfloat16)
            del qh
    return dict(q=q, k=k, v=v, spec=spec, heads=spec.heads, segs=spec.segs,
                scale=1.0 / math.sqrt(d))


# ---------------------------------------------------------------------------
# Head tables
# ---------------------------------------------------------------------------
def ashape(sink, window):
    return dict(pattern='ashape', layout='plain', sink=sink, window=window)


def vs(kv, ks, layout='plain'):
    return dict(pattern='vs', layout=layout, k_vertical=kv, k_slash=ks)


def block(kb):
    return dict(pattern='block', layout='plain', k_blocks=kb)


def grid(w=1, lo=64, hi=512, clip=8, layout='plain', sink=0, window=0):
    """Grid head; sink / window > 0 add a sink and a local window to the rows
    that are not on a line."""
    return dict(pattern='grid', layout=layout, grid_phases=w, stride_lo=lo, stride_hi=hi, grid_clip=clip,
                sink=sink, window=window)


def parallel(sink, block, question):
    """Parallel-encoding head: sink block, context blocks and question block
    lengths in tokens."""
    return dict(pattern='parallel', layout='plain', sink=sink, window=block, question=question)


def interleaved_segments(n_chunks, frames, per_frame, text_len, lead_text=0):
    """[T0?][V0][T][V1]...[T][V_{n-1}] with `text_len` text between chunks."""
    segs, pos = [], 0
    if lead_text:
        segs.append((0, lead_text, TEXT))
        pos = lead_text
    for c in range(n_chunks):
        if c > 0 and text_len:
            segs.append((pos, text_len, TEXT))
            pos += text_len
        n = frames * per_frame
        segs.append((pos, n, VIDEO))
        pos += n
    return segs, pos


def scene_cut(frames=40, per=196, text=512, cut=True, targets=64, amp=10.0, heads=None, seed=7, d=128):
    """A text prompt then one video segment whose queries aim at one set of
    planted keys, except its last 64 queries, which aim at another (a scene
    cut at the segment end); with cut=False every video query aims at the
    first set.  Default heads: plain, Q-boundary and 2D-boundary
    vertical-slash (256 / 512)."""
    L = text + frames * per
    segs = [(0, text, TEXT), (text, frames * per, VIDEO)]
    heads = heads or [vs(256, 512), vs(256, 512, 'q_boundary'), vs(256, 512, 'boundary_2d')]
    c = L - 64 if cut else L
    return LayerSpec('scene-cut' if cut else 'no-cut', L, len(heads), 1, d, seed, heads, segs=segs,
                     targets=targets, target_amp=amp, target_rows=(text, c, L))


def config(i, L=None, seed=None):
    """The eight named workloads (1-based), optionally shortened to L tokens
    (structure kept, sizes scaled) for parity tests the oracle finishes fast."""
    s = i if seed is None else seed
    if i == 1:
        L_ = L or 4096
        return LayerSpec('tiny-4k', L_, 2, 2, 64, s, [ashape(64, 512), vs(128, 256)],
                         rope_base=1e4, strong_cols=16, strong_shared=True)
    if i == 2:
        L_ = L or 131072
        heads = []
        for h in range(32):
            r = h % 4
            heads.append(vs(1000, 4096) if r in (0, 1) else block(100) if r == 2 else ashape(128, 4096))
        return LayerSpec('llama3-8b-128k', L_, 32, 8, 128, s, heads, rope_base=5e5,
                         strong_cols=64, strong_shared=False)
    if i == 3:
        L_ = L or 262144
        return LayerSpec('block-stress-256k', L_, 32, 8, 128, s, [block(128)] * 32,
                         cluster_blocks=min(512, L_ // 64 // 2))
    if i == 4:
        if L is None:
            text, frames, per = 512, 1600, 196
        else:
            per = 49
            text = 64
            frames = max(2, (L - text) // per)
        segs = [(0, text, TEXT), (text, frames * per, VIDEO)]
        L_ = text + frames * per
        heads = []
        for g in range(4):
            for hh in range(7):
                if hh < 5:
                    heads.append(grid(1, 64 if L is None else 16, 512 if L is None else 128))
                else:
                    heads.append(vs(1000, 4096) if L is None else vs(64, 128))
        return LayerSpec('qwen2-7b-video-314k', L_, 28, 4, 128, s, heads, segs=segs, period=per)
    if i == 5:
        if L is None:
            chunks, frames, per, text = 8, 640, 196, 2048
        else:
            chunks, per, text = 3, 49, 100
            frames = max(1, (L - 2 * text) // (chunks * per))
        segs, L_ = interleaved_segments(chunks, frames, per, text)
        gh = torch.Generator().manual_seed(s * 7 + 5)
        heads = []
        for h in range(32):
            r = h % 4
            if L is None:
                kv = int(torch.randint(5, 21, (1,), generator=gh)) * 100
                ks = int(torch.randint(2, 17, (1,), generator=gh)) * 512
            else:
                kv = int(torch.randint(1, 5, (1,), generator=gh)) * 16
                ks = int(torch.randint(1, 5, (1,), generator=gh)) * 32
            if r == 0:
                w = int(torch.randint(1, 3, (1,), generator=gh))
                heads.append(grid(w, 64 if L is None else 16, 512 if L is None else 128,
                                  layout='modality_grouped'))
            elif r == 1:
                heads.append(vs(kv, ks, 'q_boundary'))
            elif r == 2:
                heads.append(vs(kv, ks, 'boundary_2d'))
            else:
                heads.append(vs(kv, ks, 'plain'))
        return LayerSpec('mixed-1m', L_, 32, 8, 128, s, heads, segs=segs, period=per)
    if i == 8:
        # the video grid layer with its grid heads widened by a sink (the text
        # prompt) and a local window of four frames on the rows off the lines
        base = config(4, L=L, seed=s)
        per = base.period
        sink, window = (512, 4 * 196) if L is None else (64, 4 * per)
        heads = [dict(h, sink=sink, window=window) if h['pattern'] == 'grid' else h for h in base.heads]
        return replace(base, name='qwen2-7b-video-314k-window', heads=heads)
    if i == 7:
        # the 1M mixed layer with per-segment estimation in place of the
        # per-modality (Q-boundary) heads: 15 segments, 15 estimates per head
        base = config(5, L=L, seed=s)
        heads = [dict(h, layout='q_segment') if h['layout'] == 'q_boundary' else h for h in base.heads]
        return replace(base, name='mixed-1m-segments', heads=heads)
    if i == 6:
        # parallel encoding over a long video: a prompt, frames of 196 tokens,
        # a question as long as the prompt; the sink block is the prompt and
        # the first 16 frames, context blocks are 16 frames
        if L is None:
            text, frames, per, fpb = 512, 512, 196, 16
        else:
            text, per, fpb = 64, 49, 2
            frames = max(2 * fpb + 1, (L - 2 * text) // per)
        segs = [(0, text, TEXT), (text, frames * per, VIDEO), (text + frames * per, text, TEXT)]
        L_ = 2 * text + frames * per
        heads = [parallel(text + fpb * per, fpb * per, text)] * 28
        return LayerSpec('pevlm-video-101k', L_, 28, 4, 128, s, heads, segs=segs, period=per)
    raise ValueError(i)


def small_spec(name, L, Hq, Hkv, d, heads, seed=0, **kw):
    return LayerSpec(name, L, Hq, Hkv, d, seed, heads, **kw)


def with_heads(spec, heads, **kw):
    return replace(spec, heads=heads, **kw)
