"""Benchmark of one sparse-prefill layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--no-cpu] [--materialize]
    python bench.py --copy-calibration     # plain copy of known size, for counter scaling
    python bench.py --peaks                # measured MFMA and copy peaks only

A step is one pass of the whole path (estimate_vs, estimate_blocks, permute,
sparse_prefill, unpermute) over one layer of synthetic bf16 inputs resident in
HBM.  The default workload is the 1M-token mixed-modality layer (L = 1,017,856:
8 video chunks of 640 frames x 196 tokens between 2048-token text spans;
32 q / 8 KV heads, d = 128; grid, Q-boundary, 2D-boundary and plain
vertical-slash heads); --config 2 is the LLaMA-3-8B-shaped layer at 131,072
tokens.  Prints one JSON line: `value` is the effective TFLOP/s (4 * d *
exactly selected (query, key) pairs / wall time per layer), with the attention
kernel's roofline (planned 64x64 tile FLOPs against the bf16 MFMA peak), the
other calls against the roof that bounds each, peaks measured on this GPU
beside the datasheet ones, and the CPU oracle timed on a bounded sample of
the same layer with its time extrapolated to the whole layer.
"""
from __future__ import annotations

import argparse
import collections
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from dynamic_sparse_attention_head_amd import mmsa, synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (datasheet)
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector (datasheet)
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E (datasheet)
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)   # FLOP per byte where the two roofs meet
CSRC = os.path.join(ROOT, "dynamic_sparse_attention_head_amd", "csrc")
ATTN_SOURCES = ("k_attention.hip", "mmsa_device.h", "mmsa_internal.h", "k_permute.hip")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30
CALLS = ["estimate_vs", "estimate_blocks", "permute", "sparse_prefill", "unpermute"]
TEXT, VIDEO = 0, 1


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic work of each call (what the roofline fractions divide by)
# ---------------------------------------------------------------------------
def plan_totals(L, spec):
    """Over all heads: exact selected pairs, computed 64x64 tile chunks, and
    staged chunks (per pair of adjacent query tiles: the union of their key
    tiles plus their gathered 64-column chunks, each staged once)."""
    pairs = tiles = staged = 0
    for h in range(spec.Hq):
        pairs += int(L.view("tile_pairs", h).sum().item())
        info = L.view("tile_info", h).view(-1, 4).to(torch.int64)
        tiles += int(info[:, 2].sum().item())
        bm = L.view("tile_bitmap", h)
        nT = info.shape[0]
        W = bm.numel() // max(nT, 1)
        bm = bm.view(nT, W)
        if nT % 2:
            bm = torch.cat([bm, torch.zeros_like(bm[:1])])
            info = torch.cat([info, torch.zeros_like(info[:1])])
        u = (bm[0::2] | bm[1::2]).view(torch.uint8).cpu().numpy()
        staged += int(np.unpackbits(u).sum())
        g = info[:, 1]
        gch = (g + 63) // 64
        if spec.heads[h]["pattern"] == "grid":    # both tiles read one shared line list
            staged += int(torch.maximum(gch[0::2], gch[1::2]).sum().item())
        else:
            staged += int(gch.sum().item())
    return pairs, tiles, staged


def est_regions(spec):
    """(q head, rows, largest row position, keys of the pass-2 view) of every
    estimation region: the last 64 queries of the layer, of each modality or
    segment, or of the grid order."""
    L = spec.L
    segs = spec.segs or [(0, L, TEXT)]
    last = {}
    n_mod = collections.Counter()
    for s, n, m in segs:
        last[m] = s + n - 1
        n_mod[m] += n
    out = []
    for h, c in enumerate(spec.heads):
        p, lay = c["pattern"], c.get("layout", "plain")
        if p == "vs" and lay == "plain" or p == "grid" and lay == "plain":
            out.append((h, min(64, L), L - 1, L))
        elif p == "vs" and lay in ("q_boundary", "boundary_2d"):
            for m in (TEXT, VIDEO):
                if n_mod[m]:
                    out.append((h, min(64, n_mod[m]), last[m], L if lay == "boundary_2d" else last[m] + 1))
        elif p == "vs" and lay == "q_segment":
            for s, n, m in segs:
                out.append((h, min(64, n), s + n - 1, s + n))
        elif p == "grid":     # modality-grouped: the last 64 video queries
            m = VIDEO if n_mod[VIDEO] else TEXT
            out.append((h, min(64, L), last[m], L))
    return out


def est_work(spec):
    """mmsa_estimate_vs: bf16 MFMA FLOPs (two passes of scale*q.k over every
    estimation row's keys) and HBM bytes (K of each KV head with an estimated
    head, streamed once per pass)."""
    d = spec.d
    regs = est_regions(spec)
    flops = sum(2.0 * d * rows * ((imax + 1) + view) for _, rows, imax, view in regs)
    gmap = [h // (spec.Hq // spec.Hkv) for h in range(spec.Hq)]
    kvs = {gmap[h] for h, *_ in regs}
    return flops, 2.0 * len(kvs) * spec.L * d * 2


def block_work(spec):
    """mmsa_estimate_blocks: HBM bytes of the pooling (Q of each block head and
    K of its KV head read once) and fp32 FMA FLOPs of the pooled logits."""
    d, L = spec.d, spec.L
    gmap = [h // (spec.Hq // spec.Hkv) for h in range(spec.Hq)]
    heads = [h for h in range(spec.Hq) if spec.heads[h]["pattern"] == "block"]
    nB = -(-L // 64)
    by = (len(heads) + len({gmap[h] for h in heads})) * L * d * 2.0
    return 2.0 * d * nB * (nB + 1) / 2 * len(heads), by


def gather_bytes(spec):
    """Bytes moved by the explicit gathers of --materialize (mmsa_permute) and
    the output scatter (mmsa_unpermute): each permuted head's Q rows read and
    written, grouped K and V of each KV head a 2D-boundary head uses."""
    d, L = spec.d, spec.L
    gmap = [h // (spec.Hq // spec.Hkv) for h in range(spec.Hq)]
    perm = [h for h, c in enumerate(spec.heads)
            if c["pattern"] == "grid" or c.get("layout", "plain") in ("q_boundary", "boundary_2d", "q_segment")]
    kv2d = {gmap[h] for h, c in enumerate(spec.heads) if c.get("layout") == "boundary_2d"}
    g = 2.0 * len(perm) * L * d * 2 + 2.0 * 2 * len(kv2d) * L * d * 2
    return g, 2.0 * len(perm) * L * d * 2


def roof(kind, amount, ms, peak, unit):
    a = amount / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
    return {"bound": kind, "achieved": round(a, 2), "peak": peak, "unit": unit, "frac": round(a / peak, 4)}


# ---------------------------------------------------------------------------
# Counter figures and measured peaks
# ---------------------------------------------------------------------------
def attn_source_digest():
    """sha256 over the attention kernel's sources and the plan kernels that
    order its work queue: counter figures taken on another version of either
    are not reported."""
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_summary(workload, what):
    """The machine-readable lines ("- key: value") of a committed counter
    summary of the attention kernel on this workload, or None when it is
    missing or was taken on other sources."""
    path = os.path.join(PROFILES, f"k_attn_{workload}_{what}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                kv[k.strip()] = v.strip().strip("`")
    if kv.get("attention sources sha256") != attn_source_digest():
        return None
    return kv


def read_traffic(workload):
    """HBM bytes per attention launch (FETCH_SIZE + WRITE_SIZE, scaled)."""
    kv = read_summary(workload, "traffic")
    try:
        return int(float(kv["traffic bytes per launch"])) if kv else None
    except (KeyError, ValueError):
        return None


def read_mfma_busy(workload):
    """Share of the launch's SIMD cycles in which the matrix cores were busy
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE), and the clock it ran at."""
    kv = read_summary(workload, "mfma")
    try:
        return {"fraction": float(kv["mfma busy fraction"]), "clock_ghz": float(kv["clock ghz"]),
                "counters": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE"} if kv else None
    except (KeyError, ValueError):
        return None


def copy_calibration(steps):
    """A plain streaming kernel of known size: y = x * 1 over COPY_BYTES of bf16
    (reads and writes COPY_BYTES each per launch)."""
    n = COPY_BYTES // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        torch.mul(x, 1.0, out=y)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "launches": steps,
                      "ms_per_launch": round(ms, 4), "gbps": round(2 * COPY_BYTES / ms / 1e6, 1)}), flush=True)


def measured_peaks():
    """An MFMA loop (v_mfma_f32_32x32x16_bf16, two workgroups of 4 waves per
    CU, as the attention kernel runs) and a 16-byte-per-lane copy of 2 GiB,
    each timed with events over several launches after a warm-up launch."""
    from dynamic_sparse_attention_head_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        return None
    P = ctypes.CDLL(B.PROBE_LIB)
    P.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    P.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * n_cu, 20000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    ms = timed(lambda: P.probe_mfma(blocks, iters, ctypes.c_void_p(sink.data_ptr()), st), 5)
    mfma = blocks * 4.0 * iters * 4 * 32 * 32 * 16 * 2 / (ms * 1e-3) / 1e12
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms_c = timed(lambda: P.probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                                      32 * n_cu, st), 10)
    copy = 2.0 * nbytes / (ms_c * 1e-3) / 1e9
    rsink = torch.empty(32 * n_cu * 256, dtype=torch.int32, device="cuda")
    ms_r = timed(lambda: P.probe_read(ctypes.c_void_p(src.data_ptr()), nbytes, 32 * n_cu,
                                      ctypes.c_void_p(rsink.data_ptr()), st), 10)
    read = nbytes / (ms_r * 1e-3) / 1e9
    del src, dst, sink, rsink
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma, 1), "copy_gbps": round(copy, 1), "read_gbps": round(read, 1),
            "datasheet": {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbps": PEAK_HBM_GBPS},
            "how": f"bf16 32x32x16 MFMA loop, {blocks} workgroups x 4 waves; copy (read + write) and read-only "
                   f"stream of 2 GiB, 16 B per lane"}


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, lay, eff_flops, seed=0, rows_per_head=24):
    """The CPU oracle, as written, on a bounded sample of the layer: for one
    head of each (pattern, layout), its full index estimation and its float64
    attention on sampled rows (the first and the last row, the rest uniform).
    Estimation time is scaled by the heads of each kind; attention time by the
    per-row cost weights (a row's causal length i + 1) summed over the layer.
    `value` is the layer's effective FLOPs over that extrapolated time."""
    import oracle.mmsa_oracle as O
    try:
        from threadpoolctl import threadpool_limits
        cores = len(os.sched_getaffinity(0))
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
        limiter = None
    gmap = O.kv_head_map(spec.Hq, spec.Hkv)
    kinds = collections.OrderedDict()
    for h in range(spec.Hq):
        kinds.setdefault((spec.heads[h]["pattern"], spec.heads[h].get("layout", "plain")), []).append(h)
    rng = np.random.default_rng(seed)
    L = spec.L
    layer_weight = L * (L + 1) / 2.0
    est_s = att_s = 0.0
    t_all = time.perf_counter()
    for key, hs in kinds.items():
        h = hs[0]
        qh = lay["q"][0, h].float().cpu().numpy().astype(np.float64)
        kh = lay["k"][0, gmap[h]].float().cpu().numpy().astype(np.float64)
        vh = lay["v"][0, gmap[h]].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        hi = O.estimate_head(spec.heads[h], qh, kh, spec.segs, lay["scale"])
        est_s += (time.perf_counter() - t0) * len(hs)
        rows = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, rows_per_head - 2)]))
        t0 = time.perf_counter()
        O.head_attention(hi, qh, kh, vh, lay["scale"], rows)
        dt = time.perf_counter() - t0
        att_s += dt / float(np.sum(rows + 1.0)) * layer_weight * len(hs)
        del qh, kh, vh, hi
    wall = time.perf_counter() - t_all
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    total_ms = (est_s + att_s) * 1e3
    sample = (f"one head per kind ({', '.join(f'{p}/{l}' for p, l in kinds)}): full oracle estimation, "
              f"float64 attention on {rows_per_head} rows each; scaled to {spec.Hq} heads and to all {L} rows "
              f"by causal length")
    return dict(value=eff_flops / (total_ms * 1e-3) / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                sample=sample, cpu_model=cpu_model(), oracle_estimation_ms=round(est_s * 1e3, 1),
                oracle_attention_ms_extrapolated=round(att_s * 1e3, 1), oracle_layer_ms_extrapolated=round(total_ms, 1),
                seconds=round(wall, 2))


def grid_sigma_report(L, spec):
    """Detected strides of the grid heads (the generator's sanity check: the
    planted period is 196 tokens per frame)."""
    sig = [int(L.view("grid", h)[0].item()) for h in range(spec.Hq) if spec.heads[h]["pattern"] == "grid"]
    if not sig:
        return None
    c = collections.Counter(sig)
    return {"heads": len(sig), "period": spec.period, "detected_period": c.get(spec.period, 0),
            "share": round(c.get(spec.period, 0) / len(sig), 3), "strides": dict(sorted(c.items()))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="oracle rows per head kind (default: 24 at 1M tokens, more for shorter layers)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--peaks", action="store_true", help="measure the MFMA and copy peaks only")
    ap.add_argument("--materialize", action="store_true",
                    help="explicit gathers of permuted Q / grouped K,V and an output scatter "
                         "instead of index-based loads and stores in the attention call")
    ap.add_argument("--keys", choices=["auto", "asc", "desc"], default="auto",
                    help="key-tile walk order of the attention call (default: chosen by size)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the path would shard by KV "
              f"head without collectives, but no multi-GPU launch is implemented.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(max(args.steps, 1))
        return
    if args.peaks:
        print(json.dumps(measured_peaks()), flush=True)
        return
    dev = torch.device("cuda")
    peaks = None if args.no_peaks else measured_peaks()
    if peaks:
        log(f"[bench] measured peaks: {peaks['mfma_bf16_tflops']} TFLOP/s bf16 MFMA, {peaks['copy_gbps']} GB/s copy")
    spec = synth.config(args.config)
    log(f"[bench] generating {spec.name}: L={spec.L} Hq={spec.Hq} Hkv={spec.Hkv} d={spec.d}")
    lay = synth.make_layer(spec, dev)
    q, k, v = lay["q"], lay["k"], lay["v"]
    flags = {"auto": 0, "asc": mmsa.FLAG_KEYS_ASCENDING, "desc": mmsa.FLAG_KEYS_DESCENDING}[args.keys]
    L = mmsa.Layer(q, k, v, spec.heads, segs=spec.segs, materialize=args.materialize, flags=flags)
    L.alloc_workspace()
    o = torch.empty((1, spec.Hq, spec.L, spec.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, spec.Hq, spec.L), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"[bench] workspace {L.workspace_bytes() / 1e9:.2f} GB; warmup {args.warmup}")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        L.estimate_vs(q, k)
        if ev is not None:
            ev[1].record(stream)
        L.estimate_blocks(q, k)
        if ev is not None:
            ev[2].record(stream)
        L.permute(q, k, v)
        if ev is not None:
            ev[3].record(stream)
        L.sparse_prefill(q, k, v, o, lse)
        if ev is not None:
            ev[4].record(stream)
        L.unpermute(o)
        if ev is not None:
            ev[5].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warm-up step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    # timed region: exactly K steps between two synchronisations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the plan every step rebuilt (read after the timed region, so that a run
    # without warm-up steps reads a built plan too)
    pairs, tiles, staged = plan_totals(L, spec)
    log(f"[bench] selected pairs {pairs:.4e}, computed 64x64 tiles {tiles}, staged chunks {staged}")
    per = np.array([[e[c].elapsed_time(e[c + 1]) for c in range(5)] for e in evs])   # [steps, calls] ms
    per_step = per.sum(axis=1)
    mean_call = per.mean(axis=0)
    ms_wall = wall * 1e3 / args.steps
    log(f"[bench] {args.steps} steps: {ms_wall:.3f} ms/layer (wall), events mean {per_step.mean():.3f} / median "
        f"{np.median(per_step):.3f} / min {per_step.min():.3f} ms")
    for c, name in enumerate(CALLS):
        log(f"[bench]   {name:16s} mean {mean_call[c]:9.3f} ms  median {np.median(per[:, c]):9.3f}  "
            f"min {per[:, c].min():9.3f}")
    eff_flops = 4.0 * spec.d * pairs
    eff_tflops = eff_flops / (ms_wall * 1e-3) / 1e12
    attn_ms = float(mean_call[3])
    tile_flops = 4.0 * spec.d * 64 * 64 * tiles
    attn_roof = roof("mfma", tile_flops, attn_ms, PEAK_BF16_TFLOPS, "TFLOP/s")
    attn_roof.update({"traffic": read_traffic(spec.name), "kernel": "k_attn (mmsa_sparse_prefill)",
                      "launch_ms": round(attn_ms, 3), "mfma_busy": read_mfma_busy(spec.name)})
    if peaks:
        attn_roof["frac_of_measured_peak"] = round(attn_roof["achieved"] / peaks["mfma_bf16_tflops"], 4)
    # the other calls, each against the roof that bounds it
    calls_roof = {}
    ef, eb = est_work(spec)
    if ef > 0 and mean_call[0] > 0:
        kind = "mfma" if ef / eb > RIDGE else "hbm"
        calls_roof["estimate_vs"] = (roof("mfma", ef, mean_call[0], PEAK_BF16_TFLOPS, "TFLOP/s") if kind == "mfma"
                                     else roof("hbm", eb, mean_call[0], PEAK_HBM_GBPS, "GB/s"))
        calls_roof["estimate_vs"]["flop_per_byte"] = round(ef / eb, 1)
        calls_roof["estimate_vs"]["hbm_gbps"] = round(eb / (mean_call[0] * 1e-3) / 1e9, 1)
        calls_roof["estimate_vs"]["hbm_frac"] = round(eb / (mean_call[0] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)
    bf, bb = block_work(spec)
    if bb > 0 and mean_call[1] > 0:
        calls_roof["estimate_blocks"] = roof("hbm", bb, mean_call[1], PEAK_HBM_GBPS, "GB/s")
        calls_roof["estimate_blocks"]["logit_fp32_tflops"] = round(bf / (mean_call[1] * 1e-3) / 1e12, 2)
    if args.materialize:
        gb, ub = gather_bytes(spec)
        if gb > 0:
            calls_roof["permute"] = roof("hbm", gb, mean_call[2], PEAK_HBM_GBPS, "GB/s")
            calls_roof["unpermute"] = roof("hbm", ub, mean_call[4], PEAK_HBM_GBPS, "GB/s")
    else:
        calls_roof["permute"] = {"bound": "alu", "ms": round(float(mean_call[2]), 3),
                                 "note": "plan compile only (integer work); no tensor is moved"}
    out = {
        "metric": "sparse prefill ms/layer + effective TFLOP/s (% MFMA peak) at 128K-1M tokens",
        "value": round(eff_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}: one causal prefill layer, L={spec.L}, {spec.Hq} q / {spec.Hkv} kv "
                               f"heads, d={spec.d}", "batch": 1, "seq_len": spec.L,
                   "permutation": "materialised" if args.materialize else "index-based",
                   "key_order": args.keys,
                   "heads": ", ".join(f"{n} {p}" for p, n in collections.Counter(
                       f"{h['pattern']}/{h.get('layout', 'plain')}" for h in spec.heads).items())},
        "roofline": attn_roof,
        "effective_pct_mfma_peak": round(100 * eff_tflops / PEAK_BF16_TFLOPS, 2),
        "ms_per_step_events": {"mean": round(float(per_step.mean()), 3), "median": round(float(np.median(per_step)), 3),
                               "min": round(float(per_step.min()), 3)},
        "ms_per_call": {n: {"mean": round(float(per[:, c].mean()), 3), "median": round(float(np.median(per[:, c])), 3),
                            "min": round(float(per[:, c].min()), 3)} for c, n in enumerate(CALLS)},
        "calls_roofline": calls_roof,
        "selected_pairs": pairs,
        "computed_tiles": tiles,
        "staged_chunks": staged,
        "measured_peaks": peaks,
        "grid_stride": grid_sigma_report(L, spec),
    }
    if not args.no_cpu:
        del L
        torch.cuda.empty_cache()
        log("[bench] timing the CPU oracle on a bounded sample")
        # about the same oracle time at any length: a row costs ~ its causal length
        rows = args.cpu_rows or max(24, min(768, int(24 * 1017856 / max(spec.L, 1))))
        out["cpu_baseline"] = cpu_baseline(spec, lay, eff_flops, rows_per_head=rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
