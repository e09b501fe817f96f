"""Benchmark of one sparse-prefill layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu]
    python bench.py --copy-calibration     # plain copy of known size, for counter scaling

A step is one pass of the whole path (estimate_vs, estimate_blocks, permute,
sparse_prefill, unpermute) over one layer of synthetic bf16 inputs resident in
HBM.  The default workload is the LLaMA-3-8B-shaped layer at 131072 tokens
(32 q / 8 KV heads, d = 128; 16 vertical-slash, 8 block-sparse, 8 A-shape
heads).  Prints one JSON line: `value` is the effective TFLOP/s
(4 * d * exactly selected (query, key) pairs / time per layer), with the
attention kernel's roofline (tile FLOPs against the bf16 MFMA peak) and the
CPU oracle timed on a bounded sample of the same layer.
"""
from __future__ import annotations

import argparse
import collections
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

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0
CSRC = os.path.join(ROOT, "dynamic_sparse_attention_head_amd", "csrc")
ATTN_SOURCES = ("k_attention.hip", "mmsa_device.h", "mmsa_internal.h", "k_permute.hip")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def plan_totals(L, spec):
    """Sum over heads of exact selected pairs and computed 64x64 tile chunks."""
    pairs = 0
    tiles = 0
    for h in range(spec.Hq):
        pairs += int(L.view("tile_pairs", h).sum().item())
        info = L.view("tile_info", h).view(-1, 4)
        tiles += int(info[:, 2].to(torch.int64).sum().item())
    return pairs, tiles


def est_bytes(spec):
    """Algorithmic HBM bytes of mmsa_estimate_vs: K of every KV head that has a
    vertical-slash or grid head is streamed twice; the estimation rows of Q are
    read twice (negligible)."""
    gmap = [h // (spec.Hq // spec.Hkv) for h in range(spec.Hq)]
    kvs = {gmap[h] for h in range(spec.Hq) if spec.heads[h]["pattern"] in ("vs", "grid")}
    return 2 * len(kvs) * spec.L * spec.d * 2


def attn_source_digest():
    """sha256 over the attention kernel's sources and the plan kernels that
    order its work queue: counter figures taken on another version of either
    are not reported."""
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary of
    this workload, or None when it is missing or was taken on other sources."""
    path = os.path.join(PROFILES, f"k_attn_{workload}_traffic.md")
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
    try:
        return int(float(kv["traffic bytes per launch"]))
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


def cpu_baseline(spec, lay, seed=0, rows_per_head=768):
    """The CPU oracle, as written, on a bounded sample: for one head of each
    pattern present, full index estimation plus attention on sampled rows.
    Returns effective TFLOP/s of the sample (4 d |selected pairs| / time)."""
    import oracle.mmsa_oracle as O
    try:
        from threadpoolctl import threadpool_limits
        cores = len(os.sched_getaffinity(0))
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
        limiter = None
    gmap = O.kv_head_map(spec.Hq, spec.Hkv)
    seen, heads = set(), []
    for h in range(spec.Hq):
        key = (spec.heads[h]["pattern"], spec.heads[h].get("layout", "plain"))
        if key not in seen:
            seen.add(key)
            heads.append(h)
    rng = np.random.default_rng(seed)
    flops = 0.0
    t0 = time.perf_counter()
    for h in heads:
        qh = lay["q"][0, h].float().cpu().numpy().astype(np.float64)
        kh = lay["k"][0, gmap[h]].float().cpu().numpy().astype(np.float64)
        vh = lay["v"][0, gmap[h]].float().cpu().numpy().astype(np.float64)
        hi = O.estimate_head(spec.heads[h], qh, kh, spec.segs, lay["scale"])
        rows = np.sort(rng.integers(0, spec.L, rows_per_head))
        cache = {}
        n_sel = sum(int(O.row_mask(hi, int(i), cache).sum()) for i in rows)
        O.head_attention(hi, qh, kh, vh, lay["scale"], rows)
        flops += 4.0 * spec.d * n_sel
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    sample = (f"{len(heads)} heads ({', '.join(spec.heads[h]['pattern'] for h in heads)}): full oracle "
              f"estimation + float64 attention on {rows_per_head} random rows each")
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=cores, kind="oracle", sample=sample,
                seconds=round(dt, 2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=768)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--materialize", action="store_true",
                    help="explicit gathers of permuted Q / grouped K,V and an output scatter "
                         "instead of index-based loads and stores in the attention call")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the path would shard by KV "
              f"head without collectives, but no multi-GPU launch is implemented.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(max(args.steps, 1))
        return
    dev = torch.device("cuda")
    spec = synth.config(args.config)
    log(f"[bench] generating {spec.name}: L={spec.L} Hq={spec.Hq} Hkv={spec.Hkv} d={spec.d}")
    lay = synth.make_layer(spec, dev)
    q, k, v = lay["q"], lay["k"], lay["v"]
    L = mmsa.Layer(q, k, v, spec.heads, segs=spec.segs, materialize=args.materialize)
    L.alloc_workspace()
    o = torch.empty((1, spec.Hq, spec.L, spec.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, spec.Hq, spec.L), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"[bench] workspace {L.workspace_bytes() / 1e9:.2f} GB; warmup {args.warmup}")
    calls = ["estimate_vs", "estimate_blocks", "permute", "sparse_prefill", "unpermute"]

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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pairs, tiles = plan_totals(L, spec)
    log(f"[bench] selected pairs {pairs:.4e}, computed 64x64 tiles {tiles}")
    # timed region
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = np.zeros(5)
    for e in evs:
        for c in range(5):
            per_call[c] += e[c].elapsed_time(e[c + 1])
    per_call /= args.steps
    ms_step = sum(per_call)
    ms_wall = wall * 1e3 / args.steps
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/layer (events), {ms_wall:.3f} ms/layer (wall)")
    for c, name in enumerate(calls):
        log(f"[bench]   {name:16s} {per_call[c]:9.3f} ms")
    eff_tflops = 4.0 * spec.d * pairs / (ms_step * 1e-3) / 1e12
    attn_ms = per_call[3]
    tile_flops = 4.0 * spec.d * 64 * 64 * tiles
    achieved = tile_flops / (attn_ms * 1e-3) / 1e12
    est_gbps = est_bytes(spec) / (per_call[0] * 1e-3) / 1e9 if per_call[0] > 0 else None
    out = {
        "metric": "sparse prefill ms/layer + effective TFLOP/s (% MFMA peak) at 128K-1M tokens",
        "value": round(eff_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}: one causal prefill layer, L={spec.L}, {spec.Hq} q / {spec.Hkv} kv "
                               f"heads, d={spec.d}", "batch": 1, "seq_len": spec.L,
                   "permutation": "materialised" if args.materialize else "index-based",
                   "heads": "16 vertical-slash (1000/4096), 8 block (top-100), 8 A-shape (128, 4096)"
                   if args.config == 2 else ", ".join(f"{n} {p}" for p, n in collections.Counter(
                       f"{h['pattern']}/{h.get('layout', 'plain')}" for h in spec.heads).items())},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(spec.name),
                     "kernel": "k_attn (mmsa_sparse_prefill)", "launch_ms": round(attn_ms, 3)},
        "effective_pct_mfma_peak": round(100 * eff_tflops / PEAK_BF16_TFLOPS, 2),
        "selected_pairs": pairs,
        "computed_tiles": tiles,
        "ms_per_call": {n: round(float(x), 3) for n, x in zip(calls, per_call)},
        "estimation_gbps": None if est_gbps is None else round(est_gbps, 1),
        "estimation_pct_hbm": None if est_gbps is None else round(100 * est_gbps / PEAK_HBM_GBPS, 2),
        "ms_per_step_wall": round(ms_wall, 3),
    }
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(spec, lay, rows_per_head=args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
