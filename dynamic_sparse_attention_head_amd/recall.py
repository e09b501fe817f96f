"""Attention recall of the estimated masks, and a kernel-aware budget search.

MInference 1.0 summary page, "Approach": each head's pattern and sparsity
budget are chosen offline by a kernel-aware search that scores a choice by its
attention recall at the FLOPs the GPU kernel really spends.  The pages run it
on a calibration sample of a real model; here it runs on the synthetic layers
only, so its numbers describe those layers, not a model.

Recall of query row i is the share of its dense causal softmax mass that falls
on the keys its mask selects.  Both log-sum-exps come from the library's own
attention call:

    recall(i) = exp(LSE_mask(i) - LSE_dense(i))

with the dense one taken over an all-causal A-shape plan (sink 0, window L).
FLOPs are kernel-aware: the plan's computed 64x64 tile chunks per head
(4 d 64 64 each), which is what the attention kernel executes, beside the
exact selected pairs (4 d per pair).

This module analyses the path; it is not part of it.  Its statistics are
torch reductions over the two LSE vectors and the plan's counters.
"""
from __future__ import annotations

import torch

from . import mmsa


def _forward(q, k, v, heads, segs, materialize=False):
    lay = mmsa.Layer(q, k, v, heads, segs=segs, materialize=materialize)
    B, Hq, L, d = q.shape
    o = torch.empty((B, Hq, L, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device)
    lay.forward(q, k, v, o, lse)
    return lay, lse


def dense_heads(Hq, L):
    """Every causal key of every row: A-shape with no sink and a window of L."""
    return [dict(pattern="ashape", layout="plain", sink=0, window=max(L, 1))] * Hq


def dense_lse(q, k, v, segs=None):
    """LSE of dense causal attention, [B, Hq, L] float32."""
    _, lse = _forward(q, k, v, dense_heads(q.shape[1], q.shape[2]), segs)
    return lse


def row_recall(q, k, v, heads, segs=None, lse_dense=None):
    """(layer, recall [Hq, L] float64 of batch 0): per row, the share of its
    dense causal softmax mass on the keys its mask selects."""
    if lse_dense is None:
        lse_dense = dense_lse(q, k, v, segs)
    lay, lse = _forward(q, k, v, heads, segs)
    torch.cuda.synchronize()
    return lay, torch.exp((lse[0].double() - lse_dense[0].double()).clamp(max=0.0))


def layer_recall(q, k, v, heads, segs=None, lse_dense=None):
    """Per head of batch 0: recall statistics over all rows and the plan's FLOPs.

    Returns a list of dicts (one per q head) with mean_recall, min_recall,
    p05_recall (5th percentile), planned_flops, selected_flops, dense_flops."""
    lay, rec = row_recall(q, k, v, heads, segs, lse_dense)
    B, Hq, L, d = q.shape
    dense_pairs = L * (L + 1) // 2
    out = []
    for h in range(Hq):
        info = lay.view("tile_info", h).view(-1, 4)
        chunks = int(info[:, 2].clamp(min=0).sum().item())
        pairs = int(lay.view("tile_pairs", h).sum().item())
        r = rec[h]
        out.append(dict(head=h, pattern=heads[h]["pattern"], layout=heads[h].get("layout", "plain"),
                        mean_recall=float(r.mean()), min_recall=float(r.min()),
                        p05_recall=float(torch.quantile(r.float(), 0.05)) if L > 0 else 1.0,
                        planned_flops=4.0 * d * 64 * 64 * chunks, selected_flops=4.0 * d * pairs,
                        dense_flops=4.0 * d * dense_pairs))
    return out


def sweep(base_heads, pattern, budgets):
    """Candidate head lists: every head of `pattern` in base_heads gets each
    budget dict in turn (merged over its own config); the others are kept."""
    cands = []
    for b in budgets:
        cands.append([dict(h, **b) if h["pattern"] == pattern else dict(h) for h in base_heads])
    return cands


def budget_search(q, k, v, candidates, target=0.95, segs=None):
    """Kernel-aware per-head choice: among the candidate head lists, each head
    takes the configuration of least planned FLOPs whose mean recall reaches
    `target`, else the one of highest recall.  Returns (chosen heads, table),
    the table holding every candidate's statistics per head."""
    lse_d = dense_lse(q, k, v, segs)
    table = [layer_recall(q, k, v, heads, segs, lse_d) for heads in candidates]
    chosen = []
    for h in range(q.shape[1]):
        opts = [(table[c][h], candidates[c][h]) for c in range(len(candidates))]
        ok = [o for o in opts if o[0]["mean_recall"] >= target]
        if ok:
            best = min(ok, key=lambda o: (o[0]["planned_flops"], -o[0]["mean_recall"]))
        else:
            best = max(opts, key=lambda o: o[0]["mean_recall"])
        chosen.append(dict(best[1]))
    return chosen, table


def scene_cut_recall(spec, lse_dense=None):
    """Mean recall per head of the video rows before the scene cut that come
    after the planted keys (rows [(r0 + cut) // 2, cut)), and of the rows from
    the cut on, for a layer from `synth.scene_cut`."""
    q, k, v = spec["q"], spec["k"], spec["v"]
    s = spec["spec"]
    _, rec = row_recall(q, k, v, s.heads, s.segs, lse_dense)
    r0, cut, r1 = s.target_rows
    pre = rec[:, (r0 + cut) // 2:cut].mean(dim=1)
    post = rec[:, cut:r1].mean(dim=1) if r1 > cut else torch.full_like(pre, float("nan"))
    return pre, post


def scene_cut_study(frames=160, per=196, text=512, amps=(6.0, 10.0), budgets=((256, 512), (1000, 4096))):
    """The MMInference verdict page's falsifier on synthetic input: a video
    segment whose last 64 queries (the rows the per-modality estimate uses)
    aim at other keys than the rest of the segment.  For each amplitude and
    vertical-slash budget, the recall of the earlier rows with and without the
    cut, per layout (plain, Q-boundary, 2D-boundary)."""
    from . import synth
    out = []
    for amp in amps:
        for kv, ks in budgets:
            heads = [synth.vs(kv, ks), synth.vs(kv, ks, "q_boundary"), synth.vs(kv, ks, "boundary_2d")]
            row = dict(amp=amp, k_vertical=kv, k_slash=ks)
            for cut in (False, True):
                spec = synth.scene_cut(frames, per, text, cut=cut, amp=amp, heads=heads)
                lay = synth.make_layer(spec, "cuda")
                pre, post = scene_cut_recall(lay)
                row["cut" if cut else "no_cut"] = [round(float(x), 4) for x in pre]
                if cut:
                    row["after_cut"] = [round(float(x), 4) for x in post]
                del lay
            out.append(row)
    return out


def _summary(rows):
    groups = {}
    for r in rows:
        groups.setdefault((r["pattern"], r["layout"]), []).append(r)
    lines = []
    for (p, l), rs in groups.items():
        n = len(rs)
        lines.append(f"  {p + '/' + l:22s} heads {n:2d}  mean recall {sum(r['mean_recall'] for r in rs) / n:.4f}"
                     f"  min {min(r['min_recall'] for r in rs):.4f}"
                     f"  planned density {sum(r['planned_flops'] for r in rs) / sum(r['dense_flops'] for r in rs):.4f}"
                     f"  selected density {sum(r['selected_flops'] for r in rs) / sum(r['dense_flops'] for r in rs):.4f}")
    return "\n".join(lines)


def main():
    import argparse
    import time

    from . import synth

    ap = argparse.ArgumentParser(description="recall vs kernel FLOPs of the estimated masks on a synthetic layer")
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--target", type=float, default=0.95)
    ap.add_argument("--scene-cut", action="store_true",
                    help="run the scene-cut stress (recall of a video segment's earlier rows when its last "
                         "64 queries attend elsewhere) instead of the budget sweep")
    args = ap.parse_args()
    if args.scene_cut:
        print("scene cut at the end of the video segment; recall of the earlier rows "
              "(plain, Q-boundary, 2D-boundary vertical-slash heads)", flush=True)
        for r in scene_cut_study():
            print(f"  amp {r['amp']:4.1f} budget {r['k_vertical']}/{r['k_slash']}: no cut {r['no_cut']}  "
                  f"cut {r['cut']}  rows after the cut {r['after_cut']}", flush=True)
        return
    spec = synth.config(args.config)
    lay = synth.make_layer(spec, "cuda")
    q, k, v = lay["q"], lay["k"], lay["v"]
    dense_lse(q, k, v, spec.segs)   # warm-up (library load, workspace)
    torch.cuda.synchronize()
    t0 = time.time()
    lse_d = dense_lse(q, k, v, spec.segs)
    torch.cuda.synchronize()
    t1 = time.time()
    rows = layer_recall(q, k, v, spec.heads, spec.segs, lse_d)
    t2 = time.time()
    print(f"{spec.name}: L={spec.L}; dense pass {1e3 * (t1 - t0):.1f} ms, sparse pass + statistics "
          f"{1e3 * (t2 - t1):.1f} ms", flush=True)
    print("configured budgets:")
    print(_summary(rows), flush=True)
    sweeps = {
        "vs": [dict(k_vertical=a, k_slash=b) for a, b in ((125, 512), (250, 1024), (500, 2048), (1000, 4096),
                                                            (2000, 8192))],
        "block": [dict(k_blocks=kb) for kb in (25, 50, 100, 200, 400)],
        "ashape": [dict(sink=128, window=w) for w in (1024, 2048, 4096, 8192, 16384)],
        "grid": [dict(grid_phases=w) for w in (1, 2, 4)],
    }
    cands, tables = [], []
    for pat, budgets in sweeps.items():
        if not any(h["pattern"] == pat for h in spec.heads):
            continue
        for b, heads in zip(budgets, sweep(spec.heads, pat, budgets)):
            rows = layer_recall(q, k, v, heads, spec.segs, lse_d)
            print(f"{pat} {b}:")
            print(_summary([r for r in rows if r["pattern"] == pat]), flush=True)
            cands.append(heads)
            tables.append(rows)
    if cands:
        # per head: the cheapest swept budget reaching the target
        chosen = []
        for h in range(spec.Hq):
            opts = [(tables[c][h], cands[c][h]) for c in range(len(cands))]
            ok = [o for o in opts if o[0]["mean_recall"] >= args.target]
            best = min(ok, key=lambda o: o[0]["planned_flops"]) if ok else max(opts, key=lambda o: o[0]["mean_recall"])
            chosen.append(best)
        tot_p = sum(o[0]["planned_flops"] for o in chosen)
        tot_d = sum(o[0]["dense_flops"] for o in chosen)
        print(f"budget search at mean recall >= {args.target}: planned density {tot_p / tot_d:.4f}, "
              f"mean recall {sum(o[0]['mean_recall'] for o in chosen) / len(chosen):.4f}")
        for o in chosen:
            c = o[1]
            print(f"  head {o[0]['head']:2d} {c['pattern']:6s} "
                  + " ".join(f"{key}={c[key]}" for key in ("k_vertical", "k_slash", "k_blocks", "window", "grid_phases")
                             if key in c)
                  + f"  recall {o[0]['mean_recall']:.4f}  planned density {o[0]['planned_flops'] / o[0]['dense_flops']:.4f}")


if __name__ == "__main__":
    main()
