"""On-device tuner of the tile table (the M-bucket table of moe_tuned.h).

    python -m routed_grouped_gemm_amd.tune [--out PATH] [--report PATH] [--quick]

For each weight dtype (and for fp8 weights also in the fp8-activation mode, which has its own
m-tile kernels up to 160 rows) it times the layer, on random inputs of a real layer shape, at a
sweep of token counts M, under every candidate tile (m-tile rows x group size of the
grouped item order), and keeps per M the fastest candidate.  Neighbouring M with the same
winner merge into one bucket; the bucket boundary between two winners is the geometric
mean of their mean rows per routed expert.  The m-tile never shrinks as M grows (a candidate
smaller than the previous M's winner is not taken), and a candidate replaces the previous
M's winner, or else the current table's choice, only when more than 2% faster, so timing
noise does not split buckets.  The result is written as moe_tuned.h (rebuild the library
afterwards) and as a report of every measurement.

This is the per-device, per-M tuning the vLLM config page describes (sections 03 and 08:
one tile setting per M bucket, found by timing a grid of candidates on the device), done
for this kernel's own tile parameters.  Inputs are random (hidden ~ N(0,1), weights
~ N(0, 1/fan_in), fp8 weights block-quantised with 128x128 scales) and made with torch on
the device; only their shapes and routing statistics matter to the timing.
"""
from __future__ import annotations

import argparse
import datetime
import math
import os
import statistics
import sys

import torch

import routed_grouped_gemm_amd as moe

_PKG = os.path.dirname(os.path.abspath(__file__))
DEFAULT_OUT = os.path.join(_PKG, "csrc", "moe_tuned.h")

# table row -> (layer shape, token counts swept, candidate m-tile rows); "fp8a": fp8 weights
# with fp8 activations (moe_problem.act_quant)
SWEEPS = {
    "bf16": (dict(d=2048, n=512, E=256, k=8), [16, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384],
             [16, 32, 64, 128, 160]),
    "fp8": (dict(d=7168, n=2048, E=256, k=8), [1, 8, 32, 64, 128, 256, 512, 1024, 2048, 4096],
            [16, 32, 64, 128, 160]),
    "fp8a": (dict(d=7168, n=2048, E=256, k=8), [1, 8, 32, 64, 128, 256, 512, 1024, 2048, 4096],
             [16, 32, 64, 128, 160]),
}
GROUPS = [1, 4]
ROWS = ("f32", "bf16", "fp8", "fp8a")   # rule lists of moe_tuned.h, in order
WDTYPE = {"bf16": "bf16", "fp8": "fp8", "fp8a": "fp8"}


def _weights(d, n, E, w, dev):
    """Random row-major expert weights of a layer, on the device (fp8: block-quantised)."""
    def mat(rows, cols, fan_in):
        x = torch.randn(E, rows, cols, device=dev) / math.sqrt(fan_in)
        if w == "bf16":
            return x.to(torch.bfloat16), None
        b = x.view(E, rows // 128, 128, cols // 128, 128)
        s = b.abs().amax(dim=(2, 4)).clamp_min(1e-30) / 448.0
        q = (b / s[:, :, None, :, None]).clamp(-448, 448).view(E, rows, cols).to(torch.float8_e4m3fn)
        return q, s.float().contiguous()
    (g, sg), (u, su), (dn, sd) = mat(n, d, d), mat(n, d, d), mat(d, n, n)
    out = dict(w_gate=g, w_up=u, w_down=dn)
    if w == "fp8":
        out.update(s_gate=sg, s_up=su, s_down=sd)
    return out


def _time(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return statistics.median(s.elapsed_time(e) * 1e3 for s, e in ev)


def choose(cand, floor, prev, dkey, margin=0.02):
    """The winner at one M: the fastest candidate (rows, group) whose m-tile is at least `floor`
    (the previous M's winner), except that the previous M's winner, or else the current table's
    choice `dkey`, is kept unless the fastest is more than `margin` faster (so timing noise
    does not split buckets)."""
    allowed = {c: t for c, t in cand.items() if c[0] >= floor}
    best = min(allowed, key=allowed.get)
    for keep in (prev, dkey):
        if keep in allowed and allowed[best] > (1.0 - margin) * allowed[keep]:
            return keep
    return best


def sweep(row, quick=False, log=print):
    shape, Ts, rows_list = SWEEPS[row]
    w, aq = WDTYPE[row], row == "fp8a"
    d, n, E, k = shape["d"], shape["n"], shape["E"], shape["k"]
    dev = "cuda"
    torch.manual_seed(1234)
    p0 = moe.problem(1, d, n, E, k, 0, "bf16", w, layout="rowmajor")
    W = moe.pack_weights(p0, _weights(d, n, E, w, dev))
    wr = (torch.randn(E, d, device=dev) / math.sqrt(d)).to(torch.bfloat16)
    Tmax = max(Ts)
    xall = torch.randn(Tmax, d, device=dev).to(torch.bfloat16)
    results = []
    floor, prev = 0, None  # a larger M never takes a smaller m-tile than a smaller M took
    for T in (Ts[::3] if quick else Ts):
        p = moe.problem(T, d, n, E, k, 0, "bf16", w, layout="packed", act_quant=aq)
        # one workspace for every candidate tile: the w8a16 layout (bf16 H, the larger one) plus,
        # for the fp8-activation tiles, their quantised hidden rows and block scales, plus room
        # for the m-tile descriptors of the smallest tile
        pw = moe.problem(T, d, n, E, k, 0, "bf16", w, layout="packed")
        ws = moe.alloc_workspace(pw, extra=(8 << 20) + (T * d * 2 + T * k * n // 32 if aq else 0))
        x = xall[:T].contiguous()
        out = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
        cand = {}
        for rows in rows_list:
            for gm in (GROUPS if rows > 16 else [GROUPS[-1]]):
                steps = 10 if T * k / E < 64 else 6
                us = _time(lambda: moe.forward(p, x, wr, None, W, ws, out=out, m_tile_rows=rows, group_m=gm), steps, 3)
                assert moe.last_device_error(ws) == 0
                cand[(rows, gm)] = us
        default = moe.plan_describe(p)
        dkey = (default["m_tile_rows"], default["group_m"])
        best = choose(cand, floor, prev, dkey)
        floor, prev = best[0], best
        mean = T * k / E
        results.append(dict(T=T, mean_rows=mean, best=best, us=cand, default=dkey))
        log(f"[tune] {row} T={T} mean={mean:g}: best {best} {cand[best]:.1f} us (table {dkey} "
            f"{cand.get(dkey, float('nan')):.1f} us)")
        del ws
    del W
    torch.cuda.empty_cache()
    return results


def rules_from(results, max_rows):
    """Bucket rules: consecutive M with the same winner merge; boundaries at geometric means."""
    rules = []
    for i, r in enumerate(results):
        if rules and rules[-1][1] == r["best"]:
            rules[-1][0] = i
            continue
        rules.append([i, r["best"]])
    out = []
    for j, (last, best) in enumerate(rules):
        if j + 1 < len(rules):
            nxt = results[last + 1]["mean_rows"]
            bound = math.sqrt(results[last]["mean_rows"] * nxt)
        else:
            bound = 1e30
        out.append((bound, min(best[0], max_rows), best[1]))
    return out


def write_header(path, table, sources):
    lines = [
        "// moe_tuned.h -- the M-bucket tile table of the MoE-layer forward (included by moe_plan.h).",
        "//",
        "// One rule list per weight dtype (f32, bf16, fp8, and fp8 weights with fp8 activations): the",
        "// first rule whose max_mean_rows is at least the problem's mean rows per routed expert (T*k/E)",
        "// gives the m-tile size and the group size of the late phase's grouped item order.  Written by",
        "// the tuner (python -m routed_grouped_gemm_amd.tune) from timings on the device:",
    ] + [f"//   {s}" for s in sources] + [
        "#pragma once",
        "",
        "namespace moe {",
        "namespace {",
        "",
        "struct TileRule {",
        "  float max_mean_rows;  // upper bound (inclusive) of the bucket's mean rows per routed expert",
        "  int m_tile_rows;      // 16, 32, 64, 128 or 160",
        "  int group_m;          // late phase: m-tiles per group (m-tiles above 16 rows)",
        "};",
        "",
    ]
    n = max(len(v) for v in table.values())
    lines.append(f"constexpr int kNumTileRules = {n};")
    lines.append(f"constexpr TileRule kTileRules[{len(ROWS)}][kNumTileRules] = {{")
    for name in ROWS:
        rules = list(table[name])
        while len(rules) < n:
            rules.append(rules[-1])
        body = ", ".join(f"{{{b:.6f}f, {r}, {g}}}" if b < 1e29 else f"{{1e30f, {r}, {g}}}" for b, r, g in rules)
        lines.append(f"    // {name}")
        lines.append(f"    {{{body}}},")
    lines.append("};")
    lines.append(f'constexpr const char *kTileTableSource = "tuned on the device";')
    lines += ["", "}  // namespace", "}  // namespace moe", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=DEFAULT_OUT)
    ap.add_argument("--report", default=None)
    ap.add_argument("--quick", action="store_true")
    a = ap.parse_args()
    assert torch.cuda.is_available(), "the tuner runs on the GPU"
    report = [f"# Tile-table tuning ({datetime.date.today()}, {torch.cuda.get_device_name(0)})", "",
              "Command: `python -m routed_grouped_gemm_amd.tune " + " ".join(sys.argv[1:]) + "`", ""]
    table, sources = {}, []
    for w in ("bf16", "fp8", "fp8a"):
        res = sweep(w, quick=a.quick)
        shape = SWEEPS[w][0]
        table[w] = rules_from(res, max(SWEEPS[w][2]))
        label = "fp8 weights, fp8 activations" if w == "fp8a" else f"{w} weights"
        sources.append(f"{w}: d={shape['d']} n={shape['n']} E={shape['E']} k={shape['k']}, "
                       f"M in {[r['T'] for r in res]}")
        report += [f"## {label}, d={shape['d']} n={shape['n']} E={shape['E']} k={shape['k']}", "",
                   "| T | mean rows | chosen (rows, group) | " + " | ".join(f"{c}" for c in res[0]["us"]) + " |",
                   "|---|---|---|" + "---|" * len(res[0]["us"])]
        for r in res:
            report.append(f"| {r['T']} | {r['mean_rows']:g} | {r['best']} | " +
                          " | ".join(f"{r['us'].get(c, float('nan')):.1f}" for c in res[0]["us"]) + " |")
        report += ["", "Rules: " + ", ".join(f"mean <= {b:g}: {rr} rows, group {g}" for b, rr, g in table[w]), ""]
    # fp32 weights (the small test workload's dtype) follow the bf16 buckets
    table["f32"] = table["bf16"]
    write_header(a.out, table, sources)
    if a.report:
        with open(a.report, "w") as f:
            f.write("\n".join(report) + "\n")
    print("\n".join(report))


if __name__ == "__main__":
    main()
