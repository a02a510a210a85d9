"""Benchmark of the MoE-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--T T]
                    [--configs LIST | --configs none] [--no-cpu-baseline] [--fp8act]
    python bench.py --item-trace [--config NAME] [--T T] [--fp8act]

A step is one moe_forward call (the whole layer: route, permute, grouped SwiGLU
GEMM, combine) over one batch of seeded synthetic input already resident in HBM.
The headline workload is the decode-shaped bf16 layer (T=16, d=2048, E=256, top-8,
n=512).  Weights are rotated over several identical copies so that consecutive
steps stream weights the 256 MB Infinity Cache does not hold, like consecutive
layers of a model.  The expert weights are converted to the library's packed
fragment layout once, with moe_pack_weights, before anything is timed (a
load-time step, like the fp8 quantisation of the weights).

Prints one JSON line: tokens/s of the headline workload, the roofline of the
dominant (and only) kernel measured with HIP events on its launch stream, the
CPU oracle timed on a bounded sample on this host (cpu_baseline), and a
`configs` list with the same measurements for the other workloads: prefill (HBM
and MFMA fractions), the skewed-load layer under the dynamic queue and under the
static schedule, the large fp8 layer at T = 1, 8, 512 and 4096 (at 4096 also with fp8
activations), and the compute-bound points: prefill at T = 16384 and 32768, the
large fp8 layer at T = 16384 (both activation modes).  `--configs` takes a
comma-separated list of NAME[@T][:static][:fp8act] entries instead (:fp8act: the
fp8-activation mode of the expert GEMMs, fp8-weight workloads only).
"""
import os

# the oracle's BLAS uses the cores this process may run on; set before numpy loads
_CORES = len(os.sched_getaffinity(0))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = str(_CORES)

import argparse  # noqa: E402
import json  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
MALL_BYTES = 256 << 20
DEFAULT_CONFIGS = ("prefill_bf16,skewed_bf16,skewed_bf16:static,large_fp8@1,large_fp8@8,large_fp8@512,large_fp8@4096,"
                   "large_fp8@4096:fp8act,prefill_bf16@16384,prefill_bf16@32768,large_fp8@16384,large_fp8@16384:fp8act")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_bf16")
    ap.add_argument("--T", type=int, default=None, help="token count of the headline workload")
    ap.add_argument("--configs", default=DEFAULT_CONFIGS,
                    help="other workloads for the configs list: NAME[@T][:static][:fp8act],... or 'none'")
    ap.add_argument("--config-steps", type=int, default=30, help="timed steps per entry of the configs list")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--schedule", type=int, default=0)
    ap.add_argument("--item-trace", action="store_true",
                    help="instead: print the per-item trace summary of one forward of the headline workload")
    ap.add_argument("--fp8act", action="store_true",
                    help="headline workload in the fp8-activation mode (fp8-weight workloads only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead: time a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def copy_calibration(steps):
    """A plain device-to-device copy of a known size, to scale the HBM byte counters."""
    import torch
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1e3 / steps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "avg_us": round(us, 2),
                      "GBps_read_plus_write": round(2 * nbytes / us / 1e3, 1)}), flush=True)


def algorithmic(cfg, counts, n_shared):
    """Algorithmic bytes and flops of one forward (nothing counted twice, no H/Y round
    trips): touched expert weights (+ fp8 scales), shared expert, router weights, the
    token rows read once and the output written once."""
    T, d, n, E, k = cfg["T"], cfg["d"], cfg["n"], cfg["E"], cfg["k"]
    wsz = {"f32": 4, "bf16": 2, "fp8": 1}[cfg["w"]]
    asz = {"f32": 4, "bf16": 2}[cfg["act"]]
    touched = int((counts > 0).sum())
    per_expert = 3 * d * n * wsz
    if cfg["w"] == "fp8":
        per_expert += 3 * (d // 128) * (n // 128) * 4
    b = (touched + n_shared) * per_expert + E * d * asz + 2 * T * d * asz
    f = 2 * T * d * E + 2 * (T * k + n_shared * T) * 3 * d * n
    return b, f, touched


KERNEL_SOURCES = ("routed_grouped_gemm_amd/csrc/moe_kernels.hip", "routed_grouped_gemm_amd/csrc/moe_plan.h",
                  "routed_grouped_gemm_amd/csrc/moe_tuned.h", "routed_grouped_gemm_amd/build.py")


def kernel_sha():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_name(workload, T):
    return f"moe_persistent_{workload}" + ("" if T is None else f"_T{T}")


def synth_default_T(name):
    import synth
    return synth.config(name)["T"]


def measured_traffic(workload, T=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this workload
    (DRAM read and write requests of the L2s, in 32-byte units), or None when there is none
    or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", profile_name(workload, T) + ".md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "kernel_source_sha"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if fields.get("kernel_source_sha") != kernel_sha() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def blas_vendor():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        return ",".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info})) or "unknown"
    except Exception:
        return "unknown"


def cpu_baseline(inp, budget_s=12.0):
    """The oracle as it stands, on this host: whole forwards of the same workload
    (or its first tokens, for the large configs) repeated within a time budget."""
    import numpy as np
    import oracle
    v = oracle.InputsView(inp)
    T = v.x.shape[0]
    reps, tokens, t0 = 0, 0, time.perf_counter()
    if T <= 64:
        while True:
            oracle.moe_forward_view(v)
            reps += 1
            tokens += T
            if time.perf_counter() - t0 > budget_s or reps >= 20:
                break
        sample = f"whole forward of all {T} tokens, repeated {reps} times"
    else:
        toks = np.arange(min(T, 8))
        oracle.moe_forward_tokens(v, toks)
        tokens = len(toks)
        sample = f"first {len(toks)} of {T} tokens, one by one (every routed and shared expert they touch)"
    dt = time.perf_counter() - t0
    return {"value": round(tokens / dt, 3), "unit": "tokens/s", "cores": _CORES, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2), "blas": blas_vendor(),
            "threads_env": {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}}


class Workloads:
    """Synthetic inputs, drawn once per weight set (workloads sharing a seed and shapes share
    weights; the large fp8 sweep shares one weight set over T), kept on the device."""

    def __init__(self):
        self.host = {}
        self.dev = {}

    def inputs(self, name, T):
        import synth
        cfg = synth.config(name, T)
        key = (cfg["seed"], cfg["d"], cfg["n"], cfg["E"], cfg["w"], cfg["shared"])
        if key not in self.host:
            for k2 in list(self.host):  # one weight set at a time (the fp8 one is 11 GB)
                del self.host[k2]
                self.dev.pop(k2, None)
            full = synth.config(name, synth.config(name)["T_gen"])
            self.host[key] = synth.make_inputs(full)
        base = self.host[key]
        inp = synth.MoEInputs(**{f: getattr(base, f) for f in base.__dataclass_fields__})
        inp.cfg = cfg
        inp.hidden = base.hidden[:cfg["T"]]
        inp.bias = synth.load_zipf_bias(cfg) if cfg.get("zipf") else None
        return key, cfg, inp

    def device_weights(self, key, inp):
        from devinputs import to_device
        if key not in self.dev:
            self.dev[key] = to_device(inp)[4]
        return self.dev[key]


def measure(wl, name, T, steps, warmup, copies=0, grid=0, schedule=0, want_inputs=False, act_quant=False):
    """Times `steps` launches of one workload; returns a dict of its measurements."""
    import numpy as np
    import torch

    import routed_grouped_gemm_amd as moe
    from devinputs import tensor

    key, cfg, inp = wl.inputs(name, T)
    W = wl.device_weights(key, inp)
    p = moe.problem(cfg["T"], cfg["d"], cfg["n"], cfg["E"], cfg["k"], cfg["shared"], cfg["act"], cfg["w"],
                    layout="packed", act_quant=act_quant)
    plan = moe.plan_describe(p)
    x, wr, bias = tensor(inp.hidden), tensor(inp.w_router), tensor(inp.bias)
    ws = moe.alloc_workspace(p)
    # routing of this batch (for the algorithmic byte count) from the library itself
    out, r = moe.forward(p, x, wr, bias, W, ws, route_out=True)
    torch.cuda.synchronize()
    assert moe.last_device_error(ws) == 0
    counts = r["counts"].cpu().numpy()
    B, F, touched = algorithmic(cfg, counts, cfg["shared"])
    wbytes = sum(t.numel() * t.element_size() for t in W.values())
    if not copies:
        copies = int(min(16, max(2, -(-4 * MALL_BYTES // max(1, min(wbytes, B))))))
        if wbytes > (8 << 30):
            copies = 2
    Ws = [moe.make_weights(W)]
    keep = [W]
    for _ in range(copies - 1):
        Wc = {k2: t.clone() for k2, t in W.items()}
        keep.append(Wc)
        Ws.append(moe.make_weights(Wc))

    def step(i):
        moe.forward(p, x, wr, bias, Ws[i % copies], ws, out=out, grid_wgs=grid, schedule=schedule)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert moe.last_device_error(ws) == 0, "device fault flag set during the timed steps"
    per = np.array([s.elapsed_time(e) * 1e3 for s, e in ev])  # us per launch
    avg_us = float(per.mean())
    # fp8 weights are decoded to bf16 for the MFMA, unless the GEMMs read fp8 activations
    mfma = ("fp8" if plan["fp8_activations"] else "bf16") if cfg["w"] == "fp8" else cfg["w"]
    peak_mfma = MFMA_PEAK_TFLOPS[mfma]
    gbs = B / (avg_us * 1e-6) / 1e9
    tfl = F / (avg_us * 1e-6) / 1e12
    t_hbm, t_mfma = B / (HBM_PEAK_GBS * 1e9), F / (peak_mfma * 1e12)
    wl_name = name + ("_fp8act" if plan["fp8_activations"] else "")
    # profiles exist per T for the large fp8 layer, else for the workload's own T only
    if name == "large_fp8":
        traffic = measured_traffic(wl_name, cfg["T"])
    elif T is None or T == synth_default_T(name):
        traffic = measured_traffic(wl_name)
    else:
        traffic = None
    res = dict(workload=name, T=cfg["T"], schedule="static" if schedule == 1 else "dynamic",
               fp8_activations=bool(plan["fp8_activations"]),
               m_tile_rows=plan["m_tile_rows"], experts_touched=touched,
               p50_us=round(float(np.percentile(per, 50)), 2), p99_us=round(float(np.percentile(per, 99)), 2),
               avg_launch_us=round(avg_us, 2), steps=steps, wall_s=wall,
               tokens_per_s=round(cfg["T"] / (avg_us * 1e-6), 1),
               GB_s=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
               TFLOP_s=round(tfl, 2), mfma_dtype=mfma, mfma_frac=round(tfl / peak_mfma, 4),
               roofline_bound="hbm" if t_hbm >= t_mfma else "mfma",
               roofline_time_frac=round(max(t_hbm, t_mfma) / (avg_us * 1e-6), 4),
               bytes_per_launch=int(B), flops_per_launch=int(F), traffic=traffic,
               traffic_over_algorithmic=round(traffic / B, 3) if traffic else None,
               weight_copies_rotated=copies)
    del keep, Ws, ws, out, r
    torch.cuda.empty_cache()
    if want_inputs:
        return res, cfg, inp
    return res


ITEM_KINDS = {0: "clear", 1: "router", 2: "topk", 3: "shared_gateup", 4: "scatter", 5: "gateup", 6: "down",
              7: "combine", 8: "act_quant"}


def item_trace(wl, name, T, act_quant=False):
    """Per-item trace of one forward (moe_launch_options.trace): the span of the launch, the
    busy share of the workgroups (item time over workgroups x span; the rest is waiting for a
    dependency or for the queue), the gaps between consecutive items of a workgroup, and per
    item kind the count, durations, tile-loop time and the first start / last end (us from
    the launch's first item)."""
    import numpy as np
    import torch

    import routed_grouped_gemm_amd as moe
    from devinputs import tensor

    key, cfg, inp = wl.inputs(name, T)
    W = wl.device_weights(key, inp)
    p = moe.problem(cfg["T"], cfg["d"], cfg["n"], cfg["E"], cfg["k"], cfg["shared"], cfg["act"], cfg["w"],
                    layout="packed", act_quant=act_quant)
    x, wr, bias = tensor(inp.hidden), tensor(inp.w_router), tensor(inp.bias)
    ws = moe.alloc_workspace(p)
    tr = torch.zeros(4 * 400000, dtype=torch.int64, device="cuda")
    for _ in range(5):
        moe.forward(p, x, wr, bias, W, ws)
    torch.cuda.synchronize()
    moe.forward(p, x, wr, bias, W, ws, trace=tr)
    torch.cuda.synchronize()
    assert moe.last_device_error(ws) == 0
    rec = tr.view(-1, 4).cpu().numpy().astype(np.uint64)
    rec = rec[rec[:, 1] > 0]
    t0 = rec[:, 0].min()
    start = (rec[:, 0] - t0).astype(np.float64) / 100.0  # the device clock runs at 100 MHz
    end = (rec[:, 1] - t0).astype(np.float64) / 100.0
    kind = (rec[:, 3] & 0xffffffff).astype(int)
    wg = (rec[:, 3] >> 32).astype(int)
    l0 = ((rec[:, 2] >> 32) & 0xffff).astype(np.float64) / 100.0
    l1 = ((rec[:, 2] >> 48) & 0xffff).astype(np.float64) / 100.0
    span = float(end.max())
    ngrid = int(wg.max()) + 1
    gaps = []
    for w in range(ngrid):
        m = np.nonzero(wg == w)[0]
        o = m[np.argsort(start[m])]
        gaps += list(start[o][1:] - end[o][:-1])
    out = dict(workload=name, T=cfg["T"], fp8_activations=bool(moe.plan_describe(p)["fp8_activations"]),
               span_us=round(span, 1), workgroups=ngrid, items=int(len(rec)),
               busy_share=round(float((end - start).sum() / (ngrid * span)), 3),
               gap_between_items_us={"mean": round(float(np.mean(gaps)), 2) if gaps else 0.0,
                                     "p90": round(float(np.percentile(gaps, 90)), 2) if gaps else 0.0},
               kinds={})
    for k in sorted(set(kind.tolist())):
        m = kind == k
        d = end[m] - start[m]
        loop = np.where(l1[m] > 0, l1[m] - l0[m], 0.0)
        out["kinds"][ITEM_KINDS.get(k, str(k))] = dict(
            n=int(m.sum()), dur_mean_us=round(float(d.mean()), 2), dur_max_us=round(float(d.max()), 2),
            tile_loop_mean_us=round(float(loop.mean()), 2), first_start_us=round(float(start[m].min()), 1),
            last_end_us=round(float(end[m].max()), 1))
    return out


def parse_entry(e):
    """NAME[@T][:static][:fp8act] -> (name, T, static, fp8act)"""
    head, *flags = e.split(":")
    bad = [f for f in flags if f not in ("static", "fp8act")]
    if bad:
        raise SystemExit(f"unknown config flag(s) {bad} in {e!r}")
    name, _, t = head.partition("@")
    return name, (int(t) if t else None), "static" in flags, "fp8act" in flags


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark measures the layer on one GPU; more than one GPU is not "
                                   "supported (use --gpus 1)"}))
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration(a.steps)
        return
    import routed_grouped_gemm_amd as moe

    if not os.path.exists(moe.LIB_PATH):
        raise SystemExit(f"{moe.LIB_PATH} is not built: run `python -m routed_grouped_gemm_amd.build` first")
    wl = Workloads()
    if a.item_trace:
        print(json.dumps(item_trace(wl, a.config, a.T, a.fp8act)), flush=True)
        return
    head, cfg, inp = measure(wl, a.config, a.T, a.steps, a.warmup, copies=a.copies, grid=a.grid,
                             schedule=a.schedule, want_inputs=True, act_quant=a.fp8act)
    roof = {"bound": head["roofline_bound"]}
    if head["roofline_bound"] == "hbm":
        roof.update(achieved=head["GB_s"], peak=HBM_PEAK_GBS, unit="GB/s", frac=head["hbm_frac"])
    else:
        roof.update(achieved=head["TFLOP_s"], peak=MFMA_PEAK_TFLOPS[head["mfma_dtype"]], unit="TFLOP/s",
                    frac=head["mfma_frac"])
    roof.update(traffic=head["traffic"],
                traffic_unit="HBM bytes per launch (rocprofv3 TCC_EA0_RDREQ_DRAM_32B_sum + "
                             "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum, x32 bytes; copy-calibrated factor 1.0)",
                traffic_over_algorithmic=head["traffic_over_algorithmic"],
                bytes_per_launch=head["bytes_per_launch"], flops_per_launch=head["flops_per_launch"],
                kernel="moe_persistent", avg_launch_us=head["avg_launch_us"],
                roofline_time_frac=head["roofline_time_frac"], mfma_frac=head["mfma_frac"])
    res = {
        "metric": "MoE-layer tokens/sec + % roofline (HBM GB/s decode, MFMA TFLOP/s prefill)",
        "value": round(cfg["T"] * a.steps / head["wall_s"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(head["wall_s"] * 1e3 / a.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if cfg["act"] == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "T": cfg["T"], "d": cfg["d"], "E": cfg["E"], "k": cfg["k"],
                   "fp8_activations": head["fp8_activations"],
                   "n": cfg["n"], "shared_experts": cfg["shared"], "act": cfg["act"], "weights": cfg["w"],
                   "weight_layout": "packed (moe_pack_weights at load time)",
                   "experts_touched": head["experts_touched"], "m_tile_rows": head["m_tile_rows"],
                   "weight_copies_rotated": head["weight_copies_rotated"], "parallelism": "none (1 GPU)"},
        "latency_us": {"p50": head["p50_us"], "p99": head["p99_us"]},
        "tflops": head["TFLOP_s"],
        "roofline": roof,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp)
    if a.configs and a.configs != "none":
        entries = []
        for e in a.configs.split(","):
            name, T, static, fp8act = parse_entry(e.strip())
            r = measure(wl, name, T, a.config_steps, 3, schedule=1 if static else 0, act_quant=fp8act)
            r.pop("wall_s")
            entries.append(r)
            print(f"[bench] {name} T={r['T']} {r['schedule']}{' fp8act' if r['fp8_activations'] else ''}: "
                  f"{r['avg_launch_us']} us, hbm {r['hbm_frac']}, mfma {r['mfma_frac']} ({r['mfma_dtype']})",
                  file=sys.stderr, flush=True)
        res["configs"] = entries
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
