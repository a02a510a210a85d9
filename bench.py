"""Benchmark of the MoE-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--T T]

A step is one moe_forward call (the whole layer: route, permute, grouped SwiGLU
GEMM, combine) over one batch of seeded synthetic input already resident in HBM.
The default workload is the decode-shaped bf16 layer (T=16, d=2048, E=256, top-8,
n=512).  Weights are rotated over several identical copies so that consecutive
steps stream weights the 256 MB Infinity Cache does not hold, like consecutive
layers of a model.  The expert weights are converted to the library's packed
fragment layout once, with moe_pack_weights, before anything is timed (a
load-time step, like the fp8 quantisation of the weights).

Prints one JSON line: tokens/s, the roofline of the dominant (and only) kernel
measured with HIP events on its launch stream, and the CPU oracle timed on a
bounded sample on this host (cpu_baseline).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_bf16")
    ap.add_argument("--T", type=int, default=None, help="token count (large_fp8 sweep)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=0, help="weight copies to rotate (0 = auto)")
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--schedule", type=int, default=0)
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


KERNEL_SOURCES = ("routed_grouped_gemm_amd/csrc/moe_kernels.hip", "routed_grouped_gemm_amd/csrc/moe_plan.h")


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this workload
    (FETCH_SIZE and WRITE_SIZE scaled by a plain-copy calibration), or None when there is
    none or the kernel sources changed since the counters were taken."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    sha = h.hexdigest()[:16]
    path = os.path.join(ROOT, "profiles", f"moe_persistent_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "kernel_source_sha"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    if fields.get("kernel_source_sha") != sha or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_baseline(inp, budget_s=12.0):
    """The oracle as it stands, on this host: whole forwards of the same workload
    (or its first tokens, for the large configs) repeated within a time budget."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = int(os.environ.get("OMP_NUM_THREADS", "1"))
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
    return {"value": round(tokens / dt, 3), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2)}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark measures the layer on one GPU; more than one GPU is not "
                                   "supported (use --gpus 1)"}))
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration(a.steps)
        return
    import numpy as np
    import torch

    import routed_grouped_gemm_amd as moe
    import synth
    from devinputs import to_device

    if not os.path.exists(moe.LIB_PATH):
        from routed_grouped_gemm_amd import build as b
        b.build()
    cfg = synth.config(a.config, a.T)
    inp = synth.make_inputs(cfg)
    p, x, wr, bias, W = to_device(inp)
    ws = moe.alloc_workspace(p)

    # routing of this batch (for the algorithmic byte count) from the library itself
    out, r = moe.forward(p, x, wr, bias, W, ws, route_out=True)
    torch.cuda.synchronize()
    assert moe.last_device_error(ws) == 0
    counts = r["counts"].cpu().numpy()
    B, F, touched = algorithmic(cfg, counts, cfg["shared"])

    wbytes = sum(t.numel() * t.element_size() for t in W.values())
    copies = a.copies or int(min(16, max(2, -(-4 * MALL_BYTES // max(1, min(wbytes, B))))))
    if cfg["w"] == "fp8" and wbytes > (8 << 30):
        copies = max(2, min(copies, 2))
    Ws = [moe.make_weights(W)]
    keep = [W]
    for _ in range(copies - 1):
        Wc = {k2: t.clone() for k2, t in W.items()}
        keep.append(Wc)
        Ws.append(moe.make_weights(Wc))
    out = torch.empty((cfg["T"], cfg["d"]), dtype=x.dtype, device="cuda")

    def step(i):
        moe.forward(p, x, wr, bias, Ws[i % copies], ws, out=out, grid_wgs=a.grid, schedule=a.schedule)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    K = a.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert moe.last_device_error(ws) == 0, "device fault flag set during the timed steps"
    per = np.array([s.elapsed_time(e) * 1e3 for s, e in ev])  # us per launch
    avg_us = float(per.mean())
    T = cfg["T"]
    value = T * K / wall
    gbs = B / (avg_us * 1e-6) / 1e9
    tfl = F / (avg_us * 1e-6) / 1e12
    peak_mfma = MFMA_PEAK_TFLOPS["bf16" if cfg["w"] == "fp8" else cfg["w"]]
    t_hbm = B / (HBM_PEAK_GBS * 1e9)
    t_mfma = F / (peak_mfma * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tfl, 2), "peak": peak_mfma, "unit": "TFLOP/s",
                "frac": round(tfl / peak_mfma, 4)}
    traffic = measured_traffic(cfg["name"])
    roof["traffic"] = traffic
    roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1)"
    if traffic:
        roof["traffic_over_algorithmic"] = round(traffic / B, 3)
    roof["bytes_per_launch"] = int(B)
    roof["flops_per_launch"] = int(F)
    roof["kernel"] = "moe_persistent"
    roof["avg_launch_us"] = round(avg_us, 2)
    roof["roofline_time_frac"] = round(max(t_hbm, t_mfma) / (avg_us * 1e-6), 4)
    res = {
        "metric": "MoE-layer tokens/sec + % roofline (HBM GB/s decode, MFMA TFLOP/s prefill)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": a.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if cfg["act"] == "f32" else "bf16", "data": "synthetic",
        "config": {"workload": cfg["name"], "T": T, "d": cfg["d"], "E": cfg["E"], "k": cfg["k"], "n": cfg["n"],
                   "shared_experts": cfg["shared"], "act": cfg["act"], "weights": cfg["w"],
                   "weight_layout": "packed (moe_pack_weights at load time)",
                   "experts_touched": touched, "weight_copies_rotated": copies, "parallelism": "none (1 GPU)"},
        "latency_us": {"p50": round(float(np.percentile(per, 50)), 2),
                       "p99": round(float(np.percentile(per, 99)), 2)},
        "tflops": round(tfl, 3),
        "roofline": roof,
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
