"""Write tests/golden/skewed_router_bias.json: the frozen router bias of the
skewed-load workload (T=2048, d=4096, E=64, top-4, n=1536).

Expert popularity on real MoE traffic is close to a Zipf law, with hot and cold
experts (Weave review, section 1.1).  This script fits one float32 bias per
expert so that the oracle's routing of the seeded tokens gives expert counts
close to Zipf(s=1.1) over popularity ranks; a seeded permutation maps ranks to
expert ids.  It calls only the synthetic-input module and the CPU oracle.

Fit: start from b_e = ln p_e and take 60 fixed damped steps
    b_e += 0.3 * ln((target_e + 1/2) / (count_e + 1/2)),
where count_e is the oracle's routing count.  A token picks an expert at most
once, so no target may exceed T: targets above T are clamped to T and the rest
is renormalised (water filling).

Run:  python tests/golden/make_zipf_bias.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(HERE, "skewed_router_bias.json")
ITERS = 60
STEP = 0.3


def zipf_targets(E, total, cap, s):
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    t = p * total
    fixed = np.zeros(E, bool)
    while np.any(t[~fixed] > cap):
        over = (~fixed) & (t > cap)
        fixed |= over
        t[fixed] = cap
        rest = total - t[fixed].sum()
        t[~fixed] = p[~fixed] / p[~fixed].sum() * rest
    return p, t


def fit_exponent(counts_by_rank):
    c = np.asarray(counts_by_rank, np.float64)
    r = np.arange(1, len(c) + 1, dtype=np.float64)
    ok = c > 0
    A = np.stack([np.log(r[ok]), np.ones(ok.sum())], 1)
    slope, _ = np.linalg.lstsq(A, np.log(c[ok]), rcond=None)[0]
    return float(-slope)


def main():
    cfg = synth.config("skewed_bf16")
    T, E, k = cfg["T"], cfg["E"], cfg["k"]
    x = oracle.widen(synth.make_hidden(cfg), cfg["act"])
    wr = oracle.widen(synth.make_router(cfg), cfg["act"])
    L0 = oracle.router_logits(x, wr)
    rank_to_expert = synth.zipf_rank_permutation(cfg)
    p_rank, t_rank = zipf_targets(E, T * k, T, cfg["zipf_s"])
    target = np.zeros(E)
    p = np.zeros(E)
    target[rank_to_expert] = t_rank
    p[rank_to_expert] = p_rank
    b = np.log(p)
    for it in range(ITERS):
        ids = oracle.select_topk(L0 + b[None, :], k)
        cnt = np.bincount(ids.reshape(-1), minlength=E)
        b = b + STEP * np.log((target + 0.5) / (cnt + 0.5))
    b32 = b.astype(np.float32)
    ids = oracle.select_topk(oracle.router_logits(x, wr, b32.astype(np.float64)), k)
    cnt = np.bincount(ids.reshape(-1), minlength=E)
    by_rank = cnt[rank_to_expert]
    rec = dict(config=cfg["name"], zipf_s=cfg["zipf_s"], iterations=ITERS, step=STEP,
               bias_f32_hex=[float(v).hex() for v in b32],
               achieved_counts_by_rank=[int(v) for v in by_rank],
               target_counts_by_rank=[round(float(v), 3) for v in t_rank],
               fitted_exponent=round(fit_exponent(by_rank), 4),
               max_over_mean=round(float(cnt.max() / cnt.mean()), 3),
               generated_by="tests/golden/make_zipf_bias.py")
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1)
    print("wrote", OUT, "fitted exponent", rec["fitted_exponent"], "max/mean", rec["max_over_mean"],
          "hottest", by_rank[:4].tolist(), "coldest", by_rank[-4:].tolist())


if __name__ == "__main__":
    main()
